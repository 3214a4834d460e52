/*
 * deltakv.h - C ABI of the DeltaKV hot path on AMD Instinct MI355X (gfx950).
 *
 * DeltaKV ("DeltaKV: Residual-Based KV Cache Compression via Long-Range
 * Similarity", arXiv 2602.08005; explainer pages on gist.science) stores a
 * KV cache as a few full reference tokens taken at a fixed stride plus, for
 * every other token, a short code of its residual against the most similar
 * earlier reference, after a component shared by all tokens is removed.
 * Two calls make up the hot path:
 *
 *   deltakv_compress     prefill K/V -> compressed cache
 *   deltakv_decode_attn  decode queries x compressed cache -> attention output
 *
 * Method statement implemented here (per stream = one sequence b, one KV
 * head h, one of K or V; rnd = round to the storage dtype, nearest even):
 *
 *   mu      = rnd(mean_t k_t)                          shared component
 *   x~_t    = rnd(k_t - mu)
 *   refs[r] = x~_{r*s}            r = 0 .. R-1, R = ceil(T / s)
 *   ref(t)  = argmax over r with r*s < t of cos(x~_t, refs[r]),
 *             lowest r on exact ties, cos = 0 for a zero vector
 *             (top_k > 1 or metric = L2: the k best by that metric, and
 *             refs[ref(t)] below stands for their mean)
 *   code_t  = rnd(W_down ((k_t - mu) - refs[ref(t)]))   d_c values
 *   decode: k^_t = mu + refs[ref(t)] + W_up code_t (refs are tokens too:
 *           k^_{r*s} = mu + refs[r]); out_g = softmax_t(q_g . k^_t * scale) V^
 *
 * Sources (English page unless noted): Technical Summary §2 "Highly Shared
 * Latent Components" (shared high-norm component removed first); §3
 * "Strided Reference Selection" (references at stride s, retrieval of the
 * nearest earlier references for each token); §3 "Residual Encoding"
 * (z = f_c(KV) - f_c(KV^R)); §3 "Reconstruction" (KV^ = f_d(z) + KV^R);
 * French page, Méthodologie §2 "Architecture de compression" (linear
 * projection to a d_c-dimensional code).  Top-1 cosine, the mean as the
 * shared component and a linear code are this library's concrete reading of
 * the pages' retrieval, shared-component and compressor descriptions.
 *
 * Conventions for every entry point:
 *  - Pointers named as device pointers must be device memory on the current
 *    HIP device; every other pointer is host memory and is only read during
 *    the call.  The caller owns all memory, including workspaces.  The
 *    library never allocates, frees or synchronises.
 *  - Work is enqueued on `stream` (a hipStream_t, passed as void* so that
 *    this header needs no HIP header; NULL = the null stream) and runs
 *    asynchronously; outputs are valid once the stream reaches it.
 *  - Argument checks run on the host before anything is enqueued; on any
 *    error nothing is launched and outputs are untouched.  Launch failures
 *    are reported as DKV_ERR_DEVICE.  No C++ exception crosses this ABI.
 *  - The library holds no mutable global state other than the per-GPU
 *    scratch array of deltakv_decode_attn_noalloc (and the device address
 *    of that array, looked up once per GPU); calls on different streams with
 *    disjoint outputs and workspaces may run concurrently, except for that
 *    entry point, whose calls on one GPU share the array.
 *  - Results are deterministic: the same inputs give the same bytes.
 */
#ifndef DELTAKV_H
#define DELTAKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DKV_ABI_VERSION 5u

typedef enum dkv_status {
  DKV_OK = 0,
  DKV_ERR_NULL = 1,        /* a required pointer is NULL                     */
  DKV_ERR_SHAPE = 2,       /* a size is zero or sizes are inconsistent       */
  DKV_ERR_DTYPE = 3,       /* unknown storage dtype                          */
  DKV_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned         */
  DKV_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required        */
  DKV_ERR_UNSUPPORTED = 6, /* a valid but unsupported size (see dkv_layout)  */
  DKV_ERR_VERSION = 7,     /* dkv_layout.abi_version != DKV_ABI_VERSION      */
  DKV_ERR_DEVICE = 8       /* a HIP launch or device query failed            */
} dkv_status;

typedef enum dkv_dtype {
  DKV_F32 = 0,  /* IEEE binary32 storage                                   */
  DKV_BF16 = 1  /* bfloat16 storage (raw 16-bit patterns), fp32 arithmetic */
} dkv_dtype;

/*
 * Shape of one layer's compressed cache.  Plain data, passed by pointer.
 *   abi_version  must equal DKV_ABI_VERSION
 *   dtype        dkv_dtype of K, V, queries, W matrices and of refs/codes/mu
 *   head_dim     d; supported: 64 or 128
 *   code_dim     d_c; supported: a multiple of 16 with 16 <= d_c <= d
 *   stride       s >= 1 (s = 1 stores every token whole); supported up
 *                to 2^30
 *   idx_bytes    width of a stored reference ordinal: 2 (requires
 *                R_cap <= 65536) or 4
 *   n_kv_heads   H >= 1;  batch  B >= 1
 *   seq_len      T >= 1, tokens held in the cache
 *   capacity     tokens the arrays are sized for (T_cap >= T), so that
 *                tokens can be appended in place; 0 means T_cap = T;
 *                supported up to 2^30
 *   code_bits    0: codes in the storage dtype; 4: 4-bit codes, one scale
 *                per code row (DeltaKV explainer, Portuguese page, Resumo
 *                Técnico §4: the residuals cluster around zero and suit
 *                4-bit quantization; the pages give no scheme).  A row's
 *                code c (computed as for storage-dtype codes, before any
 *                rounding) is stored as scale = rnd(max_j |c_j| / 7) and
 *                q_j = clamp(round-half-even(c_j / scale), -8, 7) (q = 0
 *                when scale = 0); the decoder uses scale * q_j
 *   top_k        references each coded token keeps, 1 .. 8 (0 means 1):
 *                the k best earlier references, ties to the lower ordinal
 *                (all earlier ones when fewer than k exist); the residual
 *                and the reconstruction use their mean (English page,
 *                Technical Summary §3 "Strided Reference Selection" and
 *                "Residual Encoding": the k nearest references and their
 *                mean KV^R)
 *   metric       DKV_METRIC_COS (0): rank by cosine; DKV_METRIC_L2 (1): by
 *                smallest ||x~_t - refs[r]|| (the English page's L2 distance)
 *   order        DKV_ORDER_POSITION (0): code rows in position order (see
 *                dkv_cache); DKV_ORDER_BY_VALUE_REF (1): deltakv_compress
 *                stores the coded tokens of each (sequence, KV head) grouped
 *                by their value reference: the K and V rows (codes,
 *                ordinals, scales) of the N coded tokens are ordered by
 *                (V ordinal, position), so rows that share a value
 *                reference row are adjacent and a decode reads that row
 *                once per run instead of once per token.  Attention sums
 *                over the cached tokens, so any order of the rows decodes to
 *                the same result; the pages fix no storage order.  Requires
 *                top_k <= 1 and R_cap <= 32768; selective decode (which looks
 *                rows up by position) rejects such a cache.  Rows appended
 *                after the compress stay in position order after the N
 *                grouped rows.
 * Derived: R = ceil(T / s) references and N = T - R coded tokens per stream
 * are held; the arrays are laid out for R_cap = ceil(T_cap / s) and
 * N_cap = T_cap - R_cap (a cache's layout is fixed by T_cap, so a layout
 * with a larger seq_len and the same capacity describes the same buffer).
 */
typedef struct dkv_layout {
  uint32_t abi_version;
  uint32_t dtype;
  uint32_t head_dim;
  uint32_t code_dim;
  uint32_t stride;
  uint32_t idx_bytes;
  uint32_t n_kv_heads;
  uint32_t batch;
  uint32_t seq_len;
  uint32_t capacity;
  uint32_t code_bits;
  uint32_t top_k;
  uint32_t metric;
  uint32_t order;
} dkv_layout;

#define DKV_METRIC_COS 0u
#define DKV_METRIC_L2 1u
#define DKV_ORDER_POSITION 0u
#define DKV_ORDER_BY_VALUE_REF 1u

/*
 * Device pointers of a compressed cache.  All arrays are dense, row-major,
 * indexed [b][h][kv][...] with kv = 0 for K and 1 for V:
 *   refs   [B][H][2][R_cap][d]    storage dtype: x~ of the reference tokens
 *                                 (rows 0 .. R-1 in use)
 *   codes  [B][H][2][N_cap][d_c]  storage dtype: one row per non-reference
 *                                 token in position order; token t
 *                                 (t mod s != 0) sits in row
 *                                 t - floor(t / s) - 1 (rows 0 .. N-1 in use;
 *                                 with order = DKV_ORDER_BY_VALUE_REF rows
 *                                 0 .. N-1 hold the same tokens grouped, see
 *                                 dkv_layout)
 *                                 With code_bits = 4 a row is d_c / 2 bytes:
 *                                 element 2i in the low nibble of byte i,
 *                                 2i + 1 in the high nibble, two's complement
 *   idx    [B][H][2][N_cap][k]    uint16 or uint32 (idx_bytes): reference
 *                                 ordinals r of each row (the token at r*s),
 *                                 k = top_k, in ascending order; a token with
 *                                 c < k earlier references fills slots
 *                                 c .. k-1 with 0
 *   mu     [B][H][2][d]           storage dtype: the shared component
 *   scales [B][H][2][N_cap]       storage dtype, code_bits = 4 only (else
 *                                 ignored, may be NULL): scale of each row
 * Each pointer must be 16-byte aligned.
 */
typedef struct dkv_cache {
  void* refs;
  void* codes;
  void* idx;
  void* mu;
  void* scales;
} dkv_cache;

/*
 * Inputs of deltakv_compress.
 *   k, v       device; element (b, h, t, i) of K is at
 *              k[b*stride_b + h*stride_h + t*stride_t + i] (elements, storage
 *              dtype); the same strides apply to v; the head_dim elements of
 *              a token are contiguous; stride_t must be a multiple of 8
 *   w_down_k   device [d_c][d] storage dtype, compressor of K (row j gives
 *              code element j); w_down_v likewise for V
 *   w_head_stride  elements between consecutive heads' matrices; 0 = one
 *              matrix shared by all heads
 *   mu_in      optional device [B][H][2][d]: use this shared component
 *              instead of computing the mean (NULL = compute)
 *   stage_events  optional host array of DKV_COMPRESS_EVENTS hipEvent_t
 *              handles (NULL = none): a (start, stop) pair per stage, in the
 *              order mean, center, search, encode (with a grouped order the
 *              encode stage begins with the grouping).  Start is stamped when the
 *              stage's first kernel starts executing and stop when its last
 *              kernel ends, so hipEventElapsedTime(start, stop) is the
 *              stage's device time.  Not allowed while `stream` is being
 *              captured into a graph (DKV_ERR_UNSUPPORTED).
 */
#define DKV_COMPRESS_EVENTS 8
typedef struct dkv_compress_in {
  const void* k;
  const void* v;
  int64_t stride_b;
  int64_t stride_h;
  int64_t stride_t;
  const void* w_down_k;
  const void* w_down_v;
  int64_t w_head_stride;
  const void* mu_in;
  void* const* stage_events;
} dkv_compress_in;

/*
 * Inputs and output of deltakv_decode_attn (one query token per sequence).
 *   q          device [B][Hq][d] storage dtype, contiguous
 *   w_up_k     device [d][d_c] storage dtype, decompressor of K (column j
 *              multiplies code element j); w_up_v likewise for V
 *   w_head_stride  as in dkv_compress_in
 *   n_q_heads  Hq, a multiple of H with G = Hq / H <= 16; query head g
 *              attends over KV head g / G
 *   n_splits   sequence splits per (b, h); 0 = choose automatically (see
 *              dkv_decode_auto_splits); at most 1024
 *   softmax_scale  multiplies q . k^; 0 means 1 / sqrt(d)
 *   out        device [B][Hq][d] float32, written whole
 *   stage_events  optional host array of DKV_DECODE_EVENTS hipEvent_t
 *              handles (NULL = none): (start, stop) pairs of the stages
 *              reference scores, split, combine, as for
 *              dkv_compress_in.stage_events
 */
#define DKV_DECODE_EVENTS 6
typedef struct dkv_decode_in {
  const void* q;
  const void* w_up_k;
  const void* w_up_v;
  int64_t w_head_stride;
  uint32_t n_q_heads;
  uint32_t n_splits;
  float softmax_scale;
  uint32_t reserved; /* must be 0 */
  float* out;
  void* const* stage_events;
} dkv_decode_in;

/*
 * Inputs of deltakv_append (one new token per sequence, at position seq_len).
 *   k, v       device; element (b, h, i) of the new K token is at
 *              k[b*stride_b + h*stride_h + i] (elements, storage dtype); the
 *              same strides apply to v; the head_dim elements are contiguous
 *              and 16-byte aligned
 *   w_down_k, w_down_v, w_head_stride  as in dkv_compress_in
 *   stage_events  optional host array of DKV_APPEND_EVENTS hipEvent_t
 *              handles (NULL = none): (start, stop) pairs of the stages
 *              search and finish (merge, then store the row), as for
 *              dkv_compress_in.stage_events; for a token that becomes a
 *              reference the search pair is recorded with nothing between
 */
#define DKV_APPEND_EVENTS 4
typedef struct dkv_append_in {
  const void* k;
  const void* v;
  int64_t stride_b;
  int64_t stride_h;
  const void* w_down_k;
  const void* w_down_v;
  int64_t w_head_stride;
  void* const* stage_events;
} dkv_append_in;

/*
 * Token list of a selective decode (deltakv_decode_attn_sel).
 *   tokens     device [B][n_sel] uint32 token positions, 4-byte aligned;
 *              row b lists the tokens sequence b attends to.  Each entry is
 *              one term of the softmax: a position listed twice counts
 *              twice, and the order of a row does not matter (ascending
 *              order reads the cache in order and is fastest).  Entries at
 *              or past seq_len are skipped.
 *   n_sel      entries per sequence, 1 .. 2^30
 *   reserved   must be 0
 */
typedef struct dkv_token_sel {
  const uint32_t* tokens;
  uint32_t n_sel;
  uint32_t reserved;
} dkv_token_sel;

/* DKV_ABI_VERSION of the loaded library. */
uint32_t dkv_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* dkv_status_str(dkv_status status);

/* Validates a layout: DKV_OK or the first error found. */
dkv_status dkv_layout_check(const dkv_layout* layout);

/* Bytes of the four cache arrays, each rounded up to 256 bytes, as carved by
 * dkv_cache_carve.  0 if the layout is invalid. */
size_t dkv_cache_bytes(const dkv_layout* layout);

/* Splits one device buffer of dkv_cache_bytes(layout) bytes starting at
 * `base` (256-byte aligned) into refs, codes, idx, mu and (code_bits = 4)
 * scales, in that order, each at a 256-byte boundary; scales is NULL for
 * storage-dtype codes.  Writes only *cache. */
dkv_status dkv_cache_carve(const dkv_layout* layout, void* base, dkv_cache* cache);

/* Workspace bytes deltakv_compress needs for this layout (0 if invalid). */
size_t dkv_compress_workspace_bytes(const dkv_layout* layout);

/* Split count deltakv_decode_attn uses when n_splits = 0. */
uint32_t dkv_decode_auto_splits(const dkv_layout* layout, uint32_t n_q_heads);

/* Workspace bytes deltakv_decode_attn needs (0 if invalid); n_splits = 0
 * means the automatic count. */
size_t dkv_decode_workspace_bytes(const dkv_layout* layout, uint32_t n_q_heads, uint32_t n_splits);

/*
 * Compresses one layer's prefill K and V into `cache` (all four arrays are
 * written whole).  `ws` is a device buffer of at least
 * dkv_compress_workspace_bytes(layout) bytes, 16-byte aligned; its contents
 * on entry do not matter.  Steps: shared component (English page, Technical
 * Summary §2 "Highly Shared Latent Components"), centred references at
 * stride s and their norms, reference search (§3 "Strided Reference
 * Selection"), residual codes (§3 "Residual Encoding"; French page,
 * Méthodologie §2 "Architecture de compression").
 */
dkv_status deltakv_compress(const dkv_layout* layout, const dkv_compress_in* in, const dkv_cache* cache,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * Appends the token at position T = layout->seq_len of every sequence to a
 * cache that holds T tokens, in place: with the shared component mu kept
 * as it is in the cache, a token with T mod s = 0 becomes reference T / s;
 * any other token is searched against the references r with r*s < T and
 * stored as its ordinal and code in row T - floor(T / s) - 1, exactly as
 * deltakv_compress of the T + 1 tokens with mu_in = mu would store it (the
 * same readings; DeltaKV explainer, English page, Technical Summary §3
 * "Strided Reference Selection", which retrieves references for each new
 * token).  Requires T + 1 <= capacity; the caller then describes the cache
 * with seq_len = T + 1.  Writes only that token's row of refs, or of codes
 * and idx.  `ws` as for deltakv_compress, of at least
 * dkv_append_workspace_bytes(layout) bytes (a few bytes per stream; the
 * bound covers every length up to the capacity, so one workspace serves all
 * appends to the cache).
 */
size_t dkv_append_workspace_bytes(const dkv_layout* layout);
dkv_status deltakv_append(const dkv_layout* layout, const dkv_append_in* in, const dkv_cache* cache, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * Decode attention of one query per sequence over a compressed cache, as if
 * every token were reconstructed and attended to (English page, Technical
 * Summary §3 "Reconstruction": a token is its decoded code plus its
 * reference); mathematically equal to softmax(q K^T * scale) V^ over the
 * reconstructed K^ and V^, computed without materialising them (the shared
 * key component shifts every score equally and is not read).  `ws` as for
 * deltakv_compress, of at least dkv_decode_workspace_bytes(layout,
 * n_q_heads, n_splits) bytes.
 */
dkv_status deltakv_decode_attn(const dkv_layout* layout, const dkv_cache* cache, const dkv_decode_in* in,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * deltakv_decode_attn with its workspace taken from a device array the
 * library holds, DKV_NOALLOC_SCRATCH_BYTES bytes on each GPU it runs on
 * (created with the library's device code on that GPU and kept until the
 * process ends).  The call allocates nothing.  Returns DKV_ERR_WORKSPACE,
 * before touching the device, when dkv_decode_workspace_bytes(layout,
 * n_q_heads, n_splits) exceeds that size (16 MiB covers, for example, 16
 * sequences x 8 KV heads x 32768 tokens at stride 16).  Every call on a GPU
 * uses that GPU's one array: calls that overlap on one GPU (different
 * streams, or several threads) race and must not be issued; calls ordered
 * on one stream are fine.  Arguments (no workspace) and results as
 * deltakv_decode_attn, on the current device.
 */
#define DKV_NOALLOC_SCRATCH_BYTES (16u << 20)
dkv_status deltakv_decode_attn_noalloc(const dkv_layout* layout, const dkv_cache* cache, const dkv_decode_in* in,
                                       void* stream);

/*
 * Decode attention over a chosen subset of the cached tokens: for each
 * sequence b, softmax(q k^_t^T * scale) v^_t over the entries t of row b of
 * sel->tokens, every other token left untouched (DeltaKV explainer, Spanish
 * page, Resumen Técnico §2 "Metodología": with a sparse-attention method
 * only the tokens its mask keeps are reconstructed; German page §2, an
 * engine that decompresses only those tokens).  A sequence whose row holds
 * no entry below seq_len gets an output of zeros.  Arguments as for
 * deltakv_decode_attn; in->n_splits = 0 takes
 * dkv_decode_sel_auto_splits, which never exceeds dkv_decode_auto_splits,
 * so a workspace of dkv_decode_workspace_bytes(layout, n_q_heads, 0) bytes
 * serves both calls.  stage_events as for deltakv_decode_attn.  A layout
 * with order = DKV_ORDER_BY_VALUE_REF returns DKV_ERR_UNSUPPORTED (its rows
 * are not found by position).
 */
uint32_t dkv_decode_sel_auto_splits(const dkv_layout* layout, uint32_t n_q_heads, uint32_t n_sel);
dkv_status deltakv_decode_attn_sel(const dkv_layout* layout, const dkv_cache* cache, const dkv_decode_in* in,
                                   const dkv_token_sel* sel, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DELTAKV_H */
