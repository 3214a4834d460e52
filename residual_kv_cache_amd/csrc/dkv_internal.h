// Internal declarations shared by the host entry points and the kernels of
// the DeltaKV library.  Not part of the ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/deltakv.h"

namespace dkv {

// Sizes derived from a validated dkv_layout.
struct Shape {
  int d;        // head dim
  int dc;       // code dim
  int s;        // reference stride
  int R;        // references per stream, ceil(T / s)
  int N;        // coded tokens per stream, T - R
  int T;        // tokens per stream
  int Rc;       // reference rows per stream in the arrays, ceil(T_cap / s)
  int Nc;       // code rows per stream in the arrays, T_cap - Rc
  int H;        // KV heads
  int B;        // sequences
  int idx_bytes;
  int bf16;     // 1 = bfloat16 storage, 0 = float32
  int q4;       // 1 = 4-bit codes with one scale per row
  int K;        // references per coded token (top_k)
  int l2;       // 1 = references ranked by L2 distance, 0 = by cosine
  int grouped;  // 1 = coded rows of a head grouped by value reference
  // The fast paths (top-1 cosine search; token-tile decode) serve K = 1.
  __host__ __device__ bool topk_search() const { return K > 1 || l2; }
  __host__ __device__ int n_streams() const { return B * H * 2; }
  int elem() const { return bf16 ? 2 : 4; }
  // Bytes of one code row.
  __host__ __device__ int code_row_bytes() const { return q4 ? dc / 2 : dc * (bf16 ? 2 : 4); }
};

// XCD-aware block order: block L runs on XCD L % 8 (workgroups are
// dispatched to the eight XCDs round-robin).  Streams x, x + 8, ... are
// given to XCD x, so the references a stream re-reads stay in one L2; within
// an XCD, work items go in the given order across its streams.
struct XcdItem {
  int stream, item;   // stream < 0: no work
};
__device__ __forceinline__ XcdItem xcd_item(int ns) {
  const int per = (ns + 7) / 8;
  const int xcd = blockIdx.x & 7, k = blockIdx.x >> 3;
  XcdItem r;
  r.stream = xcd + 8 * (k % per);
  r.item = k / per;
  if (r.stream >= ns) r.stream = -1;
  return r;
}
inline unsigned xcd_grid(int ns, int items) { return 8u * (unsigned)((ns + 7) / 8) * (unsigned)items; }

// Tokens summed per block in the first mean stage.
constexpr int kMeanChunk = 512;

inline int mean_chunks(const Shape& sh) { return (sh.T + kMeanChunk - 1) / kMeanChunk; }

// Compress workspace: fp64 mean partials, then fp32 inverse reference norms.
inline size_t ws_mean_off(const Shape&) { return 0; }
inline size_t ws_mean_bytes(const Shape& sh) {
  return (size_t)sh.n_streams() * mean_chunks(sh) * sh.d * sizeof(double);
}
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline size_t ws_invn_off(const Shape& sh) { return align_up(ws_mean_bytes(sh), 256); }
inline size_t ws_invn_bytes(const Shape& sh) { return (size_t)sh.n_streams() * sh.R * sizeof(float); }
// Grouped layouts add: the ordinals in position order (written by the
// search, read by the grouping and the encode), the grouped row of each
// position row per head, and the per-piece reference counts per head.
constexpr int kGroupPiece = 2048;    // coded rows per grouping block
constexpr int kGroupThreads = kGroupPiece / 4;   // threads of a grouping block (4 rows each)
constexpr int kGroupMaxRefs = 32768; // LDS counters of one grouping block
inline int group_pieces(const Shape& sh) { return (sh.N + kGroupPiece - 1) / kGroupPiece; }
inline size_t ws_gidx_off(const Shape& sh) { return align_up(ws_invn_off(sh) + ws_invn_bytes(sh), 256); }
inline size_t ws_gidx_bytes(const Shape& sh) {
  return sh.grouped ? (size_t)sh.n_streams() * sh.Nc * sh.idx_bytes : 0;
}
inline size_t ws_perm_off(const Shape& sh) { return align_up(ws_gidx_off(sh) + ws_gidx_bytes(sh), 256); }
inline size_t ws_perm_bytes(const Shape& sh) { return sh.grouped ? (size_t)sh.B * sh.H * sh.Nc * 4 : 0; }
inline size_t ws_gcnt_off(const Shape& sh) { return align_up(ws_perm_off(sh) + ws_perm_bytes(sh), 256); }
inline size_t ws_gcnt_bytes(const Shape& sh) {
  return sh.grouped ? (size_t)sh.B * sh.H * ((sh.Nc + kGroupPiece - 1) / kGroupPiece) * sh.Rc * 4 : 0;
}
inline size_t ws_gtot_off(const Shape& sh) { return align_up(ws_gcnt_off(sh) + ws_gcnt_bytes(sh), 256); }
inline size_t ws_gtot_bytes(const Shape& sh) { return sh.grouped ? (size_t)sh.B * sh.H * sh.Rc * 4 : 0; }
inline size_t compress_ws_bytes(const Shape& sh) { return align_up(ws_gtot_off(sh) + ws_gtot_bytes(sh), 256); }

// Decode workspace: reference scores S [B][H][R][Gs] (Gs = G rounded up to
// a multiple of 4, padding zero), projected queries q' [B][H][G][dc] and
// split partials [B][H][splits][G][rec].
__host__ __device__ inline int partial_rec(const Shape& sh) { return (2 + sh.dc + sh.d + 3) / 4 * 4; }
__host__ __device__ inline int score_cols(int G) { return (G + 3) / 4 * 4; }
inline size_t ws_score_bytes(const Shape& sh, int G) {
  return (size_t)sh.B * sh.H * sh.R * score_cols(G) * sizeof(float);
}
inline size_t ws_qp_off(const Shape& sh, int G) { return align_up(ws_score_bytes(sh, G), 256); }
inline size_t ws_qp_bytes(const Shape& sh, int G) { return (size_t)sh.B * sh.H * G * sh.dc * sizeof(float); }
inline size_t ws_part_off(const Shape& sh, int G) { return align_up(ws_qp_off(sh, G) + ws_qp_bytes(sh, G), 256); }
inline size_t ws_part_bytes(const Shape& sh, int G, int splits) {
  return (size_t)sh.B * sh.H * splits * G * partial_rec(sh) * sizeof(float);
}
inline size_t decode_ws_bytes(const Shape& sh, int G, int splits) {
  return align_up(ws_part_off(sh, G) + ws_part_bytes(sh, G, splits), 256);
}

// MFMA decode (decode_mfma.hip): bfloat16 storage, head dim 128, up to 4
// query heads per KV head, code dim up to 48, at most kMfmaMaxSplits splits.
constexpr int kMfmaMaxSplits = 256;
bool decode_fused_supported(const Shape& sh, int G, int splits);
// The same path over a token list (d_c <= 32).
bool decode_sel_fused_supported(const Shape& sh, int G, int splits);
// The MFMA reference-score and combine kernels alone (any code format).
bool mfma_side_kernels_supported(const Shape& sh, int G, int splits);
int decode_fused_auto_splits(const Shape& sh);

struct CompressArgs {
  const void* k;
  const void* v;
  int64_t sb, sh, st;        // element strides of k and v
  const void* wdk;
  const void* wdv;
  int64_t w_hs;              // head stride of W_down (elements), 0 = shared
  const void* mu_in;
  void* refs;
  void* codes;
  void* idx;
  void* mu;
  void* scales;              // 4-bit codes: per-row scales, else NULL
  double* mean_part;
  float* inv_n;
  // Grouped layouts (else NULL): idx above is the position-order workspace
  // copy; idx_out is the cache's array, perm the grouped row of each
  // position row [B*H][N_cap], gcnt the per-piece counts [B*H][pieces][R]
  // (then each piece's count of the ordinal in earlier pieces), gtot the
  // rows per ordinal [B*H][R].
  void* idx_out;
  int* perm;
  int* gcnt;
  int* gtot;
  void* const* events;       // DKV_COMPRESS_EVENTS hipEvent_t or NULL
};

struct DecodeArgs {
  const void* q;
  const void* wuk;
  const void* wuv;
  int64_t w_hs;
  int G;                     // query heads per KV head
  int Hq;
  int splits;
  float scale;
  float* out;
  const void* refs;
  const void* codes;
  const void* idx;
  const void* mu;
  const void* scales;        // 4-bit codes: per-row scales, else NULL
  float* score;              // [B][H][R][score_cols(G)]
  float* qp;                 // [B][H][G][dc]
  float* part;               // [B][H][splits][G][rec]
  void* const* events;       // DKV_DECODE_EVENTS hipEvent_t or NULL
  const uint32_t* sel;       // selective decode: token positions [B][n_sel], else NULL
  int n_sel;
};

// Stage timing: event pair (start, stop) of stage i from an optional array.
inline hipEvent_t ev_start(void* const* ev, int i) { return ev ? (hipEvent_t)ev[2 * i] : nullptr; }
inline hipEvent_t ev_stop(void* const* ev, int i) { return ev ? (hipEvent_t)ev[2 * i + 1] : nullptr; }

// Launches a kernel; with events, the start event is stamped when the
// kernel begins executing and the stop event when it ends (AMD's extended
// launch), so host-side launch gaps never enter the measured time.
template <typename... KArgs, typename... Args>
inline hipError_t launch_lds(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t st,
                             hipEvent_t start, hipEvent_t stop, Args... args) {
  if (start || stop)
    hipExtLaunchKernelGGL(kernel, grid, block, lds, st, start, stop, 0, args...);
  else
    kernel<<<grid, block, lds, st>>>(args...);
  return hipGetLastError();
}
template <typename... KArgs, typename... Args>
inline hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t st, hipEvent_t start,
                         hipEvent_t stop, Args... args) {
  return launch_lds(kernel, grid, block, 0, st, start, stop, args...);
}

struct AppendArgs {
  const void* k;
  const void* v;
  int64_t sb, sh;            // element strides of k and v
  const void* wdk;
  const void* wdv;
  int64_t w_hs;
  void* refs;
  void* codes;
  void* idx;
  const void* mu;
  void* scales;              // 4-bit codes: per-row scales, else NULL
  void* const* events;       // DKV_APPEND_EVENTS hipEvent_t or NULL
};

// Append search: about kAppendBlocks blocks over all streams, each scoring a
// chunk of at least kAppendMinChunk references (a multiple of it).
constexpr int kAppendBlocks = 2048;
constexpr int kAppendMinChunk = 64;
int append_chunk(const Shape& sh, int nref);
int append_parts(const Shape& sh, int nref);
size_t append_ws_bytes(const Shape& sh);

hipError_t launch_compress(const Shape& sh, const CompressArgs& a, hipStream_t st);
// sh describes the cache after the append (T = position of the new token + 1).
hipError_t launch_append(const Shape& sh, const AppendArgs& a, void* ws, hipStream_t st);
hipError_t launch_decode(const Shape& sh, const DecodeArgs& a, hipStream_t st);
hipError_t launch_decode_fused(const Shape& sh, const DecodeArgs& a, hipStream_t st);
hipError_t launch_decode_sel_fused(const Shape& sh, const DecodeArgs& a, hipStream_t st);
// Decode over a token list (a.sel): reference scores, the list's split, combine.
hipError_t launch_decode_sel(const Shape& sh, const DecodeArgs& a, hipStream_t st);
// The MFMA reference-score kernel alone (shapes decode_fused_supported accepts).
hipError_t launch_refscore_mfma(const Shape& sh, const DecodeArgs& a, hipStream_t st);
// The MFMA path's combine alone (reads partial records of any split kernel).
hipError_t launch_combine_mfma(const Shape& sh, const DecodeArgs& a, hipStream_t st);

}  // namespace dkv
