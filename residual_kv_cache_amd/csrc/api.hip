// Host side of the DeltaKV C ABI: validation, layout arithmetic, workspace
// carving and kernel dispatch.  Every check runs before anything is
// enqueued; on error nothing is launched.

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "dkv_internal.h"

using dkv::Shape;

namespace {

constexpr size_t kAlign = 256;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

dkv_status check_layout(const dkv_layout* L, Shape* out) {
  if (!L) return DKV_ERR_NULL;
  if (L->abi_version != DKV_ABI_VERSION) return DKV_ERR_VERSION;
  if (L->dtype != DKV_F32 && L->dtype != DKV_BF16) return DKV_ERR_DTYPE;
  if (L->head_dim == 0 || L->code_dim == 0 || L->stride == 0 || L->n_kv_heads == 0 || L->batch == 0 ||
      L->seq_len == 0)
    return DKV_ERR_SHAPE;
  const uint32_t cap = L->capacity ? L->capacity : L->seq_len;
  if (cap < L->seq_len) return DKV_ERR_SHAPE;
  if (L->code_dim > L->head_dim) return DKV_ERR_SHAPE;
  if (L->idx_bytes != 2 && L->idx_bytes != 4) return DKV_ERR_SHAPE;
  if (L->code_bits != 0 && L->code_bits != 4) return DKV_ERR_SHAPE;
  if (L->metric != DKV_METRIC_COS && L->metric != DKV_METRIC_L2) return DKV_ERR_SHAPE;
  if (L->order != DKV_ORDER_POSITION && L->order != DKV_ORDER_BY_VALUE_REF) return DKV_ERR_SHAPE;
  if (L->top_k > 8) return DKV_ERR_UNSUPPORTED;
  if (L->order == DKV_ORDER_BY_VALUE_REF && L->top_k > 1) return DKV_ERR_UNSUPPORTED;
  if (L->head_dim != 64 && L->head_dim != 128) return DKV_ERR_UNSUPPORTED;
  if (L->code_dim % 16 != 0) return DKV_ERR_UNSUPPORTED;
  // Strides up to 2^30 (one reference per 2^30 tokens) keep every
  // position and slot computation of the kernels inside int32.
  if (cap > (1u << 30) || L->stride > (1u << 30) || L->n_kv_heads > 4096 || L->batch > 65535)
    return DKV_ERR_UNSUPPORTED;
  const uint64_t R = ((uint64_t)L->seq_len + L->stride - 1) / L->stride;
  const uint64_t Rc = ((uint64_t)cap + L->stride - 1) / L->stride;
  if (L->idx_bytes == 2 && Rc > 65536) return DKV_ERR_UNSUPPORTED;
  if (L->order == DKV_ORDER_BY_VALUE_REF && Rc > (uint64_t)dkv::kGroupMaxRefs) return DKV_ERR_UNSUPPORTED;
  const uint64_t streams = 2ull * L->batch * L->n_kv_heads;
  if (streams > 65535) return DKV_ERR_UNSUPPORTED;  // grid y limit of the stream axis
  if (out) {
    out->d = (int)L->head_dim;
    out->dc = (int)L->code_dim;
    out->s = (int)L->stride;
    out->T = (int)L->seq_len;
    out->R = (int)R;
    out->N = (int)(L->seq_len - R);
    out->Rc = (int)Rc;
    out->Nc = (int)(cap - Rc);
    out->H = (int)L->n_kv_heads;
    out->B = (int)L->batch;
    out->idx_bytes = (int)L->idx_bytes;
    out->bf16 = L->dtype == DKV_BF16;
    out->q4 = L->code_bits == 4;
    out->K = L->top_k ? (int)L->top_k : 1;
    out->l2 = L->metric == DKV_METRIC_L2;
    out->grouped = L->order == DKV_ORDER_BY_VALUE_REF;
  }
  return DKV_OK;
}

struct ArrayBytes {
  size_t refs, codes, idx, mu, scales;
};

ArrayBytes array_bytes(const Shape& sh) {
  const size_t n = (size_t)sh.n_streams();
  ArrayBytes a;
  a.refs = n * sh.Rc * sh.d * sh.elem();
  a.codes = n * sh.Nc * sh.code_row_bytes();
  a.idx = n * sh.Nc * sh.K * sh.idx_bytes;
  a.mu = n * sh.d * sh.elem();
  a.scales = sh.q4 ? n * sh.Nc * sh.elem() : 0;
  return a;
}

size_t pad(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

dkv_status check_cache(const dkv_cache* c, const Shape& sh) {
  if (!c) return DKV_ERR_NULL;
  if (!c->refs || !c->mu) return DKV_ERR_NULL;
  if (sh.Nc > 0 && (!c->codes || !c->idx)) return DKV_ERR_NULL;
  if (sh.q4 && sh.Nc > 0 && !c->scales) return DKV_ERR_NULL;
  if (!aligned16(c->refs) || !aligned16(c->codes) || !aligned16(c->idx) || !aligned16(c->mu)) return DKV_ERR_ALIGN;
  if (sh.q4 && !aligned16(c->scales)) return DKV_ERR_ALIGN;
  return DKV_OK;
}

uint32_t auto_splits(const Shape& sh, int G) {
  if (dkv::decode_fused_supported(sh, G, 1)) return (uint32_t)dkv::decode_fused_auto_splits(sh);
  // General path (256-thread blocks): about 2048 blocks over the B*H heads,
  // at least 256 cached tokens per split, at most 1024 splits.
  const int64_t heads = (int64_t)sh.B * sh.H;
  int64_t by_chip = (2048 + heads - 1) / heads;
  int64_t by_len = (sh.T + 255) / 256;
  int64_t s = by_chip < by_len ? by_chip : by_len;
  if (s < 1) s = 1;
  if (s > 1024) s = 1024;
  return (uint32_t)s;
}

dkv_status from_hip(hipError_t e) { return e == hipSuccess ? DKV_OK : DKV_ERR_DEVICE; }

// Stage events use the extended launch, which stream capture does not take.
dkv_status check_events(void* const* ev, void* stream) {
  if (!ev) return DKV_OK;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing((hipStream_t)stream, &cs) != hipSuccess) return DKV_ERR_DEVICE;
  return cs == hipStreamCaptureStatusNone ? DKV_OK : DKV_ERR_UNSUPPORTED;
}

}  // namespace

extern "C" {

uint32_t dkv_abi_version(void) { return DKV_ABI_VERSION; }

const char* dkv_status_str(dkv_status s) {
  switch (s) {
    case DKV_OK: return "DKV_OK";
    case DKV_ERR_NULL: return "DKV_ERR_NULL: a required pointer is NULL";
    case DKV_ERR_SHAPE: return "DKV_ERR_SHAPE: a size is zero or sizes are inconsistent";
    case DKV_ERR_DTYPE: return "DKV_ERR_DTYPE: unknown storage dtype";
    case DKV_ERR_ALIGN: return "DKV_ERR_ALIGN: a device pointer or stride is not 16-byte aligned";
    case DKV_ERR_WORKSPACE: return "DKV_ERR_WORKSPACE: workspace missing or too small";
    case DKV_ERR_UNSUPPORTED: return "DKV_ERR_UNSUPPORTED: valid but unsupported size";
    case DKV_ERR_VERSION: return "DKV_ERR_VERSION: ABI version mismatch";
    case DKV_ERR_DEVICE: return "DKV_ERR_DEVICE: a HIP launch or device query failed";
  }
  return "DKV_ERR_UNKNOWN";
}

dkv_status dkv_layout_check(const dkv_layout* layout) { return check_layout(layout, nullptr); }

size_t dkv_cache_bytes(const dkv_layout* layout) {
  Shape sh;
  if (check_layout(layout, &sh) != DKV_OK) return 0;
  const ArrayBytes a = array_bytes(sh);
  return pad(a.refs) + pad(a.codes) + pad(a.idx) + pad(a.mu) + pad(a.scales);
}

dkv_status dkv_cache_carve(const dkv_layout* layout, void* base, dkv_cache* cache) {
  Shape sh;
  dkv_status st = check_layout(layout, &sh);
  if (st != DKV_OK) return st;
  if (!base || !cache) return DKV_ERR_NULL;
  if (((uintptr_t)base % kAlign) != 0) return DKV_ERR_ALIGN;
  const ArrayBytes a = array_bytes(sh);
  char* p = (char*)base;
  cache->refs = p;
  p += pad(a.refs);
  cache->codes = p;
  p += pad(a.codes);
  cache->idx = p;
  p += pad(a.idx);
  cache->mu = p;
  p += pad(a.mu);
  cache->scales = sh.q4 ? p : nullptr;
  return DKV_OK;
}

size_t dkv_compress_workspace_bytes(const dkv_layout* layout) {
  Shape sh;
  if (check_layout(layout, &sh) != DKV_OK) return 0;
  return dkv::compress_ws_bytes(sh);
}

uint32_t dkv_decode_auto_splits(const dkv_layout* layout, uint32_t n_q_heads) {
  Shape sh;
  if (check_layout(layout, &sh) != DKV_OK) return 0;
  if (n_q_heads == 0 || n_q_heads % sh.H != 0 || n_q_heads / sh.H > 16) return 0;
  return auto_splits(sh, (int)(n_q_heads / sh.H));
}

size_t dkv_decode_workspace_bytes(const dkv_layout* layout, uint32_t n_q_heads, uint32_t n_splits) {
  Shape sh;
  if (check_layout(layout, &sh) != DKV_OK) return 0;
  if (n_q_heads == 0 || n_q_heads % sh.H != 0 || n_q_heads / sh.H > 16) return 0;
  if (n_splits > 1024) return 0;
  const int G = (int)(n_q_heads / sh.H);
  const int splits = n_splits ? (int)n_splits : (int)auto_splits(sh, G);
  return dkv::decode_ws_bytes(sh, G, splits);
}

dkv_status deltakv_compress(const dkv_layout* layout, const dkv_compress_in* in, const dkv_cache* cache, void* ws,
                            size_t ws_bytes, void* stream) {
  Shape sh;
  dkv_status st = check_layout(layout, &sh);
  if (st != DKV_OK) return st;
  if (!in) return DKV_ERR_NULL;
  if (!in->k || !in->v || !in->w_down_k || !in->w_down_v) return DKV_ERR_NULL;
  if ((st = check_cache(cache, sh)) != DKV_OK) return st;
  if (!aligned16(in->k) || !aligned16(in->v) || !aligned16(in->w_down_k) || !aligned16(in->w_down_v) ||
      !aligned16(in->mu_in))
    return DKV_ERR_ALIGN;
  if (in->stride_t < sh.d || in->stride_b < 0 || in->stride_h < 0 || in->w_head_stride < 0) return DKV_ERR_SHAPE;
  if (in->stride_t % 8 || in->stride_b % 8 || in->stride_h % 8 || in->w_head_stride % 8) return DKV_ERR_ALIGN;
  if (in->w_head_stride != 0 && in->w_head_stride < (int64_t)sh.d * sh.dc) return DKV_ERR_SHAPE;
  const size_t need = dkv::compress_ws_bytes(sh);
  if (!ws || ws_bytes < need) return DKV_ERR_WORKSPACE;
  if (!aligned16(ws)) return DKV_ERR_ALIGN;

  dkv::CompressArgs a;
  a.k = in->k;
  a.v = in->v;
  a.sb = in->stride_b;
  a.sh = in->stride_h;
  a.st = in->stride_t;
  a.wdk = in->w_down_k;
  a.wdv = in->w_down_v;
  a.w_hs = in->w_head_stride;
  a.mu_in = in->mu_in;
  a.refs = cache->refs;
  a.codes = cache->codes;
  a.idx = cache->idx;
  a.mu = cache->mu;
  a.scales = sh.q4 ? cache->scales : nullptr;
  a.mean_part = (double*)((char*)ws + dkv::ws_mean_off(sh));
  a.inv_n = (float*)((char*)ws + dkv::ws_invn_off(sh));
  a.idx_out = nullptr;
  a.perm = nullptr;
  a.gcnt = nullptr;
  a.gtot = nullptr;
  if (sh.grouped) {
    // The search writes ordinals in position order to the workspace; the
    // grouping places them (and the encode places the codes) in the cache.
    a.idx_out = cache->idx;
    a.idx = (char*)ws + dkv::ws_gidx_off(sh);
    a.perm = (int*)((char*)ws + dkv::ws_perm_off(sh));
    a.gcnt = (int*)((char*)ws + dkv::ws_gcnt_off(sh));
    a.gtot = (int*)((char*)ws + dkv::ws_gtot_off(sh));
  }
  a.events = in->stage_events;
  if ((st = check_events(a.events, stream)) != DKV_OK) return st;
  return from_hip(dkv::launch_compress(sh, a, (hipStream_t)stream));
}

size_t dkv_append_workspace_bytes(const dkv_layout* layout) {
  Shape sh;
  if (check_layout(layout, &sh) != DKV_OK) return 0;
  return dkv::append_ws_bytes(sh);
}

dkv_status deltakv_append(const dkv_layout* layout, const dkv_append_in* in, const dkv_cache* cache, void* ws,
                          size_t ws_bytes, void* stream) {
  Shape sh;
  dkv_status st = check_layout(layout, &sh);
  if (st != DKV_OK) return st;
  if (!in) return DKV_ERR_NULL;
  if (!in->k || !in->v || !in->w_down_k || !in->w_down_v) return DKV_ERR_NULL;
  if ((st = check_cache(cache, sh)) != DKV_OK) return st;
  const uint32_t cap = layout->capacity ? layout->capacity : layout->seq_len;
  if (layout->seq_len + 1 > cap) return DKV_ERR_SHAPE;
  if (!aligned16(in->k) || !aligned16(in->v) || !aligned16(in->w_down_k) || !aligned16(in->w_down_v))
    return DKV_ERR_ALIGN;
  if (in->stride_b < 0 || in->stride_h < 0 || in->w_head_stride < 0) return DKV_ERR_SHAPE;
  if (in->stride_b % 8 || in->stride_h % 8 || in->w_head_stride % 8) return DKV_ERR_ALIGN;
  if (in->w_head_stride != 0 && in->w_head_stride < (int64_t)sh.d * sh.dc) return DKV_ERR_SHAPE;
  if (!ws || ws_bytes < dkv::append_ws_bytes(sh)) return DKV_ERR_WORKSPACE;
  if (!aligned16(ws)) return DKV_ERR_ALIGN;
  if ((st = check_events(in->stage_events, stream)) != DKV_OK) return st;
  // The new token is position T: references and codes of T + 1 tokens.
  Shape s2 = sh;
  s2.T = sh.T + 1;
  s2.R = (s2.T + sh.s - 1) / sh.s;
  s2.N = s2.T - s2.R;
  dkv::AppendArgs a;
  a.k = in->k;
  a.v = in->v;
  a.sb = in->stride_b;
  a.sh = in->stride_h;
  a.wdk = in->w_down_k;
  a.wdv = in->w_down_v;
  a.w_hs = in->w_head_stride;
  a.refs = cache->refs;
  a.codes = cache->codes;
  a.idx = cache->idx;
  a.mu = cache->mu;
  a.scales = sh.q4 ? cache->scales : nullptr;
  a.events = in->stage_events;
  return from_hip(dkv::launch_append(s2, a, ws, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Validation and argument set-up shared by the two decode entry points;
// `sel_splits` > 0 replaces the automatic split count (selective decode).
dkv_status decode_setup(const dkv_layout* layout, const dkv_cache* cache, const dkv_decode_in* in, void* ws,
                        size_t ws_bytes, void* stream, int sel_splits, Shape* sh, dkv::DecodeArgs* a) {
  dkv_status st = check_layout(layout, sh);
  if (st != DKV_OK) return st;
  if (!in) return DKV_ERR_NULL;
  if ((st = check_cache(cache, *sh)) != DKV_OK) return st;
  if (!in->q || !in->w_up_k || !in->w_up_v || !in->out) return DKV_ERR_NULL;
  if (!aligned16(in->q) || !aligned16(in->w_up_k) || !aligned16(in->w_up_v) || !aligned16(in->out))
    return DKV_ERR_ALIGN;
  if (in->reserved != 0) return DKV_ERR_SHAPE;
  if (in->n_q_heads == 0 || in->n_q_heads % sh->H != 0) return DKV_ERR_SHAPE;
  if (in->n_q_heads / sh->H > 16) return DKV_ERR_UNSUPPORTED;
  if (in->n_splits > 1024) return DKV_ERR_UNSUPPORTED;
  if (in->w_head_stride < 0) return DKV_ERR_SHAPE;
  if (in->w_head_stride % 8) return DKV_ERR_ALIGN;
  if (in->w_head_stride != 0 && in->w_head_stride < (int64_t)sh->d * sh->dc) return DKV_ERR_SHAPE;
  if (!(in->softmax_scale >= 0.f) || isinf(in->softmax_scale)) return DKV_ERR_SHAPE;
  const int G = (int)(in->n_q_heads / sh->H);
  const int splits = in->n_splits ? (int)in->n_splits : sel_splits > 0 ? sel_splits : (int)auto_splits(*sh, G);
  const size_t need = dkv::decode_ws_bytes(*sh, G, splits);
  if (!ws || ws_bytes < need) return DKV_ERR_WORKSPACE;
  if (!aligned16(ws)) return DKV_ERR_ALIGN;

  a->q = in->q;
  a->wuk = in->w_up_k;
  a->wuv = in->w_up_v;
  a->w_hs = in->w_head_stride;
  a->G = G;
  a->Hq = (int)in->n_q_heads;
  a->splits = splits;
  a->scale = in->softmax_scale > 0.f ? in->softmax_scale : 1.0f / sqrtf((float)sh->d);
  a->out = in->out;
  a->refs = cache->refs;
  a->codes = cache->codes;
  a->idx = cache->idx;
  a->mu = cache->mu;
  a->scales = sh->q4 ? cache->scales : nullptr;
  a->score = (float*)ws;
  a->qp = (float*)((char*)ws + dkv::ws_qp_off(*sh, G));
  a->part = (float*)((char*)ws + dkv::ws_part_off(*sh, G));
  a->events = in->stage_events;
  a->sel = nullptr;
  a->n_sel = 0;
  return check_events(a->events, stream);
}

// Automatic split count of a selective decode: the full decode's count,
// lowered to keep at least 256 list entries per split (so a workspace sized
// for deltakv_decode_attn always suffices).
uint32_t sel_auto_splits(const Shape& sh, int G, uint32_t n_sel) {
  const uint32_t full = auto_splits(sh, G);
  const uint32_t by_len = (n_sel + 255) / 256;
  const uint32_t s = by_len < full ? by_len : full;
  return s < 1 ? 1 : s;
}

}  // namespace

extern "C" {

dkv_status deltakv_decode_attn(const dkv_layout* layout, const dkv_cache* cache, const dkv_decode_in* in, void* ws,
                               size_t ws_bytes, void* stream) {
  Shape sh;
  dkv::DecodeArgs a;
  const dkv_status st = decode_setup(layout, cache, in, ws, ws_bytes, stream, 0, &sh, &a);
  if (st != DKV_OK) return st;
  return from_hip(dkv::launch_decode(sh, a, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Workspace of deltakv_decode_attn_noalloc: one array per GPU, part of the
// library's device code, so it exists on every GPU the library runs on from
// the time the code is loaded there until the process ends.  Host code uses
// its device address from hipGetSymbolAddress (kept per device below), never
// the array's name, which on the host is only a stand-in.  The decode
// kernels write every byte they read in a call (scores, projected queries,
// split records), so nothing in it has to start at zero.
static __device__ __align__(256) unsigned char scratch[DKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];   // device address of `scratch` on each device, once looked up

// The current device's scratch address: looked up on the device's first
// call (with that device current), then reused.
dkv_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DKV_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DKV_ERR_DEVICE;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return DKV_OK;
}

}  // namespace

extern "C" {

dkv_status deltakv_decode_attn_noalloc(const dkv_layout* layout, const dkv_cache* cache, const dkv_decode_in* in,
                                       void* stream) {
  // The shape's workspace must fit the scratch array; checked before the
  // device is touched.
  Shape sh;
  dkv_status st = check_layout(layout, &sh);
  if (st != DKV_OK) return st;
  if (!in) return DKV_ERR_NULL;
  if (in->n_q_heads == 0 || in->n_q_heads % sh.H != 0) return DKV_ERR_SHAPE;
  if (in->n_q_heads / sh.H > 16) return DKV_ERR_UNSUPPORTED;
  if (in->n_splits > 1024) return DKV_ERR_UNSUPPORTED;
  const int G = (int)(in->n_q_heads / sh.H);
  const int splits = in->n_splits ? (int)in->n_splits : (int)auto_splits(sh, G);
  if (dkv::decode_ws_bytes(sh, G, splits) > (size_t)DKV_NOALLOC_SCRATCH_BYTES) return DKV_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != DKV_OK) return st;
  dkv::DecodeArgs a;
  st = decode_setup(layout, cache, in, ws, (size_t)DKV_NOALLOC_SCRATCH_BYTES, stream, 0, &sh, &a);
  if (st != DKV_OK) return st;
  return from_hip(dkv::launch_decode(sh, a, (hipStream_t)stream));
}

uint32_t dkv_decode_sel_auto_splits(const dkv_layout* layout, uint32_t n_q_heads, uint32_t n_sel) {
  Shape sh;
  if (check_layout(layout, &sh) != DKV_OK) return 0;
  if (n_q_heads == 0 || n_q_heads % sh.H != 0 || n_q_heads / sh.H > 16 || n_sel == 0) return 0;
  return sel_auto_splits(sh, (int)(n_q_heads / sh.H), n_sel);
}

dkv_status deltakv_decode_attn_sel(const dkv_layout* layout, const dkv_cache* cache, const dkv_decode_in* in,
                                   const dkv_token_sel* sel, void* ws, size_t ws_bytes, void* stream) {
  if (!sel) return DKV_ERR_NULL;
  if (!sel->tokens) return DKV_ERR_NULL;
  if (sel->n_sel == 0 || sel->n_sel > (1u << 30) || sel->reserved != 0) return DKV_ERR_SHAPE;
  if ((uintptr_t)sel->tokens % 4) return DKV_ERR_ALIGN;
  Shape sh;
  const dkv_status lst = check_layout(layout, &sh);
  if (lst != DKV_OK) return lst;
  if (sh.grouped) return DKV_ERR_UNSUPPORTED;
  const int G = in && in->n_q_heads && in->n_q_heads % sh.H == 0 ? (int)(in->n_q_heads / sh.H) : 1;
  dkv::DecodeArgs a;
  const dkv_status st =
      decode_setup(layout, cache, in, ws, ws_bytes, stream, (int)sel_auto_splits(sh, G, sel->n_sel), &sh, &a);
  if (st != DKV_OK) return st;
  a.sel = sel->tokens;
  a.n_sel = (int)sel->n_sel;
  return from_hip(dkv::launch_decode_sel(sh, a, (hipStream_t)stream));
}

}  // extern "C"
