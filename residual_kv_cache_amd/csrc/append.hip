// DeltaKV decode-time append: the token at position t of every stream joins
// a cache that holds positions 0 .. t-1, with the shared component frozen
// (DeltaKV explainer, English page, Technical Summary §3 "Strided Reference
// Selection": references are kept at a fixed stride and each new token
// retrieves the nearest earlier one; §3 "Residual Encoding").  The result is
// the row that compressing all t + 1 tokens with the same mean would store:
//
//   t mod s == 0   refs[t / s] = rnd(k_t - mu)
//   otherwise      ref(t) = argmax over r with r*s < t of cos(x~_t, refs[r]),
//                  lowest r on ties;  code_t = rnd(W_down ((k_t - mu) - refs[ref(t)]))
//
// The search is one pass over the stream's references, which is HBM-bound,
// so it is spread over many blocks per stream (k_append_search): block p of
// a stream scores references [p*chunk, (p+1)*chunk) with 16-lane groups, one
// reference row per group and one 16-byte load per lane, four rows in flight
// per group, and writes its best (score, ordinal) together with that
// candidate's code, encoded in the same block while the row is at hand.
// k_append_finish takes the maximum of the candidates under the total order
// (higher score, then lower ordinal) -- unique, so independent of the merge
// tree -- and copies its code and ordinal into the cache.  Scores are
// <x~_t, x~_r> / ||x~_r||, which orders the references as the cosine does
// (||x~_t|| is common to all of them).

#include <algorithm>

#include "dkv_device.h"
#include "dkv_internal.h"

namespace dkv {

namespace {

typedef const __attribute__((address_space(1))) uint32_t* GWords;

// E consecutive storage elements as raw 32-bit words.
template <class S, int E>
struct RowSlice {
  static constexpr int kWords = E * (int)sizeof(typename S::T) / 4;
  uint32_t w[kWords];
  __device__ __forceinline__ void load(const void* p) {
    GWords g = (GWords)p;
    if constexpr (kWords % 4 == 0) {
#pragma unroll
      for (int i = 0; i < kWords; i += 4) {
        const u32x4 v = *(const __attribute__((address_space(1))) u32x4*)(g + i);
        w[i] = v.x;
        w[i + 1] = v.y;
        w[i + 2] = v.z;
        w[i + 3] = v.w;
      }
    } else {
      const u32x2 v = *(const __attribute__((address_space(1))) u32x2*)g;
      w[0] = v.x;
      w[1] = v.y;
    }
  }
  // Element e as float.
  __device__ __forceinline__ float at(int e) const {
    if constexpr (sizeof(typename S::T) == 2)
      return __uint_as_float((e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16));
    else
      return __uint_as_float(w[e]);
  }
};

__device__ __forceinline__ bool better(float s1, int r1, float s2, int r2) {
  return (s1 > s2) | ((s1 == s2) & (r1 < r2));   // bitwise: no divergent branches
}

constexpr int kUnroll = 4;

// Search partials in the workspace: (score, ordinal) per block, then the
// block's winner already encoded, [n_streams][parts][d_c] storage dtype.
inline size_t pcode_off(int ns, int parts) { return align_up((size_t)ns * parts * sizeof(float2), 256); }

template <class S, int D>
__global__ __launch_bounds__(256) void k_append_search(AppendArgs a, Shape sh, int chunk, int P, float2* part,
                                                       void* pcode) {
  constexpr int E = D / 16;  // elements per lane of a reference row
  constexpr int Q = D / 4;   // elements per lane of a W_down row
  typedef typename S::T T;
  const XcdItem xi = xcd_item(sh.n_streams());  // a stream's blocks share its XCD
  if (xi.stream < 0) return;
  const int stream = xi.stream, p = xi.item;
  const int kv = stream & 1, bh = stream >> 1, b = bh / sh.H, h = bh - b * sh.H;
  const int t = sh.T - 1;
  const int nref = t / sh.s + 1;  // references r with r*s < t (t is not a multiple of s)
  const int r0 = p * chunk, r1 = min(nref, r0 + chunk);
  const int tid = threadIdx.x, grp = tid >> 4, l16 = tid & 15;
  const int j = tid >> 2, l4 = tid & 3;
  constexpr size_t e = sizeof(T);

  // Every load that does not depend on another goes out first: the first
  // reference rows, the new token and the mean, this lane's W_down slice.
  const char* refs = (const char*)a.refs + ((size_t)stream * sh.Rc * D + l16 * E) * e;
  RowSlice<S, E> row[kUnroll];
  int r = r0 + grp;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) row[u].load(refs + (size_t)min(r + 16 * u, r1 - 1) * D * e);
  const char* src = (const char*)(kv ? a.v : a.k) + ((int64_t)b * a.sb + (int64_t)h * a.sh + l16 * E) * e;
  RowSlice<S, E> ks, ms;
  ks.load(src);
  ms.load((const char*)a.mu + ((size_t)stream * D + l16 * E) * e);
  const T* wd = (const T*)(kv ? a.wdv : a.wdk) + (size_t)h * a.w_hs;
  RowSlice<S, Q> wrow;  // rows past d_c load row d_c - 1 (unconditional loads keep the wait counts exact)
  wrow.load(wd + (size_t)min(j, sh.dc - 1) * D + l4 * Q);

  float x[E], ds[E];  // x~_t = rnd(k_t - mu) and k_t - mu
#pragma unroll
  for (int i = 0; i < E; ++i) {
    ds[i] = ks.at(i) - ms.at(i);
    x[i] = S::load(S::sub_rn(ks.at(i), ms.at(i)));
  }

  float best = -INFINITY;
  int bidx = 0x7FFFFFFF;
  RowSlice<S, E> brow = row[0];  // the group's best row so far
  for (;;) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float dot = 0.f, n2 = 0.f;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const float v = row[u].at(i);
        dot = fmaf(x[i], v, dot);
        n2 = fmaf(v, v, n2);
      }
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) {
        dot += __shfl_xor(dot, o, 64);
        n2 += __shfl_xor(n2, o, 64);
      }
      const float sc = n2 > 0.f ? dot * (1.0f / sqrtf(n2)) : 0.f;
      const int ru = r + 16 * u;
      if (ru < r1 && sc > best) {  // ordinals rise within a group: '>' keeps the lowest on ties
        best = sc;
        bidx = ru;
        brow = row[u];
      }
    }
    r += 16 * kUnroll;
    if (r >= r1) break;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) row[u].load(refs + (size_t)min(r + 16 * u, r1 - 1) * D * e);
  }

  __shared__ float red_s[16];
  __shared__ int red_r[16];
  __shared__ float diff[D];
  if (l16 == 0) {
    red_s[grp] = best;
    red_r[grp] = bidx;
  }
  __syncthreads();
  float bs = red_s[0];
  int br = red_r[0];
  for (int g = 1; g < 16; ++g)
    if (better(red_s[g], red_r[g], bs, br)) {
      bs = red_s[g];
      br = red_r[g];
    }
  // Ordinal br was scored by group (br - r0) mod 16, which holds its row.
  if (grp == ((br - r0) & 15)) {
#pragma unroll
    for (int i = 0; i < E; ++i) diff[l16 * E + i] = ds[i] - brow.at(i);
  }
  __syncthreads();

  // The block's candidate code: rnd(W_down (k_t - mu - refs[br])) (for
  // 4-bit codes the unrounded value, quantized once the winner is known),
  // four lanes per element, 64 elements per pass.
  T* out = (T*)pcode + ((size_t)stream * P + p) * sh.dc;
  float* out32 = (float*)pcode + ((size_t)stream * P + p) * sh.dc;
  for (int j0 = 0; j0 < sh.dc; j0 += 64) {
    const int jj = j0 + j;
    if (j0 > 0) wrow.load(wd + (size_t)min(jj, sh.dc - 1) * D + l4 * Q);
    float c = 0.f;
    if (jj < sh.dc) {
#pragma unroll
      for (int i = 0; i < Q; ++i) c = fmaf(wrow.at(i), diff[l4 * Q + i], c);
    }
    c += __shfl_xor(c, 1, 64);
    c += __shfl_xor(c, 2, 64);
    if (jj < sh.dc && l4 == 0) {
      if (sh.q4)
        out32[jj] = c;
      else
        out[jj] = S::from_f32(c);
    }
  }
  if (tid == 0) part[(size_t)stream * P + p] = make_float2(bs, __int_as_float(br));
}

// One wave per stream (block x runs on XCD x mod 8, beside the stream's
// search blocks): the maximum of the search partials under the total order,
// then its code and ordinal are stored; or, for a token at a reference
// position, its centred row.
template <class S, int D>
__global__ __launch_bounds__(64) void k_append_finish(AppendArgs a, Shape sh, int P, const float2* part,
                                                      const void* pcode) {
  typedef typename S::T T;
  const int stream = blockIdx.x;
  const int kv = stream & 1, bh = stream >> 1, b = bh / sh.H, h = bh - b * sh.H;
  const int t = sh.T - 1;
  const int lane = threadIdx.x;
  if (t % sh.s == 0) {
    // The token's centred row becomes a reference (both elements of a lane
    // loaded before either is stored).
    const T* src = (const T*)(kv ? a.v : a.k) + (int64_t)b * a.sb + (int64_t)h * a.sh;
    const T* mu = (const T*)a.mu + (size_t)stream * D;
    T* row = (T*)a.refs + ((size_t)stream * sh.Rc + t / sh.s) * D;
    constexpr int PER = D / 64;
    T x[PER], m[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      x[j] = src[lane + 64 * j];
      m[j] = mu[lane + 64 * j];
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) row[lane + 64 * j] = S::sub_rn(S::load(x[j]), S::load(m[j]));
    return;
  }
  // Merge the blocks' candidates.  A lane loads up to kMergeLoads of them at
  // once (clamped addresses; duplicates of the last one cannot change the
  // maximum), then compares; larger P loops.
  constexpr int kMergeLoads = 4;
  float bs = -INFINITY;
  int br = 0x7FFFFFFF, bp = 0;
  const float2* pp = part + (size_t)stream * P;
  for (int i0 = 0; i0 < P; i0 += 64 * kMergeLoads) {
    float2 v[kMergeLoads];
#pragma unroll
    for (int u = 0; u < kMergeLoads; ++u) v[u] = pp[min(i0 + lane + 64 * u, P - 1)];
#pragma unroll
    for (int u = 0; u < kMergeLoads; ++u) {
      const int i = min(i0 + lane + 64 * u, P - 1);
      if (better(v[u].x, __float_as_int(v[u].y), bs, br)) {
        bs = v[u].x;
        br = __float_as_int(v[u].y);
        bp = i;
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float os = __shfl_xor(bs, o, 64);
    const int orr = __shfl_xor(br, o, 64);
    const int op = __shfl_xor(bp, o, 64);
    if (better(os, orr, bs, br)) {
      bs = os;
      br = orr;
      bp = op;
    }
  }
  const size_t slot = (size_t)stream * sh.Nc + (size_t)(t - t / sh.s - 1);
  if (!sh.q4) {
    const T* c = (const T*)pcode + ((size_t)stream * P + bp) * sh.dc;
    for (int jj = lane; jj < sh.dc; jj += 64) ((T*)a.codes)[slot * sh.dc + jj] = c[jj];
  } else {
    // 4-bit codes: the row's scale from its largest magnitude, then each
    // even lane packs its element with its neighbour's (d_c <= 128).
    const float* c = (const float*)pcode + ((size_t)stream * P + bp) * sh.dc;
    // Both loads unconditional (clamped), masked after: one round trip.
    const float l0 = c[min(lane, sh.dc - 1)], l1 = c[min(lane + 64, sh.dc - 1)];
    const float c0 = lane < sh.dc ? l0 : 0.f, c1 = lane + 64 < sh.dc ? l1 : 0.f;
    const float amax = wave_max(fmaxf(fabsf(c0), fabsf(c1)));
    const T sbits = S::from_f32(amax / 7.0f);
    const float scale = S::load(sbits);
    const int q0 = q4_quant(c0, scale), q1 = q4_quant(c1, scale);
    const int n0 = __shfl_down(q0, 1, 64), n1 = __shfl_down(q1, 1, 64);
    uint8_t* row = (uint8_t*)a.codes + slot * (sh.dc / 2);
    if (!(lane & 1)) {
      if (lane < sh.dc) row[lane >> 1] = (uint8_t)(((uint32_t)q0 & 15u) | (((uint32_t)n0 & 15u) << 4));
      if (lane + 64 < sh.dc) row[(lane + 64) >> 1] = (uint8_t)(((uint32_t)q1 & 15u) | (((uint32_t)n1 & 15u) << 4));
    }
    if (lane == 0) ((T*)a.scales)[slot] = sbits;
  }
  if (lane == 0) store_idx(a.idx, slot, sh.idx_bytes, (uint32_t)br);
}

// ---------------------------------------------------------------------------
// k references or the L2 metric: the search blocks keep the best k of their
// chunk (per 16-lane group, then merged in the block), and one 256-thread
// block per stream merges the blocks' lists, averages the kept references
// and encodes against the mean.
// ---------------------------------------------------------------------------

template <class S, int D, int KT, bool KFULL>
__global__ __launch_bounds__(256) void k_append_search_topk(AppendArgs a, Shape sh, int chunk, int P, float2* part) {
  constexpr int E = D / 16;
  const XcdItem xi = xcd_item(sh.n_streams());
  if (xi.stream < 0) return;
  const int stream = xi.stream, p = xi.item;
  const int kv = stream & 1, bh = stream >> 1, b = bh / sh.H, h = bh - b * sh.H;
  const int t = sh.T - 1;
  const int nref = t / sh.s + 1;
  const int r0 = p * chunk, r1 = min(nref, r0 + chunk);
  const int tid = threadIdx.x, grp = tid >> 4, l16 = tid & 15;
  const int K = KFULL ? KT : sh.K;   // k equal to the list length: a compile-time constant
  constexpr size_t e = sizeof(typename S::T);
  const char* refs = (const char*)a.refs + ((size_t)stream * sh.Rc * D + l16 * E) * e;
  RowSlice<S, E> row[kUnroll];
  int r = r0 + grp;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) row[u].load(refs + (size_t)min(r + 16 * u, r1 - 1) * D * e);
  const char* src = (const char*)(kv ? a.v : a.k) + ((int64_t)b * a.sb + (int64_t)h * a.sh + l16 * E) * e;
  RowSlice<S, E> ks, ms;
  ks.load(src);
  ms.load((const char*)a.mu + ((size_t)stream * D + l16 * E) * e);
  float x[E];
#pragma unroll
  for (int i = 0; i < E; ++i) x[i] = S::load(S::sub_rn(ks.at(i), ms.at(i)));

  TopKN<KT> top;
  top.init();
  for (;;) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float dot = 0.f, n2 = 0.f;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const float v = row[u].at(i);
        dot = fmaf(x[i], v, dot);
        n2 = fmaf(v, v, n2);
      }
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) {
        dot += __shfl_xor(dot, o, 64);
        n2 += __shfl_xor(n2, o, 64);
      }
      const float sc = sh.l2 ? 2.f * dot - n2 : (n2 > 0.f ? dot * (1.0f / sqrtf(n2)) : 0.f);
      const int ru = r + 16 * u;
      if (ru < r1) top.insert(sc, ru, K);   // the group's lanes hold the same list
    }
    r += 16 * kUnroll;
    if (r >= r1) break;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) row[u].load(refs + (size_t)min(r + 16 * u, r1 - 1) * D * e);
  }
  __shared__ float red_s[16][KT];
  __shared__ int red_r[16][KT];
  if (l16 == 0) {
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      red_s[grp][j] = top.s[j];
      red_r[grp][j] = top.r[j];
    }
  }
  __syncthreads();
  if (tid == 0) {
    TopKN<KT> all;
    all.init();
    for (int g = 0; g < 16; ++g)
      for (int j = 0; j < K; ++j) all.insert(red_s[g][j], red_r[g][j], K);
    float2* out = part + ((size_t)stream * P + p) * K;
#pragma unroll
    for (int j = 0; j < KT; ++j)
      if (j < K) out[j] = make_float2(all.s[j], __int_as_float(all.r[j]));
  }
}

template <class S, int D, int KT, bool KFULL>
__global__ __launch_bounds__(256) void k_append_finish_topk(AppendArgs a, Shape sh, int P, const float2* part) {
  typedef typename S::T T;
  const int stream = blockIdx.x;
  const int kv = stream & 1, bh = stream >> 1, b = bh / sh.H, h = bh - b * sh.H;
  const int t = sh.T - 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int K = KFULL ? KT : sh.K;
  const T* src = (const T*)(kv ? a.v : a.k) + (int64_t)b * a.sb + (int64_t)h * a.sh;
  const T* mu = (const T*)a.mu + (size_t)stream * D;
  T* refs = (T*)a.refs + (size_t)stream * sh.Rc * D;
  if (t % sh.s == 0) {
    if (tid < D) refs[(size_t)(t / sh.s) * D + tid] = S::sub_rn(S::load(src[tid]), S::load(mu[tid]));
    return;
  }
  __shared__ int s_ord[KT];
  __shared__ float diff[D];
  __shared__ float red[8];
  const int cnt = min(K, t / sh.s + 1);
  if (tid < 64) {
    TopKN<KT> top;
    top.init();
    // Up to 8 list entries per lane in flight at once (clamped; a repeated
    // entry is masked out), then inserted.
    const float2* pp = part + (size_t)stream * P * K;
    const int n = P * K;
    for (int i0 = 0; i0 < n; i0 += 64 * 8) {
      float2 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = pp[min(i0 + lane + 64 * u, n - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + lane + 64 * u < n) top.insert(v[u].x, __float_as_int(v[u].y), K);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) top.merge_xor(o, K);
    if (lane == 0) {
      int o[KT];
      top.sorted_ordinals(cnt, o);
#pragma unroll
      for (int j = 0; j < KT; ++j) s_ord[j] = o[j];
    }
  }
  __syncthreads();
  if (tid < D) {
    // Every kept reference row loaded at once (slots past the count read a
    // valid row and are masked), summed in slot order.
    T rv[KT];
#pragma unroll
    for (int j = 0; j < KT; ++j) rv[j] = refs[(size_t)min(s_ord[min(j, cnt - 1)], sh.R - 1) * D + tid];
    const T xk = src[tid], xm = mu[tid];
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < KT; ++j) m += j < cnt ? S::load(rv[j]) : 0.f;
    m = cnt > 1 ? m * (1.0f / (float)cnt) : m;
    diff[tid] = (S::load(xk) - S::load(xm)) - m;
  }
  __syncthreads();
  const size_t slot = (size_t)stream * sh.Nc + (size_t)(t - t / sh.s - 1);
  const T* w = (const T*)(kv ? a.wdv : a.wdk) + (size_t)h * a.w_hs;
  constexpr int Q = D / 4;
  const int l4 = tid & 3;
  // Code element j = j0 + tid / 4 from four lanes' partial dot products.
  float cv[2] = {0.f, 0.f};   // this lane's elements of the two 64-element passes (d_c <= 128)
  for (int pass = 0; pass * 64 < sh.dc; ++pass) {
    const int jj = pass * 64 + (tid >> 2);
    float c = 0.f;
    if (jj < sh.dc) {
      const T* wr = w + (size_t)jj * D + l4 * Q;
#pragma unroll 8
      for (int i = 0; i < Q; ++i) c = fmaf(S::load(wr[i]), diff[l4 * Q + i], c);
    }
    c += __shfl_xor(c, 1, 64);
    c += __shfl_xor(c, 2, 64);
    cv[pass] = c;
    if (!sh.q4 && jj < sh.dc && l4 == 0) ((T*)a.codes)[slot * sh.dc + jj] = S::from_f32(c);
  }
  if (sh.q4) {
    float am = fmaxf(fabsf(cv[0]), fabsf(cv[1]));
    am = wave_max(am);
    if (lane == 0) red[tid >> 6] = am;
    __syncthreads();
    const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const T sbits = S::from_f32(amax / 7.0f);
    const float scale = S::load(sbits);
    uint8_t* row = (uint8_t*)a.codes + slot * (sh.dc / 2);
    for (int pass = 0; pass * 64 < sh.dc; ++pass) {
      const int jj = pass * 64 + (tid >> 2);
      const int q = q4_quant(cv[pass], scale);
      const int qn = __shfl_down(q, 4, 64);   // element jj + 1 sits four lanes up
      if (l4 == 0 && !(jj & 1) && jj < sh.dc)
        row[jj >> 1] = (uint8_t)(((uint32_t)q & 15u) | (((uint32_t)qn & 15u) << 4));
    }
    if (tid == 0) ((T*)a.scales)[slot] = sbits;
  }
  if (tid < K) store_idx(a.idx, slot * K + tid, sh.idx_bytes, (uint32_t)s_ord[tid]);
}

__global__ void k_append_empty() {}

template <class S, int D>
hipError_t launch_append_sd(const Shape& sh, const AppendArgs& a, void* ws, hipStream_t st) {
  const hipEvent_t ev[4] = {ev_start(a.events, 0), ev_stop(a.events, 0), ev_start(a.events, 1),
                            ev_stop(a.events, 1)};
  const int t = sh.T - 1, ns = sh.n_streams();
  const int P = t % sh.s == 0 ? 0 : append_parts(sh, t / sh.s + 1);
  if (sh.topk_search()) {
    float2* part = (float2*)ws;
    hipError_t err;
    // Lists of 4 or 8; k equal to the list length is a compile-time constant.
    auto search = sh.K == 4   ? k_append_search_topk<S, D, 4, true>
                  : sh.K < 4  ? k_append_search_topk<S, D, 4, false>
                  : sh.K == 8 ? k_append_search_topk<S, D, 8, true>
                              : k_append_search_topk<S, D, 8, false>;
    auto finish = sh.K == 4   ? k_append_finish_topk<S, D, 4, true>
                  : sh.K < 4  ? k_append_finish_topk<S, D, 4, false>
                  : sh.K == 8 ? k_append_finish_topk<S, D, 8, true>
                              : k_append_finish_topk<S, D, 8, false>;
    if (P > 0)
      err = launch(search, dim3(xcd_grid(ns, P)), 256, st, ev[0], ev[1], a, sh, append_chunk(sh, t / sh.s + 1), P,
                   part);
    else
      err = ev[0] ? launch(k_append_empty, dim3(1), 64, st, ev[0], ev[1]) : hipSuccess;
    if (err != hipSuccess) return err;
    return launch(finish, dim3(ns), 256, st, ev[2], ev[3], a, sh, P, (const float2*)part);
  }
  float2* part = (float2*)ws;
  void* pcode = (char*)ws + pcode_off(ns, std::max(P, 1));
  hipError_t err;
  if (P > 0)
    err = launch(k_append_search<S, D>, dim3(xcd_grid(ns, P)), 256, st, ev[0], ev[1], a, sh,
                 append_chunk(sh, t / sh.s + 1), P, part, pcode);
  else  // a reference token needs no search: an empty stage keeps the event pairs meaningful
    err = ev[0] ? launch(k_append_empty, dim3(1), 64, st, ev[0], ev[1]) : hipSuccess;
  if (err != hipSuccess) return err;
  return launch(k_append_finish<S, D>, dim3(ns), 64, st, ev[2], ev[3], a, sh, P, (const float2*)part,
                (const void*)pcode);
}

}  // namespace

int append_chunk(const Shape& sh, int nref) {
  const int target = (kAppendBlocks + sh.n_streams() - 1) / sh.n_streams();
  const int per = (nref + target - 1) / target;
  return std::max(kAppendMinChunk, (per + kAppendMinChunk - 1) / kAppendMinChunk * kAppendMinChunk);
}

int append_parts(const Shape& sh, int nref) { return (nref + append_chunk(sh, nref) - 1) / append_chunk(sh, nref); }

size_t append_ws_bytes(const Shape& sh) {
  // Bound on the part count at any length the capacity allows: a chunk is
  // at least kAppendMinChunk references and at least nref / target, so
  // parts <= min(target, ceil(Rc / kAppendMinChunk)).  The code partials
  // are laid out with the actual count, which never exceeds the bound.
  const int ns = sh.n_streams();
  const int target = (kAppendBlocks + ns - 1) / ns;
  const int most = std::max(1, std::min(target, (sh.Rc + kAppendMinChunk - 1) / kAppendMinChunk));
  const size_t code_bytes = sh.q4 ? sizeof(float) : (size_t)sh.elem();   // 4-bit: unrounded candidates
  const size_t one = align_up(pcode_off(ns, most) + (size_t)ns * most * sh.dc * code_bytes, 256);
  const size_t lists = align_up((size_t)ns * most * sh.K * sizeof(float2), 256);   // k references / L2
  return sh.topk_search() ? lists : one;
}

hipError_t launch_append(const Shape& sh, const AppendArgs& a, void* ws, hipStream_t st) {
  if (sh.bf16)
    return sh.d == 128 ? launch_append_sd<BF16, 128>(sh, a, ws, st) : launch_append_sd<BF16, 64>(sh, a, ws, st);
  return sh.d == 128 ? launch_append_sd<F32, 128>(sh, a, ws, st) : launch_append_sd<F32, 64>(sh, a, ws, st);
}

}  // namespace dkv
