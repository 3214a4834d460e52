// DeltaKV decode-time append: the token at position t of every stream joins
// a cache that holds positions 0 .. t-1, with the shared component frozen
// (DeltaKV explainer, English page, Technical Summary §3 "Strided Reference
// Selection": references are kept at a fixed stride and each new token
// retrieves the nearest earlier ones; §3 "Residual Encoding").  The result
// is the row that compressing all t + 1 tokens with the same mean would
// store:
//
//   t mod s == 0   refs[t / s] = rnd(k_t - mu)
//   otherwise      ref(t) = argmax over r with r*s < t of cos(x~_t, refs[r]),
//                  lowest r on ties;  code_t = rnd(W_down ((k_t - mu) - refs[ref(t)]))
//
// One 256-thread block per stream: 16 groups of 16 lanes walk the references
// (group g takes r = g, g + 16, ...; a lane holds d/16 elements of the row),
// each group keeps its best (score, ordinal) with a strict '>' over
// increasing ordinals, and the groups merge in a fixed order.  Scores are
// <x~_t, x~_r> / ||x~_r||, as in the compress search.

#include "dkv_device.h"
#include "dkv_internal.h"

namespace dkv {

namespace {

template <class S, int D>
__global__ __launch_bounds__(256) void k_append(AppendArgs a, Shape sh) {
  constexpr int E = D / 16;   // elements per lane
  __shared__ float xs[D];     // x~_t
  __shared__ float ds[D];     // k_t - mu
  __shared__ float red_s[16];
  __shared__ int red_r[16];
  const int stream = blockIdx.x;
  const int kv = stream & 1, bh = stream >> 1, b = bh / sh.H, h = bh % sh.H;
  const int t = sh.T - 1;     // the new token's position
  const int tid = threadIdx.x;
  const typename S::T* src = (const typename S::T*)(kv ? a.v : a.k) + (int64_t)b * a.sb + (int64_t)h * a.sh;
  const typename S::T* mu = (const typename S::T*)a.mu + (size_t)stream * D;
  typename S::T* refs = (typename S::T*)a.refs + (size_t)stream * sh.Rc * D;
  if (tid < D) {
    const float x = S::load(src[tid]), m = S::load(mu[tid]);
    const typename S::T xt = S::sub_rn(x, m);
    xs[tid] = S::load(xt);
    ds[tid] = x - m;
    if (t % sh.s == 0) refs[(size_t)(t / sh.s) * D + tid] = xt;
  }
  if (t % sh.s == 0) return;  // a reference token stores no code
  __syncthreads();

  // ---- search over references r = 0 .. t / s ----
  const int grp = tid >> 4, l16 = tid & 15;
  const int nref = t / sh.s + 1;
  float x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = xs[l16 * E + e];
  float best = -INFINITY;
  int bidx = 0;
  for (int r = grp; r < nref; r += 16) {
    const typename S::T* row = refs + (size_t)r * D + l16 * E;
    float dot = 0.f, n2 = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float v = S::load(row[e]);
      dot = fmaf(x[e], v, dot);
      n2 = fmaf(v, v, n2);
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) {
      dot += __shfl_xor(dot, o, 64);
      n2 += __shfl_xor(n2, o, 64);
    }
    const float sc = n2 > 0.f ? dot * (1.0f / sqrtf(n2)) : 0.f;
    if (sc > best) {
      best = sc;
      bidx = r;
    }
  }
  if (l16 == 0) {
    red_s[grp] = best;
    red_r[grp] = bidx;
  }
  __syncthreads();
  // Fixed-order merge: larger score, then lower ordinal.
  float bs = red_s[0];
  int br = red_r[0];
  for (int g = 1; g < 16; ++g) {
    const float v = red_s[g];
    const int r = red_r[g];
    if (v > bs || (v == bs && r < br)) {
      bs = v;
      br = r;
    }
  }

  // ---- code: rnd(W_down ((k - mu) - refs[br])) ----
  const size_t slot = (size_t)stream * sh.Nc + (size_t)(t - t / sh.s - 1);
  if (tid < sh.dc) {
    const typename S::T* w = (const typename S::T*)(kv ? a.wdv : a.wdk) + (size_t)h * a.w_hs + (size_t)tid * D;
    const typename S::T* rrow = refs + (size_t)br * D;
    float c = 0.f;
    for (int e = 0; e < D; ++e) c = fmaf(S::load(w[e]), ds[e] - S::load(rrow[e]), c);
    ((typename S::T*)a.codes)[slot * sh.dc + tid] = S::from_f32(c);
  }
  if (tid == 0) store_idx(a.idx, slot, sh.idx_bytes, (uint32_t)br);
}

template <class S>
hipError_t launch_append_s(const Shape& sh, const AppendArgs& a, hipStream_t st) {
  const dim3 grid(sh.n_streams());
  return sh.d == 128 ? launch(k_append<S, 128>, grid, 256, st, nullptr, nullptr, a, sh)
                     : launch(k_append<S, 64>, grid, 256, st, nullptr, nullptr, a, sh);
}

}  // namespace

hipError_t launch_append(const Shape& sh, const AppendArgs& a, hipStream_t st) {
  return sh.bf16 ? launch_append_s<BF16>(sh, a, st) : launch_append_s<F32>(sh, a, st);
}

}  // namespace dkv
