// DeltaKV compression kernels for gfx950.
//
// One stream = one (sequence b, KV head h, tensor kv) with kv = 0 for K and
// 1 for V; stream id = (b * H + h) * 2 + kv.  Four steps per stream:
//
//   mean    mu = rnd(mean_t k_t), fp64 partial sums then a fixed-order fp64
//           total (the component all tokens share; DeltaKV explainer,
//           English page, Technical Summary §2 "Highly Shared Latent
//           Components")
//   center  refs[r] = rnd(k_{r*s} - mu) and 1/||refs[r]|| (English page §3
//           "Strided Reference Selection": references at a fixed stride)
//   search  ref(t) = argmax over earlier references of the cosine, lowest
//           ordinal on ties (same section: each token retrieves its most
//           similar references from the strided set)
//   encode  code_t = rnd(W_down ((k_t - mu) - refs[ref(t)])) (English page
//           §3 "Residual Encoding"; French page §2 "Architecture de
//           compression": projection to d_c dimensions)
//
// bfloat16 storage runs the search and the encode on MFMA: the centred
// tokens and references are exact bf16 values, so the bf16 x bf16 products
// are exact and only the fp32 accumulation rounds.  float32 storage runs
// plain fp32 VALU kernels.

#include "dkv_device.h"
#include "dkv_internal.h"

namespace dkv {

namespace {

// ---------------------------------------------------------------------------
// Loads of 8 consecutive storage elements (16-byte aligned) as floats.
// ---------------------------------------------------------------------------

// Eight packed bfloat16 values as floats.
__device__ __forceinline__ void unpack8(uint4 u, float* out) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ void load8(const uint16_t* p, float* out) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ void load8(const float* p, float* out) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pk_bf16_rn(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}


struct StreamId {
  int b, h, kv;
};

__device__ __forceinline__ StreamId decode_stream(int stream, int H) {
  StreamId id;
  id.kv = stream & 1;
  int bh = stream >> 1;
  id.b = bh / H;
  id.h = bh % H;
  return id;
}

template <class S>
__device__ __forceinline__ const typename S::T* stream_src(const CompressArgs& a, StreamId id) {
  const typename S::T* base = (const typename S::T*)(id.kv ? a.v : a.k);
  return base + id.b * a.sb + id.h * a.sh;
}

// ---------------------------------------------------------------------------
// Mean: stage 1, fp64 partial sums over kMeanChunk tokens.
// grid (chunks, streams), block 256: d/8 threads per token row, 16 bytes
// each; kMeanRows rows per thread in flight at once (clamped to the chunk's
// last row, the repeats adding nothing); the rows of a wave are summed by a
// fixed butterfly, then the four waves in order.
// ---------------------------------------------------------------------------

constexpr int kMeanRows = 2;

template <class S>
__global__ __launch_bounds__(256) void k_mean_partial(CompressArgs a, Shape sh) {
  __shared__ double red[4][128];
  const int stream = blockIdx.y;
  const StreamId id = decode_stream(stream, sh.H);
  const typename S::T* src = stream_src<S>(a, id);
  const int tpr = sh.d / 8;           // threads per token row
  const int rows = 256 / tpr;         // rows per pass
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = (tid % tpr) * 8;
  const int r0 = tid / tpr;
  const int t0 = blockIdx.x * kMeanChunk;
  const int t1 = min(sh.T, t0 + kMeanChunk);
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int t = t0 + r0; t < t1; t += kMeanRows * rows) {
    float x[kMeanRows][8];
#pragma unroll
    for (int u = 0; u < kMeanRows; ++u) load8(src + (int64_t)min(t + u * rows, t1 - 1) * a.st + c0, x[u]);
#pragma unroll
    for (int u = 0; u < kMeanRows; ++u) {
      const bool in = t + u * rows < t1;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += in ? (double)x[u][e] : 0.0;
    }
  }
  // Lanes tpr apart hold the same columns.
  for (int o = tpr; o < 64; o <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
  if (lane < tpr) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave][c0 + e] = acc[e];
  }
  __syncthreads();
  if (tid < sh.d)
    a.mean_part[((size_t)stream * gridDim.x + blockIdx.x) * sh.d + tid] =
        ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
}

// Mean: stage 2, fixed-order total, divide, round once.  grid streams,
// block 256: thread (g, i) sums chunks g, g + G, ... of column i
// (G = 256 / d groups, loads issued 8 at a time), then the G partial sums
// are added in group order.
template <class S>
__global__ __launch_bounds__(256) void k_mean_final(CompressArgs a, Shape sh, int chunks) {
  __shared__ double part[256];
  const int stream = blockIdx.x;
  const int i = threadIdx.x % sh.d, g = threadIdx.x / sh.d, G = 256 / sh.d;
  typename S::T* mu = (typename S::T*)a.mu;
  if (a.mu_in) {
    if (g == 0) mu[(size_t)stream * sh.d + i] = ((const typename S::T*)a.mu_in)[(size_t)stream * sh.d + i];
    return;
  }
  const double* src = a.mean_part + (size_t)stream * chunks * sh.d + i;
  double s = 0.0;
  int c = g;
  for (; c + 7 * G < chunks; c += 8 * G) {
    double v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = src[(size_t)(c + k * G) * sh.d];
#pragma unroll
    for (int k = 0; k < 8; ++k) s += v[k];
  }
  for (; c < chunks; c += G) s += src[(size_t)c * sh.d];
  part[threadIdx.x] = s;
  __syncthreads();
  if (g == 0) {
    double t = 0.0;
    for (int k = 0; k < G; ++k) t += part[k * sh.d + i];
    mu[(size_t)stream * sh.d + i] = S::from_f64(t / (double)sh.T);
  }
}

// ---------------------------------------------------------------------------
// Centred references and their inverse norms.  grid (ceil(R / (256 / (d/8))),
// streams), block 256: d/8 lanes per reference, eight elements per lane (one
// 16-byte load each of the row and of mu), the squared norm summed over the
// lane group by a fixed butterfly.
// ---------------------------------------------------------------------------

template <class S>
__global__ __launch_bounds__(256) void k_center_refs(CompressArgs a, Shape sh) {
  const int stream = blockIdx.y;
  const int lpr = sh.d / 8, rpb = 256 / lpr;   // lanes per reference, references per block
  const int l = threadIdx.x % lpr;
  const int r = blockIdx.x * rpb + threadIdx.x / lpr;
  if (r >= sh.R) return;
  const StreamId id = decode_stream(stream, sh.H);
  const typename S::T* src = stream_src<S>(a, id) + (int64_t)r * sh.s * a.st + l * 8;
  const typename S::T* mu = (const typename S::T*)a.mu + (size_t)stream * sh.d + l * 8;
  typename S::T* dst = (typename S::T*)a.refs + ((size_t)stream * sh.Rc + r) * sh.d + l * 8;
  float x[8], m[8];
  load8(src, x);
  load8(mu, m);
  typename S::T y[8];
  float n2 = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    y[i] = S::sub_rn(x[i], m[i]);
    const float f = S::load(y[i]);
    n2 = fmaf(f, f, n2);
  }
  if constexpr (sizeof(typename S::T) == 2) {
    uint4 o;
    o.x = (uint32_t)y[0] | ((uint32_t)y[1] << 16);
    o.y = (uint32_t)y[2] | ((uint32_t)y[3] << 16);
    o.z = (uint32_t)y[4] | ((uint32_t)y[5] << 16);
    o.w = (uint32_t)y[6] | ((uint32_t)y[7] << 16);
    *reinterpret_cast<uint4*>(dst) = o;
  } else {
    *reinterpret_cast<float4*>(dst) = make_float4(y[0], y[1], y[2], y[3]);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(y[4], y[5], y[6], y[7]);
  }
  // The lane group (lpr consecutive lanes of one wave) sums its parts.
  for (int o = 1; o < lpr; o <<= 1) n2 += __shfl_xor(n2, o, 64);
  // Norm term of the search: 1 / ||r|| (cosine; 0 for a zero reference) or
  // ||r||^2 (L2).
  if (l == 0) a.inv_n[(size_t)stream * sh.R + r] = sh.l2 ? n2 : n2 > 0.f ? 1.0f / sqrtf(n2) : 0.0f;
}

// ---------------------------------------------------------------------------
// Reference search, bfloat16 storage, MFMA.
//
// Block = 8 waves = 256 consecutive positions of one stream; wave w owns 32
// of them (2 MFMA N-tiles of 16 tokens).  The centred tokens x~_t are built
// once in registers as MFMA B operands (exact bf16).  References stream
// through LDS in double-buffered chunks of 128 (8 M-tiles of 16; the next
// chunk is loaded straight into the other LDS buffer while the current one
// is used); each M-tile x N-tile block of scores is an MFMA 16x16x32 chain
// over the head dim.  The C fragment of lane l holds references 4*(l/16)+i (i = 0..3) for
// token l%16.  Scores are <x~_t, x~_r> / ||x~_r||: the token's own norm is
// the same for every candidate and does not change the argmax.  Each score
// becomes an integer selection key (see below) so that a lane's running
// best is one max instruction per score; the four lane groups that share a
// token merge at the end (larger key, then lower ordinal).
// ---------------------------------------------------------------------------

constexpr int kTop1Refs = 128;    // references per LDS chunk (top-1 search)
// Low key bits that hold a candidate's place in its top-1 chunk: each lane
// sees 4 of every 16 references, kTop1Refs / 4 places.
constexpr uint32_t kPlaceMask = kTop1Refs / 4 - 1;
constexpr int kSearchWaves = 8;
constexpr int kSearchNT = 2;                    // 16-token MFMA tiles per wave
constexpr int kSearchThreads = 64 * kSearchWaves;
constexpr int kSearchTok = 16 * kSearchNT * kSearchWaves;   // positions per block

// Token and mean pieces of a wave's MFMA B operands: token tiles of 16
// positions from tw, lane (lrow, lgrp) holding elements ks * 32 + lgrp * 8 ..
// + 7 of position tw + 16 nt + lrow.  Every load is issued before any is used.
// Positions past the end read the last row: their columns only produce keys
// of positions that are never stored.
template <int D>
__device__ __forceinline__ void load_tokens(const uint16_t* src, int64_t st, const uint16_t* mu, int tw, int T,
                                            int lrow, int lgrp, uint4 (*xr)[D / 32], uint4* mr) {
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) mr[ks] = *reinterpret_cast<const uint4*>(mu + ks * 32 + lgrp * 8);
#pragma unroll
  for (int nt = 0; nt < kSearchNT; ++nt) {
    const int t = min(tw + nt * 16 + lrow, T - 1);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      xr[nt][ks] = *reinterpret_cast<const uint4*>(src + (int64_t)t * st + ks * 32 + lgrp * 8);
  }
}

// rnd(x - mu) of 8 bfloat16 elements as 4 packed pairs: x - mu of two bf16
// values is exact in fp32 or too far from a bf16 tie to round differently,
// so one fp32 subtraction and one rounding give rnd(x - mu).
__device__ __forceinline__ void centre8(uint4 x, uint4 m, uint32_t* w) {
  const uint32_t xv[4] = {x.x, x.y, x.z, x.w}, mv[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
  for (int e = 0; e < 4; ++e)
    w[e] = pk_bf16_rn(__uint_as_float(xv[e] << 16) - __uint_as_float(mv[e] << 16),
                      __uint_as_float(xv[e] & 0xFFFF0000u) - __uint_as_float(mv[e] & 0xFFFF0000u));
}

// Buffer load of 16 bytes per lane straight into LDS: lane l's bytes land
// at lds + 16 l; lds is wave-uniform and below 64 KB (the load takes its LDS
// address from the low 16 bits of M0).
__device__ __forceinline__ void load_to_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}


// s_waitcnt operand that waits for every vector memory operation (vmcnt 0)
// and leaves the export and LDS counters free (gfx9 encoding).
constexpr int kWaitVm0 = 0x0F70;

// Element offset of 16-byte piece pc of row `row` in an LDS reference chunk
// (unpadded rows of D / 8 pieces).  The piece index is XORed with the row
// (with the row pair for d = 64, whose rows are half as long), so the lanes
// of an MFMA A-fragment read, which take the same piece of 16 consecutive
// rows, fall on distinct LDS banks.
template <int D>
__device__ __forceinline__ int chunk_off(int row, int pc) {
  constexpr int SH = D == 128 ? 0 : 1;
  return row * D + ((pc ^ ((row >> SH) & (D / 8 - 1))) << 3);
}

template <int D>
__global__ __launch_bounds__(kSearchThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_search_mfma(CompressArgs a, Shape sh) {
  constexpr int KS = D / 32;      // MFMA K-steps over the head dim
  // Two chunk buffers as separate arrays: the loop below alternates them
  // statically, so the compiler sees that reads of one never wait for the
  // LDS loads into the other.
  __shared__ __attribute__((aligned(16))) uint16_t lds_ref0[kTop1Refs * D], lds_ref1[kTop1Refs * D];
  __shared__ float lds_inv0[kTop1Refs], lds_inv1[kTop1Refs];

  const XcdItem xi = xcd_item(sh.n_streams());
  if (xi.stream < 0) return;
  const int stream = xi.stream;
  const int tile = (sh.T + kSearchTok - 1) / kSearchTok - 1 - xi.item;   // heavy (late) tiles first
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const StreamId id = decode_stream(stream, sh.H);
  const uint16_t* src = stream_src<BF16>(a, id);
  const uint16_t* mu = (const uint16_t*)a.mu + (size_t)stream * D;
  const uint16_t* refs = (const uint16_t*)a.refs + (size_t)stream * sh.Rc * D;
  const float* inv_n = a.inv_n + (size_t)stream * sh.R;

  const int tb = tile * kSearchTok;
  const int tw = tb + wave * 16 * kSearchNT;
  // References any position of the block / wave may use: r*s < t.
  const int tmax_b = min(sh.T - 1, tb + kSearchTok - 1);
  const int rend_b = (tmax_b + sh.s - 1) / sh.s;
  const int tmax_w = min(sh.T - 1, tw + 16 * kSearchNT - 1);
  const int rend_w = tw < sh.T ? (tmax_w + sh.s - 1) / sh.s : 0;
  const int nchunks = (rend_b + kTop1Refs - 1) / kTop1Refs;

  // Chunk loads go straight from global memory to LDS (buffer loads with
  // the LDS flag, issued one chunk ahead): each wave instruction fills 1 KB of
  // the chunk, lane l its 16-byte piece l, so lane l reads the global piece
  // that the swizzle places there (the XOR swizzle is its own inverse).  The
  // buffer descriptor's base is the chunk's first row and its size covers the
  // rows that exist (r < rend_b), so rows past the end read as zeros with no
  // compare or branch; each lane's offsets are the same for every chunk.
  constexpr int NI = kTop1Refs * D * 2 / (kSearchWaves * 1024);   // 1 KB loads per wave per chunk
  uint32_t voff[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int q = (wave * NI + j) * 64 + lane;   // 16-byte piece of the chunk in LDS order
    voff[j] = (uint32_t)chunk_off<D>(q / (D / 8), q % (D / 8)) * 2;
  }
  float pinv = 0.f;
  auto fetch = [&](int ch, uint16_t* dref) {
    const int rc = ch * kTop1Refs;
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(refs + (size_t)rc * D), (short)0, (rend_b - rc) * D * 2, kBufferRsrcWord3);
#pragma unroll
    for (int j = 0; j < NI; ++j)
      load_to_lds16(rr, dref + (wave * NI + j) * 512, voff[j]);
    if (tid < kTop1Refs) {
      const __amdgpu_buffer_rsrc_t rn = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(inv_n + rc), (short)0, (rend_b - rc) * 4, kBufferRsrcWord3);
      pinv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rn, tid * 4, 0, 0));
    }
  };
  // The norm terms go through a register and an LDS store (placed before
  // the barrier that publishes the chunk): the direct LDS loads take their
  // LDS address from the low 16 bits of M0, so only the two reference
  // buffers, the first 64 KB of the block's LDS, are filled that way.
  auto stash_inv = [&](float* dinv) {
    if (tid < kTop1Refs) dinv[tid] = pinv;
  };
  if (nchunks > 0) fetch(0, lds_ref0);

  // B operands: centred tokens rnd(x - mu), [N-tile][K-step], and their
  // squared norms.
  bf16x8 bt[kSearchNT][KS];
  float n2[kSearchNT] = {};
  {
    uint4 xr[kSearchNT][KS], mr[KS];
    load_tokens<D>(src, a.st, mu, tw, sh.T, lrow, lgrp, xr, mr);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nt = 0; nt < kSearchNT; ++nt) {
        uint32_t w[4];
        centre8(xr[nt][ks], mr[ks], w);
        // Squared norm by bf16 pair dot products: it only sets the key
        // offset below, which needs no particular rounding.
#pragma unroll
        for (int e = 0; e < 4; ++e)
          n2[nt] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[e]),
                                                   __builtin_bit_cast(bf16x2_t, w[e]), n2[nt], false);
        bt[nt][ks] = __builtin_bit_cast(bf16x8, w);
      }
  }
  // Selection keys.  A candidate's score <x~_t, x~_r> / ||x~_r|| lies in
  // [-||x~_t||, ||x~_t||]; adding off = 2 ||x~_t|| (+ a tiny constant, so that
  // keys of a zero token stay positive) makes every key a positive float, so
  // keys order as unsigned integers.  The low 5 bits of a key are replaced by
  // 31 - (4 mt + i), the candidate's place in its 128-reference chunk, so an
  // integer max picks the best score and, among equal scores, the lowest
  // ordinal; the change is below 2^-18 relative to the key (below 1.2e-5 in
  // cosine, as keys are at most 3 ||x~_t||), inside the 1e-4 cosine margin
  // within which any near-best reference is accepted.  Across chunks a lane
  // keeps the earlier chunk unless the new chunk's key is strictly larger
  // above those 5 bits.
  float off[kSearchNT];
#pragma unroll
  for (int nt = 0; nt < kSearchNT; ++nt) {
    float v = n2[nt];
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    off[nt] = 2.0f * sqrtf(v) + 1e-30f;
  }
  uint32_t bkey[kSearchNT] = {};
  int bch[kSearchNT] = {};
  // Number of references before the lane's token t (those with r s < t).
  int nprev[kSearchNT];
#pragma unroll
  for (int nt = 0; nt < kSearchNT; ++nt) nprev[nt] = (tw + nt * 16 + lrow + sh.s - 1) / sh.s;

  // The chunk's LDS loads have landed (vmcnt 0) before the barrier.
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  if (nchunks > 0) stash_inv(lds_inv0);
  __syncthreads();
  // One chunk: fetch the next one into (nref, ninv) while this one (cref,
  // cinv) is scored.
  auto chunk = [&](int ch, const uint16_t* cref, const float* cinv, uint16_t* nref, float* ninv) {
    const int rc = ch * kTop1Refs;
    if (ch + 1 < nchunks) fetch(ch + 1, nref);
    uint32_t ckey[kSearchNT] = {};
    const int nmt = min(kTop1Refs / 16, (rend_w - rc + 15) / 16);
    if (rc < rend_w && nmt == kTop1Refs / 16 && (rc + kTop1Refs - 1) * sh.s < tw) {
      // Fast path: a full chunk entirely before the wave's first position
      // needs no causal mask.  The issue order is fixed by hand: K-step ks of
      // tile mt issues its two MFMAs, refills the A-fragment register it has
      // just consumed with tile mt + 1's piece (three K-steps of LDS latency
      // cover), then computes the keys of element ks of tile mt - 1 (three
      // VALU operations per token tile), so one wave keeps the matrix core
      // and the VALU busy together.
      constexpr int MT = kTop1Refs / 16;
      bf16x8 ar[KS];
      f32x4 acc[2][kSearchNT];
      f32x4 inv4;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        ar[ks] = *reinterpret_cast<const bf16x8*>(&cref[chunk_off<D>(lrow, ks * 4 + lgrp)]);
#pragma unroll
      for (int mt = 0; mt <= MT; ++mt) {
        if (mt > 0) inv4 = *reinterpret_cast<const f32x4*>(&cinv[(mt - 1) * 16 + lgrp * 4]);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (mt < MT) {
#pragma unroll
            for (int nt = 0; nt < kSearchNT; ++nt)
              acc[mt & 1][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  ar[ks], bt[nt][ks], ks ? acc[mt & 1][nt] : f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            if (mt + 1 < MT)
              ar[ks] = *reinterpret_cast<const bf16x8*>(
                  &cref[chunk_off<D>((mt + 1) * 16 + lrow, ks * 4 + lgrp)]);
          }
          if (mt > 0) {
            // Elements of the C fragment spread over the K-steps (one per
            // step for d = 128, two for d = 64).
            const int pm = mt - 1;
#pragma unroll
            for (int i = ks * 4 / KS; i < (ks + 1) * 4 / KS; ++i)
#pragma unroll
              for (int nt = 0; nt < kSearchNT; ++nt) {
                const uint32_t k = (__float_as_uint(fmaf(acc[pm & 1][nt][i], inv4[i], off[nt])) & ~kPlaceMask) |
                                   (uint32_t)(kPlaceMask - (4 * pm + i));
                ckey[nt] = max(ckey[nt], k);
              }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else if (rc < rend_w) {
#pragma unroll
      for (int mt = 0; mt < kTop1Refs / 16; ++mt) {
        if (mt < nmt) {
          const int rbase = rc + mt * 16;
          bf16x8 ar[KS];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            ar[ks] = *reinterpret_cast<const bf16x8*>(&cref[chunk_off<D>(mt * 16 + lrow, ks * 4 + lgrp)]);
          f32x4 acc[kSearchNT];
#pragma unroll
          for (int nt = 0; nt < kSearchNT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int nt = 0; nt < kSearchNT; ++nt)
              acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar[ks], bt[nt][ks], acc[nt], 0, 0, 0);
          float inv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) inv[i] = cinv[mt * 16 + lgrp * 4 + i];
          // A tile needs the causal mask when its last reference is not
          // earlier than the wave's first position.
          const bool masked = (rbase + 15) * sh.s >= tw;
          const int r0 = rbase + lgrp * 4;
#pragma unroll
          for (int nt = 0; nt < kSearchNT; ++nt) {
            uint32_t k[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              k[i] = (__float_as_uint(fmaf(acc[nt][i], inv[i], off[nt])) & ~kPlaceMask) | (uint32_t)(kPlaceMask - (4 * mt + i));
            if (masked) {
              // Reference r0 + i precedes the token iff r0 + i < nprev.
              const int lim = nprev[nt] - r0;
#pragma unroll
              for (int i = 0; i < 4; ++i) k[i] = i < lim ? k[i] : 0u;
            }
            ckey[nt] = max(max(max(k[0], k[1]), max(k[2], k[3])), ckey[nt]);
          }
        }
      }
    }
    // A chunk without keys leaves ckey = 0, which never replaces the best.
#pragma unroll
    for (int nt = 0; nt < kSearchNT; ++nt) {
      const bool g = (ckey[nt] & ~kPlaceMask) > (bkey[nt] & ~kPlaceMask);
      bkey[nt] = g ? ckey[nt] : bkey[nt];
      bch[nt] = g ? ch : bch[nt];
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    if (ch + 1 < nchunks) stash_inv(ninv);
    __syncthreads();
  };
  for (int ch = 0; ch < nchunks; ch += 2) {
    chunk(ch, lds_ref0, lds_inv0, lds_ref1, lds_inv1);
    if (ch + 1 < nchunks) chunk(ch + 1, lds_ref1, lds_inv1, lds_ref0, lds_inv0);
  }

  // Merge the four lane groups of each token (larger key above the place
  // bits, then lower ordinal); lanes 0..15 write.
#pragma unroll
  for (int nt = 0; nt < kSearchNT; ++nt) {
    const int q = (int)kPlaceMask - (int)(bkey[nt] & kPlaceMask);
    uint32_t v = bkey[nt] & ~kPlaceMask;
    int r = bch[nt] * kTop1Refs + (q >> 2) * 16 + lgrp * 4 + (q & 3);
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const uint32_t v2 = (uint32_t)__shfl_xor((int)v, o, 64);
      const int r2 = __shfl_xor(r, o, 64);
      if (v2 > v || (v2 == v && r2 < r)) { v = v2; r = r2; }
    }
    const int t = tw + nt * 16 + lrow;
    if (lgrp == 0 && t < sh.T && t % sh.s != 0)
      store_idx(a.idx, (size_t)stream * sh.Nc + pos_to_slot(t, sh.s), sh.idx_bytes, (uint32_t)r);
  }
}

// ---------------------------------------------------------------------------
// Reference search, float32 storage: one thread per position, fp32 VALU.
// grid (ceil(T/256), streams), block 256.  References in LDS chunks of 32.
// ---------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256) void k_search_f32(CompressArgs a, Shape sh) {
  constexpr int CH = 32;
  __shared__ float lds_ref[CH][D];
  __shared__ float lds_inv[CH];
  const int stream = blockIdx.y;
  const int tile = gridDim.x - 1 - blockIdx.x;
  const StreamId id = decode_stream(stream, sh.H);
  const float* src = stream_src<F32>(a, id);
  const float* mu = (const float*)a.mu + (size_t)stream * D;
  const float* refs = (const float*)a.refs + (size_t)stream * sh.Rc * D;
  const float* inv_n = a.inv_n + (size_t)stream * sh.R;
  const int t = tile * 256 + threadIdx.x;
  const int tmax_b = min(sh.T - 1, tile * 256 + 255);
  const int rend_b = (tmax_b + sh.s - 1) / sh.s;
  float x[D];
  if (t < sh.T) {
#pragma unroll
    for (int i = 0; i < D; ++i) x[i] = src[(int64_t)t * a.st + i] - mu[i];
  } else {
#pragma unroll
    for (int i = 0; i < D; ++i) x[i] = 0.f;
  }
  float best = -INFINITY;
  int bi = 0;
  for (int rc = 0; rc < rend_b; rc += CH) {
    __syncthreads();
    for (int p = threadIdx.x; p < CH * D; p += 256) {
      const int row = p / D, col = p % D;
      lds_ref[row][col] = rc + row < rend_b ? refs[(size_t)(rc + row) * D + col] : 0.f;
    }
    if (threadIdx.x < CH) lds_inv[threadIdx.x] = rc + threadIdx.x < rend_b ? inv_n[rc + threadIdx.x] : 0.f;
    __syncthreads();
    for (int j = 0; j < CH; ++j) {
      const int r = rc + j;
      if (r * sh.s >= t) break;
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) dot = fmaf(x[i], lds_ref[j][i], dot);
      const float sc = dot * lds_inv[j];
      if (sc > best) { best = sc; bi = r; }
    }
  }
  if (t < sh.T && t % sh.s != 0)
    store_idx(a.idx, (size_t)stream * sh.Nc + pos_to_slot(t, sh.s), sh.idx_bytes, (uint32_t)bi);
}

// ---------------------------------------------------------------------------
// Encode, bfloat16 storage, MFMA.
//
// grid (ceil(N/64), streams), block 256: wave w encodes coded rows
// 64*blockIdx.x + 16*w + (0..15).  A = W_down rows (M = code elements, from
// LDS), B = residuals of 16 tokens (N), K = head dim.  The fp32 residual
// delta = (k - mu) - ref is split into bf16 parts hi + lo, which hold it to
// 16 significant bits; two MFMA passes give the projection to about 2^-16
// relative, far below the final rounding of the code to bf16 (2^-9).
// ---------------------------------------------------------------------------


// ---------------------------------------------------------------------------
// Search for k references, or by L2 distance (top_k > 1 or metric = L2).
// Each candidate (score, ordinal) enters a sorted list of the best k under
// the total order "higher score, then lower ordinal"; the lists of a token
// are merged at the end, and the kept ordinals written in ascending order,
// zero past the token's count min(k, floor(t / s) + 1).
// Scores: cosine order is dot / ||r|| (0 for a zero reference); L2 order is
// 2 dot - ||r||^2 (= ||x||^2 - ||x - r||^2, the token's norm being common).
// ---------------------------------------------------------------------------

// bfloat16: the block and chunk structure of k_search_mfma (256 positions
// per block, two 16-token MFMA tiles per wave, 128-reference chunks loaded
// straight into XOR-swizzled LDS, the norm terms through a register), with
// lists of the KT best candidates in place of the running maximum, and no
// data-dependent branches.  Candidates carry the selection key of
// k_search_mfma: an unsigned integer that orders as the score (cosine:
// dot / ||r|| offset by 2 ||x~_t||; L2: 2 dot - ||r||^2 in the usual
// sign-flip integer order of floats), with its low 5 bits replaced by
// 31 - (place in the chunk), so equal scores within a chunk order by
// ordinal; the perturbation is below 2^-18 of the key (cosine: keys are at
// most 3 ||x~_t||) or of |score| (L2), inside the 1e-4 margin.  Key 0 is
// "no candidate".  Per chunk a lane keeps a descending list of its KT best
// keys: each tile's four keys are sorted by a network and merged in with a
// bitonic step.  At the end of the chunk the list
// joins the lane's running list of (key, ordinal) under the total order
// "key above the place bits, then lower ordinal", by the same bitonic
// merge; at the end the four lane groups of a token merge their lists the
// same way and lane group 0 writes the first min(k, refs before t)
// ordinals in ascending order.  KT = 1, 4 or 8 >= k.
// ---------------------------------------------------------------------------

// a >= b afterwards.
__device__ __forceinline__ void cswap_u(uint32_t& a, uint32_t& b) {
  const uint32_t hi = max(a, b), lo = min(a, b);
  a = hi;
  b = lo;
}

// Sorts a bitonic sequence into descending order (half-cleaner stages).
template <int N>
__device__ __forceinline__ void bitonic_desc(uint32_t (&v)[N]) {
#pragma unroll
  for (int h = N / 2; h >= 1; h /= 2)
#pragma unroll
    for (int j = 0; j < N; ++j)
      if ((j & h) == 0) cswap_u(v[j], v[j + h]);
}

// The four keys of a tile into a descending list of the KT best keys.
template <int KT>
__device__ __forceinline__ void tile_into_list(uint32_t (&L)[KT], uint32_t c0, uint32_t c1, uint32_t c2,
                                               uint32_t c3) {
  if constexpr (KT == 1) {
    L[0] = max(max(L[0], c0), max(max(c1, c2), c3));
  } else {
    uint32_t c[4] = {c0, c1, c2, c3};
    cswap_u(c[0], c[1]);
    cswap_u(c[2], c[3]);
    cswap_u(c[0], c[2]);
    cswap_u(c[1], c[3]);
    cswap_u(c[1], c[2]);
    // L descending and c ascending side by side: their elementwise maxima
    // form a bitonic sequence holding the KT largest of both.
#pragma unroll
    for (int j = 0; j < 4; ++j) L[KT - 4 + j] = max(L[KT - 4 + j], c[3 - j]);
    bitonic_desc(L);
  }
}

// Running lists: keys and ordinals, ordered by the key above the place bits
// (descending), then by ordinal (ascending).
template <int KT>
struct SelList {
  uint32_t k[KT];
  int r[KT];
};

__device__ __forceinline__ bool sel_before(uint32_t ak, int ar, uint32_t bk, int br) {
  const uint32_t at = ak & ~kPlaceMask, bt = bk & ~kPlaceMask;
  return (at > bt) | ((at == bt) & (ar < br));
}

// G <- the KT first of G and (bk, br), both in list order.
template <int KT>
__device__ __forceinline__ void merge_sel(SelList<KT>& G, const uint32_t (&bk)[KT], const int (&br)[KT]) {
#pragma unroll
  for (int j = 0; j < KT; ++j) {
    const int q = KT - 1 - j;
    const bool take = sel_before(bk[q], br[q], G.k[j], G.r[j]);
    G.k[j] = take ? bk[q] : G.k[j];
    G.r[j] = take ? br[q] : G.r[j];
  }
#pragma unroll
  for (int h = KT / 2; h >= 1; h /= 2)
#pragma unroll
    for (int j = 0; j < KT; ++j)
      if ((j & h) == 0) {
        const bool sw = sel_before(G.k[j + h], G.r[j + h], G.k[j], G.r[j]);
        const uint32_t tk = G.k[j];
        const int tr = G.r[j];
        G.k[j] = sw ? G.k[j + h] : G.k[j];
        G.r[j] = sw ? G.r[j + h] : G.r[j];
        G.k[j + h] = sw ? tk : G.k[j + h];
        G.r[j + h] = sw ? tr : G.r[j + h];
      }
}

// Selection key of a candidate with accumulator acc and norm term n (off:
// the token's cosine offset).
template <bool L2>
__device__ __forceinline__ uint32_t sel_key(float acc, float n, float off, uint32_t place) {
  uint32_t u;
  if constexpr (L2) {
    const uint32_t b = __float_as_uint(fmaf(2.f, acc, -n));
    u = b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
  } else {
    u = __float_as_uint(fmaf(acc, n, off));
  }
  return (u & ~kPlaceMask) | (kPlaceMask - place);
}

template <int D, int KT, bool L2>
__global__ __launch_bounds__(kSearchThreads) __attribute__((amdgpu_waves_per_eu(KT > 4 ? 2 : 4))) void k_search_topk_mfma(
    CompressArgs a, Shape sh) {
  constexpr int KS = D / 32;
  constexpr int MT = kTop1Refs / 16;
  __shared__ __attribute__((aligned(16))) uint16_t lds_ref0[kTop1Refs * D], lds_ref1[kTop1Refs * D];
  __shared__ __attribute__((aligned(16))) float lds_n0[kTop1Refs], lds_n1[kTop1Refs];

  const XcdItem xi = xcd_item(sh.n_streams());
  if (xi.stream < 0) return;
  const int stream = xi.stream;
  const int tile = (sh.T + kSearchTok - 1) / kSearchTok - 1 - xi.item;   // heavy (late) tiles first
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const StreamId id = decode_stream(stream, sh.H);
  const uint16_t* src = stream_src<BF16>(a, id);
  const uint16_t* mu = (const uint16_t*)a.mu + (size_t)stream * D;
  const uint16_t* refs = (const uint16_t*)a.refs + (size_t)stream * sh.Rc * D;
  const float* nrm = a.inv_n + (size_t)stream * sh.R;

  const int tb = tile * kSearchTok;
  const int tw = tb + wave * 16 * kSearchNT;
  const int tmax_b = min(sh.T - 1, tb + kSearchTok - 1);
  const int rend_b = (tmax_b + sh.s - 1) / sh.s;
  const int tmax_w = min(sh.T - 1, tw + 16 * kSearchNT - 1);
  const int rend_w = tw < sh.T ? (tmax_w + sh.s - 1) / sh.s : 0;
  const int nchunks = (rend_b + kTop1Refs - 1) / kTop1Refs;

  // Chunk loads as in k_search_mfma.
  constexpr int NI = kTop1Refs * D * 2 / (kSearchWaves * 1024);
  float pn = 0.f;
  auto fetch = [&](int ch, uint16_t* dref) {
    const int rc = ch * kTop1Refs;
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(refs + (size_t)rc * D), (short)0, (rend_b - rc) * D * 2, kBufferRsrcWord3);
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int q = (wave * NI + j) * 64 + lane;
      load_to_lds16(rr, dref + (wave * NI + j) * 512, (uint32_t)chunk_off<D>(q / (D / 8), q % (D / 8)) * 2);
    }
    if (tid < kTop1Refs) {
      const __amdgpu_buffer_rsrc_t rn = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(nrm + rc), (short)0, (rend_b - rc) * 4, kBufferRsrcWord3);
      pn = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rn, tid * 4, 0, 0));
    }
  };
  auto stash = [&](float* dn) {
    if (tid < kTop1Refs) dn[tid] = pn;
  };
  if (nchunks > 0) fetch(0, lds_ref0);

  // B operands (centred tokens rnd(x - mu)) and, for cosine, the key offset
  // 2 ||x~_t|| of k_search_mfma.
  bf16x8 bt[kSearchNT][KS];
  float off[kSearchNT] = {};
  {
    uint4 xr[kSearchNT][KS], mr[KS];
    load_tokens<D>(src, a.st, mu, tw, sh.T, lrow, lgrp, xr, mr);
    float n2[kSearchNT] = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nt = 0; nt < kSearchNT; ++nt) {
        uint32_t w[4];
        centre8(xr[nt][ks], mr[ks], w);
        if (!L2) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            n2[nt] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[e]),
                                                     __builtin_bit_cast(bf16x2_t, w[e]), n2[nt], false);
        }
        bt[nt][ks] = __builtin_bit_cast(bf16x8, w);
      }
    if (!L2) {
#pragma unroll
      for (int nt = 0; nt < kSearchNT; ++nt) {
        float v = n2[nt];
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        off[nt] = 2.0f * sqrtf(v) + 1e-30f;
      }
    }
  }

  SelList<KT> best[kSearchNT];
#pragma unroll
  for (int nt = 0; nt < kSearchNT; ++nt)
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      best[nt].k[j] = 0u;
      best[nt].r[j] = 0x7FFFFFFF;
    }

  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  if (nchunks > 0) stash(lds_n0);
  __syncthreads();
  auto chunk = [&](int ch, const uint16_t* cref, const float* cn, uint16_t* nref, float* nn) {
    const int rc = ch * kTop1Refs;
    if (ch + 1 < nchunks) fetch(ch + 1, nref);
    uint32_t L[kSearchNT][KT];
#pragma unroll
    for (int nt = 0; nt < kSearchNT; ++nt)
#pragma unroll
      for (int j = 0; j < KT; ++j) L[nt][j] = 0u;
    const int nmt = min(MT, (rend_w - rc + 15) / 16);
    if (rc < rend_w && nmt == MT && (rc + kTop1Refs - 1) * sh.s < tw) {
      // Full chunk before the wave's first position: no causal mask.  The A
      // fragments of tile mt + 1 are read from LDS while tile mt's MFMAs run.
      bf16x8 ar[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        ar[ks] = *reinterpret_cast<const bf16x8*>(&cref[chunk_off<D>(lrow, ks * 4 + lgrp)]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 acc[kSearchNT];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
          for (int nt = 0; nt < kSearchNT; ++nt)
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar[ks], bt[nt][ks],
                                                              ks ? acc[nt] : f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          if (mt + 1 < MT)
            ar[ks] = *reinterpret_cast<const bf16x8*>(&cref[chunk_off<D>((mt + 1) * 16 + lrow, ks * 4 + lgrp)]);
        }
        const f32x4 n4 = *reinterpret_cast<const f32x4*>(&cn[mt * 16 + lgrp * 4]);
#pragma unroll
        for (int nt = 0; nt < kSearchNT; ++nt) {
          uint32_t c[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) c[i] = sel_key<L2>(acc[nt][i], n4[i], off[nt], (uint32_t)(4 * mt + i));
          tile_into_list<KT>(L[nt], c[0], c[1], c[2], c[3]);
        }
      }
    } else if (rc < rend_w) {
      // Partial or diagonal chunk, one tile at a time; a candidate needs
      // r s < t.
#pragma unroll 1
      for (int mt = 0; mt < nmt; ++mt) {
        const int rbase = rc + mt * 16;
        bf16x8 ar[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          ar[ks] = *reinterpret_cast<const bf16x8*>(&cref[chunk_off<D>(mt * 16 + lrow, ks * 4 + lgrp)]);
        f32x4 acc[kSearchNT];
#pragma unroll
        for (int nt = 0; nt < kSearchNT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int nt = 0; nt < kSearchNT; ++nt)
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar[ks], bt[nt][ks], acc[nt], 0, 0, 0);
        const f32x4 n4 = *reinterpret_cast<const f32x4*>(&cn[mt * 16 + lgrp * 4]);
        const int r0 = rbase + lgrp * 4;
#pragma unroll
        for (int nt = 0; nt < kSearchNT; ++nt) {
          const int t = tw + nt * 16 + lrow;
          uint32_t c[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t k = sel_key<L2>(acc[nt][i], n4[i], off[nt], (uint32_t)(4 * mt + i));
            c[i] = (r0 + i) * sh.s < t ? k : 0u;
          }
          tile_into_list<KT>(L[nt], c[0], c[1], c[2], c[3]);
        }
      }
    }
    if (rc < rend_w) {
      // The chunk's lists join the running lists (ordinals from the place
      // bits).
#pragma unroll
      for (int nt = 0; nt < kSearchNT; ++nt) {
        int lr[KT];
#pragma unroll
        for (int j = 0; j < KT; ++j) {
          const uint32_t q = kPlaceMask - (L[nt][j] & kPlaceMask);
          lr[j] = rc + (int)(q >> 2) * 16 + lgrp * 4 + (int)(q & 3);
        }
        merge_sel<KT>(best[nt], L[nt], lr);
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    if (ch + 1 < nchunks) stash(nn);
    __syncthreads();
  };
  for (int ch = 0; ch < nchunks; ch += 2) {
    chunk(ch, lds_ref0, lds_n0, lds_ref1, lds_n1);
    if (ch + 1 < nchunks) chunk(ch + 1, lds_ref1, lds_n1, lds_ref0, lds_n0);
  }

  // The four lane groups of each token merge their lists; lane group 0
  // writes the first min(k, refs before t) ordinals in ascending order.
  const int K = sh.K;
#pragma unroll
  for (int nt = 0; nt < kSearchNT; ++nt) {
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      uint32_t ok[KT];
      int orr[KT];
#pragma unroll
      for (int j = 0; j < KT; ++j) {
        ok[j] = (uint32_t)__shfl_xor((int)best[nt].k[j], o, 64);
        orr[j] = __shfl_xor(best[nt].r[j], o, 64);
      }
      merge_sel<KT>(best[nt], ok, orr);
    }
    const int t = tw + nt * 16 + lrow;
    if (lgrp == 0 && t < sh.T && t % sh.s != 0) {
      const int c = min(K, t / sh.s + 1);
      int v[KT];
#pragma unroll
      for (int j = 0; j < KT; ++j) v[j] = j < c ? best[nt].r[j] : 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < KT; ++i)
#pragma unroll
        for (int j = 0; j + 1 < KT - i; ++j) {
          const int lo = min(v[j], v[j + 1]), hi = max(v[j], v[j + 1]);
          v[j] = lo;
          v[j + 1] = hi;
        }
      const size_t base = ((size_t)stream * sh.Nc + pos_to_slot(t, sh.s)) * K;
      for (int j = 0; j < K; ++j) store_idx(a.idx, base + j, sh.idx_bytes, (uint32_t)(j < c ? v[j] : 0));
    }
  }
}

// float32 storage: one thread per token, references staged through LDS.
template <int D>
__global__ __launch_bounds__(256) void k_search_topk_f32(CompressArgs a, Shape sh) {
  constexpr int CH = 32;
  __shared__ float lds_ref[CH][D];
  __shared__ float lds_n2[CH];
  const int stream = blockIdx.y;
  const int K = sh.K;
  const StreamId id = decode_stream(stream, sh.H);
  const float* src = stream_src<F32>(a, id);
  const float* mu = (const float*)a.mu + (size_t)stream * D;
  const float* refs = (const float*)a.refs + (size_t)stream * sh.Rc * D;
  const int n = blockIdx.x * 256 + threadIdx.x;
  const bool valid = n < sh.N;
  const int t = valid ? slot_to_pos(n, sh.s) : 0;
  const int nlast = min(sh.N - 1, (int)blockIdx.x * 256 + 255);
  const int nref = (slot_to_pos(nlast, sh.s) - 1) / sh.s + 1;
  float x[D];
#pragma unroll
  for (int i = 0; i < D; ++i) x[i] = valid ? src[(int64_t)t * a.st + i] - mu[i] : 0.f;
  TopK top;
  top.init();
  for (int rc = 0; rc < nref; rc += CH) {
    __syncthreads();
    for (int p = threadIdx.x; p < CH * D; p += 256) {
      const int row = p / D, col = p % D;
      lds_ref[row][col] = rc + row < nref ? refs[(size_t)(rc + row) * D + col] : 0.f;
    }
    __syncthreads();
    if (threadIdx.x < CH) {
      float q = 0.f;
      for (int i = 0; i < D; ++i) q = fmaf(lds_ref[threadIdx.x][i], lds_ref[threadIdx.x][i], q);
      lds_n2[threadIdx.x] = q;
    }
    __syncthreads();
    for (int j = 0; j < CH; ++j) {
      const int r = rc + j;
      if (!valid || r >= nref || r * sh.s >= t) break;
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) dot = fmaf(x[i], lds_ref[j][i], dot);
      const float nn = lds_n2[j];
      const float v = sh.l2 ? 2.f * dot - nn : (nn > 0.f ? dot / sqrtf(nn) : 0.f);
      float ths;
      int thr;
      top.kth(K, ths, thr);
      if (ranks_before(v, r, ths, thr)) top.insert(v, r, K);
    }
  }
  if (valid) {
    int o[kTopMax];
    top.sorted_ordinals(min(K, t / sh.s + 1), o);
    const size_t base = ((size_t)stream * sh.Nc + n) * K;
    for (int j = 0; j < K; ++j) store_idx(a.idx, base + j, sh.idx_bytes, (uint32_t)o[j]);
  }
}

constexpr int kEncTiles = 4;   // 64-row tiles per encode block

template <int D, bool Q4>
__global__ __launch_bounds__(256) void k_encode_mfma(CompressArgs a, Shape sh) {
  constexpr int KS = D / 32;
  constexpr int LDW = D + 8;          // padded LDS row of W_down
  extern __shared__ __attribute__((aligned(16))) uint16_t w_lds[];   // [d_c][LDW]
  const XcdItem xi = xcd_item(sh.n_streams());
  if (xi.stream < 0) return;
  const int stream = xi.stream;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const StreamId id = decode_stream(stream, sh.H);
  const uint16_t* src = stream_src<BF16>(a, id);
  const uint16_t* mu = (const uint16_t*)a.mu + (size_t)stream * D;
  const uint16_t* refs = (const uint16_t*)a.refs + (size_t)stream * sh.Rc * D;
  const uint16_t* wd = (const uint16_t*)(id.kv ? a.wdv : a.wdk) + (size_t)id.h * a.w_hs;
  uint16_t* codes = (uint16_t*)a.codes + (size_t)stream * sh.Nc * sh.dc;

  // Rows of tile j (kEncTiles tiles of 64 rows per block); loads use the
  // row clamped to the last coded row, stores are masked.  The next tile's
  // ordinal and token row are loaded while this tile's reference rows are in
  // flight, so a tile costs about one memory round trip.
  const int K = sh.K;
  auto row_of = [&](int j) { return (xi.item * kEncTiles + j) * 64 + wave * 16 + lrow; };
  uint32_t r_nx;
  int s_nx;   // row the code is stored in (the grouped row for grouped layouts)
  uint4 x_nx[KS];
  auto prefetch = [&](int j) {
    const int nc = min(row_of(j), sh.N - 1);
    const int tc = slot_to_pos(nc, sh.s);
    r_nx = load_idx(a.idx, ((size_t)stream * sh.Nc + nc) * K, sh.idx_bytes);
    s_nx = a.perm ? a.perm[(size_t)(stream >> 1) * sh.Nc + nc] : nc;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      x_nx[ks] = *reinterpret_cast<const uint4*>(src + (int64_t)tc * a.st + ks * 32 + lgrp * 8);
  };
  prefetch(0);
  uint4 mr[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) mr[ks] = *reinterpret_cast<const uint4*>(mu + ks * 32 + lgrp * 8);

  for (int p = threadIdx.x; p < sh.dc * (D / 8); p += 256) {
    const int row = p / (D / 8), col = (p % (D / 8)) * 8;
    *reinterpret_cast<uint4*>(&w_lds[row * LDW + col]) = *reinterpret_cast<const uint4*>(wd + (size_t)row * D + col);
  }

#pragma unroll
  for (int jt = 0; jt < kEncTiles; ++jt) {
    const int n = row_of(jt);   // this lane's coded row
    const bool valid = n < sh.N;
    const int nc = min(n, sh.N - 1);
    const int t = slot_to_pos(nc, sh.s);
    // The row's references: one ordinal, or (top_k > 1) the first
    // c = min(k, floor(t / s) + 1) of its k, whose mean is the reference.
    const int cnt = min(K, t / sh.s + 1);
    const size_t ibase = ((size_t)stream * sh.Nc + nc) * K;
    const int r = min((int)r_nx, sh.R - 1);
    const int slot = s_nx;
    uint4 xr[KS], rr[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      xr[ks] = x_nx[ks];
      rr[ks] = *reinterpret_cast<const uint4*>(refs + (size_t)r * D + ks * 32 + lgrp * 8);
    }
    if (jt + 1 < kEncTiles) prefetch(jt + 1);

    bf16x8 bh[KS], bl[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = ks * 32 + lgrp * 8;
      float x[8], m[8], rf[8];
      unpack8(xr[ks], x);
      unpack8(mr[ks], m);
      unpack8(rr[ks], rf);
      if (K > 1) {
        for (int j = 1; j < cnt; ++j) {
          float rj[8];
          load8(refs + (size_t)min((int)load_idx(a.idx, ibase + j, sh.idx_bytes), sh.R - 1) * D + c, rj);
#pragma unroll
          for (int e = 0; e < 8; ++e) rf[e] += rj[e];
        }
        const float inv = 1.0f / (float)cnt;
#pragma unroll
        for (int e = 0; e < 8; ++e) rf[e] = cnt > 1 ? rf[e] * inv : rf[e];
      }
      uint32_t wh[4], wl[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float d0 = (x[2 * e] - m[2 * e]) - rf[2 * e];
        const float d1 = (x[2 * e + 1] - m[2 * e + 1]) - rf[2 * e + 1];
        wh[e] = pk_bf16_rn(d0, d1);
        wl[e] = pk_bf16_rn(d0 - __uint_as_float(wh[e] << 16), d1 - __uint_as_float(wh[e] & 0xFFFF0000u));
      }
      bh[ks] = __builtin_bit_cast(bf16x8, wh);
      bl[ks] = __builtin_bit_cast(bf16x8, wl);
    }
    if (jt == 0) __syncthreads();   // W_down staged

    if constexpr (!Q4) {
      for (int mt = 0; mt < sh.dc / 16; ++mt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 aw = *reinterpret_cast<const bf16x8*>(&w_lds[(mt * 16 + lrow) * LDW + ks * 32 + lgrp * 8]);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, bl[ks], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, bh[ks], acc, 0, 0, 0);
        }
        // Lane l holds code elements mt*16 + 4*(l/16) + (0..3) of row l%16.
        if (valid) {
          uint2 o;
          o.x = pk_bf16_rn(acc[0], acc[1]);
          o.y = pk_bf16_rn(acc[2], acc[3]);
          *reinterpret_cast<uint2*>(codes + (size_t)slot * sh.dc + mt * 16 + lgrp * 4) = o;
        }
      }
    } else {
      // 4-bit codes: the whole row first (up to D / 16 tiles), then its
      // maximum magnitude over the row's lanes l, l ^ 16, l ^ 32, l ^ 48, the
      // scale and the nibbles.
      const int nmt = sh.dc / 16;
      f32x4 acc[D / 16];
      float amax = 0.f;
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt) {
        acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (mt < nmt) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 aw = *reinterpret_cast<const bf16x8*>(&w_lds[(mt * 16 + lrow) * LDW + ks * 32 + lgrp * 8]);
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, bl[ks], acc[mt], 0, 0, 0);
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, bh[ks], acc[mt], 0, 0, 0);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(acc[mt][i]));
        }
      }
      amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
      const uint16_t sbits = f2bf(amax / 7.0f);
      const float scale = bf2f(sbits);
      uint8_t* qrow = (uint8_t*)a.codes + ((size_t)stream * sh.Nc + slot) * (sh.dc / 2);
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt) {
        if (mt < nmt && valid) {
          const uint32_t q0 = (uint32_t)q4_quant(acc[mt][0], scale) & 15u, q1 = (uint32_t)q4_quant(acc[mt][1], scale) & 15u;
          const uint32_t q2 = (uint32_t)q4_quant(acc[mt][2], scale) & 15u, q3 = (uint32_t)q4_quant(acc[mt][3], scale) & 15u;
          *reinterpret_cast<uint16_t*>(qrow + mt * 8 + lgrp * 2) = (uint16_t)(q0 | (q1 << 4) | (q2 << 8) | (q3 << 12));
        }
      }
      if (valid && lgrp == 0) ((uint16_t*)a.scales)[(size_t)stream * sh.Nc + slot] = sbits;
    }
  }
}

// Encode, float32 storage: one thread per coded row, fp32 VALU.
// grid (ceil(N/256), streams), block 256.
template <int D>
__global__ __launch_bounds__(256) void k_encode_f32(CompressArgs a, Shape sh) {
  const int stream = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= sh.N) return;
  const StreamId id = decode_stream(stream, sh.H);
  const float* wd = (const float*)(id.kv ? a.wdv : a.wdk) + (size_t)id.h * a.w_hs;
  const float* src = stream_src<F32>(a, id);
  const float* mu = (const float*)a.mu + (size_t)stream * D;
  const float* refs = (const float*)a.refs + (size_t)stream * sh.Rc * D;
  const int t = slot_to_pos(n, sh.s);
  const int K = sh.K;
  const int cnt = min(K, t / sh.s + 1);
  const size_t ibase = ((size_t)stream * sh.Nc + n) * K;
  const int slot = a.perm ? a.perm[(size_t)(stream >> 1) * sh.Nc + n] : n;   // row the code is stored in
  float dl[D];
#pragma unroll
  for (int i = 0; i < D; ++i) dl[i] = 0.f;
  for (int j = 0; j < cnt; ++j) {   // sum of the row's references (one when top_k = 1)
    const int r = min((int)load_idx(a.idx, ibase + j, sh.idx_bytes), sh.R - 1);
#pragma unroll
    for (int i = 0; i < D; ++i) dl[i] += refs[(size_t)r * D + i];
  }
  const float inv = 1.0f / (float)cnt;
#pragma unroll
  for (int i = 0; i < D; ++i) dl[i] = (src[(int64_t)t * a.st + i] - mu[i]) - (cnt > 1 ? dl[i] * inv : dl[i]);
  if (!sh.q4) {
    float* codes = (float*)a.codes + ((size_t)stream * sh.Nc + slot) * sh.dc;
    for (int j = 0; j < sh.dc; ++j) {
      float c = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) c = fmaf(wd[(size_t)j * D + i], dl[i], c);
      codes[j] = c;
    }
    return;
  }
  // 4-bit codes: one pass for the row's maximum magnitude, a second pass
  // recomputes each code (same order, same value) and quantizes it.
  float amax = 0.f;
  for (int j = 0; j < sh.dc; ++j) {
    float c = 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) c = fmaf(wd[(size_t)j * D + i], dl[i], c);
    amax = fmaxf(amax, fabsf(c));
  }
  const float scale = amax / 7.0f;
  uint8_t* qrow = (uint8_t*)a.codes + ((size_t)stream * sh.Nc + slot) * (sh.dc / 2);
  for (int j = 0; j < sh.dc; j += 2) {
    float c0 = 0.f, c1 = 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) {
      c0 = fmaf(wd[(size_t)j * D + i], dl[i], c0);
      c1 = fmaf(wd[(size_t)(j + 1) * D + i], dl[i], c1);
    }
    qrow[j / 2] = (uint8_t)(((uint32_t)q4_quant(c0, scale) & 15u) | (((uint32_t)q4_quant(c1, scale) & 15u) << 4));
  }
  ((float*)a.scales)[(size_t)stream * sh.Nc + slot] = scale;
}

// ---------------------------------------------------------------------------
// Grouping by value reference (layouts with order = by value reference).
// The coded rows of head (b, h) are put in the order of (V ordinal,
// position): a counting sort, stable in position, over pieces of
// kGroupPiece position rows.  k_group_count counts each piece's V ordinals;
// k_group_scan gives each piece the count of every ordinal in the pieces
// before it, and the total per ordinal; k_group_place sorts the piece's
// (ordinal, row) keys, gives each row its grouped slot (the rows of all
// lower ordinals, then this ordinal's rows in earlier pieces, then its rank
// among the piece's rows of that ordinal) and moves the K and V ordinals
// there.  Integer work only: the order is deterministic.
// ---------------------------------------------------------------------------

// grid (pieces, B*H), block kGroupThreads, dynamic LDS R * 4 bytes.
__global__ __launch_bounds__(kGroupThreads) void k_group_count(CompressArgs a, Shape sh) {
  extern __shared__ int cnt[];
  const int head = blockIdx.y, p = blockIdx.x;
  const int n0 = p * kGroupPiece, len = min(kGroupPiece, sh.N - n0);
  for (int r = threadIdx.x; r < sh.R; r += kGroupThreads) cnt[r] = 0;
  __syncthreads();
  const size_t vbase = (size_t)(2 * head + 1) * sh.Nc + n0;
  for (int i = threadIdx.x; i < len; i += kGroupThreads)
    atomicAdd(&cnt[min((int)load_idx(a.idx, vbase + i, sh.idx_bytes), sh.R - 1)], 1);
  __syncthreads();
  int* out = a.gcnt + ((size_t)head * gridDim.x + p) * sh.R;
  for (int r = threadIdx.x; r < sh.R; r += kGroupThreads) out[r] = cnt[r];
}

// grid (ceil(R / 256), B*H), block 256: thread r walks the pieces, 16 loads
// in flight at a time, leaving each piece's exclusive prefix and the total.
__global__ __launch_bounds__(256) void k_group_scan(CompressArgs a, Shape sh, int P) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= sh.R) return;
  const int head = blockIdx.y;
  int* c = a.gcnt + (size_t)head * P * sh.R + r;
  int run = 0;
  for (int p0 = 0; p0 < P; p0 += 16) {
    int v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = p0 + u < P ? c[(size_t)(p0 + u) * sh.R] : 0;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (p0 + u < P) {
        c[(size_t)(p0 + u) * sh.R] = run;
        run += v[u];
      }
    }
  }
  a.gtot[(size_t)head * sh.R + r] = run;
}

// grid (pieces, B*H), block kGroupThreads, dynamic LDS R * 4 bytes (the first
// grouped row of each ordinal).  Every global load is unconditional (clamped
// indices, masked afterwards) and issued in batches, so the kernel waits on
// few memory round trips.
template <typename IdxT>
__global__ __launch_bounds__(kGroupThreads) void k_group_place(CompressArgs a, Shape sh) {
  __shared__ uint32_t keys[2][kGroupPiece];   // (V ordinal << 12) | row in piece, two buffers
  __shared__ int wcnt[kGroupThreads / 64][256];
  __shared__ int wsum[kGroupThreads / 64];
  extern __shared__ int off[];
  static_assert(kGroupPiece == 4 * kGroupThreads && kGroupPiece <= 4096, "4 keys a thread; 12-bit row field");
  constexpr int T = kGroupThreads;
  const int head = blockIdx.y, p = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n0 = p * kGroupPiece, len = min(kGroupPiece, sh.N - n0);
  const IdxT* kin = (const IdxT*)a.idx + (size_t)(2 * head) * sh.Nc + n0;
  const IdxT* vin = kin + sh.Nc;
  // Thread t holds keys 4t .. 4t + 3 (past the piece: all ones, sorted last).
  uint32_t k[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) k[e] = (uint32_t)vin[min(4 * tid + e, len - 1)];
  // Rows per ordinal -> exclusive prefix (the grouped row of the ordinal's
  // first row): thread t scans a contiguous segment, then the segment sums
  // are scanned over the wave and over the waves.
  const int* tot = a.gtot + (size_t)head * sh.R;
  for (int r0 = tid; r0 < sh.R; r0 += 8 * T) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = tot[min(r0 + u * T, sh.R - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (r0 + u * T < sh.R) off[r0 + u * T] = v[u];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = 4 * tid + e;
    k[e] = i < len ? (min(k[e], (uint32_t)sh.R - 1u) << 12) | (uint32_t)i : 0xFFFFFFFFu;
  }
  __syncthreads();
  const int seg = (sh.R + T - 1) / T;
  const int r0 = min(tid * seg, sh.R), r1 = min(r0 + seg, sh.R);
  int sum = 0;
  for (int r = r0; r < r1; ++r) sum += off[r];
  int x = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int run = x - sum;
  for (int i = 0; i < w; ++i) run += wsum[i];
  for (int r = r0; r < r1; ++r) {
    const int v = off[r];
    off[r] = run;
    run += v;
  }
  // Stable LSD radix sort of the keys by ordinal, 8 bits a pass (two passes
  // when R > 256).  Wave w takes keys 256w .. 256w + 255 in four rounds of
  // 64, so equal ordinals keep their row order.  A key's rank among the
  // round's keys of its digit comes from eight ballots (the lanes whose
  // digit agrees bit by bit); the wave's running count per digit sits in
  // LDS; one block-wide scan over (digit, wave), digit-major, gives each
  // wave's first slot per digit.
  constexpr int NW = kGroupThreads / 64;
  static_assert(NW * 256 == 4 * kGroupThreads, "one scan entry per (digit, wave), four per thread");
  const uint64_t lanes_below = (1ull << lane) - 1ull;
#pragma unroll
  for (int e = 0; e < 4; ++e) keys[0][4 * tid + e] = k[e];
  const int passes = sh.R > 256 ? 2 : 1;
  for (int pass = 0; pass < passes; ++pass) {
    const uint32_t* src = keys[pass & 1];
    uint32_t* dst = keys[(pass + 1) & 1];
    const int shift = 12 + 8 * pass;
#pragma unroll
    for (int e = 0; e < 4; ++e) (&wcnt[0][0])[4 * tid + e] = 0;
    __syncthreads();
    int dg[4], rk[4];
    uint32_t kv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      kv[u] = src[256 * w + 64 * u + lane];
      const int d = (int)((kv[u] >> shift) & 255u);
      uint64_t m = ~0ull;
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const uint64_t bal = __ballot((d >> b) & 1);
        m &= ((d >> b) & 1) ? bal : ~bal;
      }
      const int r = __popcll(m & lanes_below);
      const int base = wcnt[w][d];
      if (r == 0) wcnt[w][d] = base + __popcll(m);
      dg[u] = d;
      rk[u] = base + r;
    }
    __syncthreads();
    int c4[4], s4 = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int f = 4 * tid + e;
      c4[e] = wcnt[f % NW][f / NW];
      s4 += c4[e];
    }
    int xs = s4;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(xs, o, 64);
      if (lane >= o) xs += y;
    }
    if (lane == 63) wsum[w] = xs;
    __syncthreads();
    int pre = xs - s4;
    for (int i = 0; i < w; ++i) pre += wsum[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int f = 4 * tid + e;
      wcnt[f % NW][f / NW] = pre;
      pre += c4[e];
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) dst[wcnt[w][dg[u]] + rk[u]] = kv[u];
    __syncthreads();
  }
  const uint32_t* key = keys[passes & 1];
#pragma unroll
  for (int e = 0; e < 4; ++e) k[e] = key[4 * tid + e];
  // Sorted entry i: its rank among the piece's rows of the same ordinal is
  // i minus the ordinal's first sorted entry (binary search).  The searches
  // run first, then every load, then the stores.
  const int* before = a.gcnt + ((size_t)head * gridDim.x + p) * sh.R;
  int first[4];
  uint32_t o[4];
  int row[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = 4 * tid + e;
    o[e] = min(k[e] >> 12, (uint32_t)sh.R - 1u);
    row[e] = (int)(k[e] & 4095u);
    int lo = 0, hi = min(i, len);
    while (lo < hi) {
      const int m = (lo + hi) >> 1;
      if ((key[m] >> 12) < o[e]) lo = m + 1;
      else hi = m;
    }
    first[e] = lo;
  }
  int bef[4];
  IdxT kord[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    bef[e] = before[o[e]];
    kord[e] = kin[min(row[e], len - 1)];
  }
  IdxT* kout = (IdxT*)a.idx_out + (size_t)(2 * head) * sh.Nc;
  IdxT* vout = kout + sh.Nc;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = 4 * tid + e;
    if (i < len) {
      const int slot = off[o[e]] + bef[e] + (i - first[e]);
      a.perm[(size_t)head * sh.Nc + n0 + row[e]] = slot;
      kout[slot] = kord[e];
      vout[slot] = (IdxT)o[e];
    }
  }
}

template <int D>
hipError_t launch_compress_d(const Shape& sh, const CompressArgs& a, hipStream_t st) {
  const int ns = sh.n_streams();
  const int chunks = mean_chunks(sh);
  const int rpb = 256 / (D / 8);   // references per k_center_refs block
  const dim3 g_mean(chunks, ns), g_ref((sh.R + rpb - 1) / rpb, ns);
  const dim3 g_search(xcd_grid(ns, (sh.T + kSearchTok - 1) / kSearchTok)), g_search32((sh.T + 255) / 256, ns);
  const dim3 g_enc(xcd_grid(ns, (sh.N + 64 * kEncTiles - 1) / (64 * kEncTiles))), g_enc32((sh.N + 255) / 256, ns);
  void* const* ev = a.events;
  hipError_t e;
#define DKV_TRY(x)                         \
  do {                                     \
    if ((e = (x)) != hipSuccess) return e; \
  } while (0)
  // Grouped layouts: count, scan and place between the search and the
  // encode (timed as the start of the encode stage).
  const int heads = sh.B * sh.H, pieces = group_pieces(sh);
  auto group = [&]() -> hipError_t {
    DKV_TRY(launch_lds(k_group_count, dim3(pieces, heads), kGroupThreads, (size_t)sh.R * 4, st, ev_start(ev, 3),
                       nullptr, a, sh));
    DKV_TRY(launch(k_group_scan, dim3((sh.R + 255) / 256, heads), 256, st, nullptr, nullptr, a, sh, pieces));
    DKV_TRY(launch_lds(sh.idx_bytes == 2 ? k_group_place<uint16_t> : k_group_place<uint32_t>, dim3(pieces, heads),
                       kGroupThreads, (size_t)sh.R * 4, st, nullptr, nullptr, a, sh));
    return hipSuccess;
  };
  hipEvent_t enc_start = ev_start(ev, 3);
  if (sh.grouped) enc_start = nullptr;
  if (sh.bf16) {
    DKV_TRY(launch(k_mean_partial<BF16>, g_mean, 256, st, ev_start(ev, 0), nullptr, a, sh));
    DKV_TRY(launch(k_mean_final<BF16>, ns, 256, st, nullptr, ev_stop(ev, 0), a, sh, chunks));
    DKV_TRY(launch(k_center_refs<BF16>, g_ref, 256, st, ev_start(ev, 1), ev_stop(ev, 1), a, sh));
    if (sh.N > 0) {
      if (sh.topk_search()) {
        // Lists of 1, 4 or 8 entries (at least k).
        auto kern = sh.l2 ? (sh.K == 1 ? k_search_topk_mfma<D, 1, true>
                             : sh.K <= 4 ? k_search_topk_mfma<D, 4, true>
                                         : k_search_topk_mfma<D, 8, true>)
                          : (sh.K <= 4 ? k_search_topk_mfma<D, 4, false> : k_search_topk_mfma<D, 8, false>);
        DKV_TRY(launch(kern, g_search, kSearchThreads, st, ev_start(ev, 2), ev_stop(ev, 2), a, sh));
      } else {
        DKV_TRY(launch(k_search_mfma<D>, g_search, kSearchThreads, st, ev_start(ev, 2), ev_stop(ev, 2), a, sh));
      }
      if (sh.grouped) DKV_TRY(group());
      if (sh.q4) {
        DKV_TRY(launch_lds(k_encode_mfma<D, true>, g_enc, 256, (size_t)sh.dc * (D + 8) * 2, st, enc_start,
                           ev_stop(ev, 3), a, sh));
      } else {
        DKV_TRY(launch_lds(k_encode_mfma<D, false>, g_enc, 256, (size_t)sh.dc * (D + 8) * 2, st, enc_start,
                           ev_stop(ev, 3), a, sh));
      }
    }
  } else {
    DKV_TRY(launch(k_mean_partial<F32>, g_mean, 256, st, ev_start(ev, 0), nullptr, a, sh));
    DKV_TRY(launch(k_mean_final<F32>, ns, 256, st, nullptr, ev_stop(ev, 0), a, sh, chunks));
    DKV_TRY(launch(k_center_refs<F32>, g_ref, 256, st, ev_start(ev, 1), ev_stop(ev, 1), a, sh));
    if (sh.N > 0) {
      if (sh.topk_search()) {
        DKV_TRY(launch(k_search_topk_f32<D>, dim3((sh.N + 255) / 256, ns), 256, st, ev_start(ev, 2), ev_stop(ev, 2),
                       a, sh));
      } else {
        DKV_TRY(launch(k_search_f32<D>, g_search32, 256, st, ev_start(ev, 2), ev_stop(ev, 2), a, sh));
      }
      if (sh.grouped) DKV_TRY(group());
      DKV_TRY(launch(k_encode_f32<D>, g_enc32, 256, st, enc_start, ev_stop(ev, 3), a, sh));
    }
  }
  if (sh.N == 0 && ev) {
    // No coded tokens: the search and encode stages are empty.
    for (int i = 2; i < 4; ++i) {
      DKV_TRY(hipEventRecord(ev_start(ev, i), st));
      DKV_TRY(hipEventRecord(ev_stop(ev, i), st));
    }
  }
#undef DKV_TRY
  return hipSuccess;
}

}  // namespace

hipError_t launch_compress(const Shape& sh, const CompressArgs& a, hipStream_t st) {
  return sh.d == 128 ? launch_compress_d<128>(sh, a, st) : launch_compress_d<64>(sh, a, st);
}

}  // namespace dkv
