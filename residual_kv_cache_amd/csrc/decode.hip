// DeltaKV decode attention over the compressed cache, gfx950.
//
// Attention of one query per sequence over every cached token as if each
// were reconstructed, k^_t = mu + ref + W_up code (DeltaKV explainer,
// English page, Technical Summary §3 "Reconstruction": KV^ = f_d(z) + KV^R),
// without materialising k^ or v^:
//
//   q . k^_t = q . mu_K + q . refs_K[ref(t)] + (W_up_K^T q) . code_K(t)
//
// The first term is the same for every token and cancels in the softmax, so
// mu_K is never read.  With S[r][g] = scale * <q_g, refs_K[r]> (one pass over
// the key references) and q'_g = scale * W_up_K^T q_g, a coded token scores
// S[ref_K(t)][g] + <q'_g, code_K(t)>, and a reference token r scores
// S[r][g].  On the value side
//
//   sum_t p_t v^_t = mu_V + sum_t p_t refs_V[ref_V(t)] + W_up_V sum_t p_t code_V(t)
//
// so each split keeps, per query head, an online-softmax state (max m, sum
// l) and two accumulators: acc_r over value references (head dim) and acc_c
// over value codes (code dim).  A final pass merges the splits and applies
// mu_V and W_up_V once per query head.  All arithmetic is fp32; scores are
// kept in base-2 units (scale * log2 e) so the exponentials are exp2.
//
// Kernels: refscore (S and q'), split (the token stream), combine.  This is
// the general path (float32 storage, head dim 64, more than 4 query heads
// per KV head, code dim 64..128); the common bfloat16 shapes take the MFMA
// kernels of decode_mfma.hip.

#include "dkv_device.h"
#include "dkv_internal.h"

namespace dkv {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <class S>
__device__ __forceinline__ float ld(const void* p, size_t i) {
  return S::load(((const typename S::T*)p)[i]);
}

// ---------------------------------------------------------------------------
// refscore: S[b][h][r][g] (row stride score_cols(G)) for 64 references per block, and q'[b][h][g][:]
// from the first block of each (b, h).  grid (ceil(R/64), B*H), block 256.
// ---------------------------------------------------------------------------

template <class S, int D>
__global__ __launch_bounds__(256) void k_refscore(DecodeArgs a, Shape sh) {
  __shared__ float qs[16][D];
  __shared__ float rs[64][D + 1];
  const int bh = blockIdx.y;
  const int b = bh / sh.H, h = bh % sh.H;
  const int G = a.G;
  const float sc = a.scale * kLog2e;
  for (int p = threadIdx.x; p < G * D; p += 256) {
    const int g = p / D, i = p % D;
    qs[g][i] = ld<S>(a.q, ((size_t)b * a.Hq + h * G + g) * D + i) * sc;
  }
  const int r0 = blockIdx.x * 64;
  const size_t rbase = ((size_t)bh * 2 + 0) * sh.Rc;  // K references of (b, h)
  for (int p = threadIdx.x; p < 64 * D; p += 256) {
    const int row = p / D, i = p % D;
    rs[row][i] = r0 + row < sh.R ? ld<S>(a.refs, (rbase + r0 + row) * D + i) : 0.f;
  }
  __syncthreads();
  for (int p = threadIdx.x; p < 64 * G; p += 256) {
    const int row = p / G, g = p % G;
    if (r0 + row >= sh.R) continue;
    float acc = 0.f;
#pragma unroll 8
    for (int i = 0; i < D; ++i) acc = fmaf(qs[g][i], rs[row][i], acc);
    a.score[((size_t)bh * sh.R + r0 + row) * score_cols(G) + g] = acc;
  }
  if (blockIdx.x == 0) {
    const typename S::T* wu = (const typename S::T*)a.wuk + (size_t)h * a.w_hs;
    for (int p = threadIdx.x; p < G * sh.dc; p += 256) {
      const int g = p / sh.dc, j = p % sh.dc;
      float acc = 0.f;
      for (int i = 0; i < D; ++i) acc = fmaf(qs[g][i], S::load(wu[(size_t)i * sh.dc + j]), acc);
      a.qp[((size_t)bh * G + g) * sh.dc + j] = acc;
    }
  }
}

// ---------------------------------------------------------------------------
// split: one block per (split, b, h); 4 waves take 64-token chunks in turn.
// Coded rows [n0, n1) and reference tokens [r0, r1) of the split.
// Score phase: lane = token.  Accumulate phase: the wave walks the chunk's
// tokens; lanes own head-dim columns (acc_r) and code columns (acc_c).
// ---------------------------------------------------------------------------

// MK: several references per coded token (top_k > 1): the key score takes
// the mean of their S rows and the value side the mean of their rows.
template <class S, int D, int GP, bool Q4, bool MK>
__global__ __launch_bounds__(256) void k_split_valu(DecodeArgs a, Shape sh) {
  constexpr int KM = MK ? 8 : 1;         // ordinals held per lane
  constexpr int RPL = D / 64;            // head-dim columns per lane
  __shared__ float qp_l[GP][D];
  __shared__ float mw[4][GP];
  __shared__ float merge[GP][2 * D + 1];   // acc_r | acc_c | l
  const int sp = blockIdx.x;
  const int bh = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int G = a.G, dc = sh.dc;
  const int n0 = (int)((int64_t)sh.N * sp / a.splits), n1 = (int)((int64_t)sh.N * (sp + 1) / a.splits);
  const int r0 = (int)((int64_t)sh.R * sp / a.splits), r1 = (int)((int64_t)sh.R * (sp + 1) / a.splits);

  for (int p = threadIdx.x; p < G * dc; p += 256) qp_l[p / dc][p % dc] = a.qp[(size_t)bh * G * dc + p];
  __syncthreads();

  const size_t sK = (size_t)bh * 2, sV = sK + 1;             // stream ids
  const int Gs = score_cols(G);
  const float* score = a.score + (size_t)bh * sh.R * Gs;
  const typename S::T* refsV = (const typename S::T*)a.refs + sV * sh.Rc * D;
  const typename S::T* codesK = (const typename S::T*)a.codes + sK * sh.Nc * dc;
  const typename S::T* codesV = (const typename S::T*)a.codes + sV * sh.Nc * dc;
  // 4-bit codes: rows of d_c / 2 bytes and one scale per row.
  const uint8_t* qK = (const uint8_t*)a.codes + sK * sh.Nc * (dc / 2);
  const uint8_t* qV = (const uint8_t*)a.codes + sV * sh.Nc * (dc / 2);

  float m[GP], lsum[GP], accr[GP][RPL], accc[GP][2];
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    m[g] = -INFINITY; lsum[g] = 0.f;
#pragma unroll
    for (int e = 0; e < RPL; ++e) accr[g][e] = 0.f;
    accc[g][0] = accc[g][1] = 0.f;
  }

  const int nc_codes = (n1 - n0 + 63) / 64;
  const int nc_refs = (r1 - r0 + 63) / 64;
  for (int c = wave; c < nc_codes + nc_refs; c += 4) {
    const bool coded = c < nc_codes;
    const int base = coded ? n0 + c * 64 : r0 + (c - nc_codes) * 64;
    const int end = coded ? n1 : r1;
    const int cnt = min(64, end - base);
    const int u = base + lane;
    const bool valid = lane < cnt;
    int rk = 0, rv = 0;
    int rvs[KM];   // MK: the token's value ordinals
    int nref = 1;  // references the token averages
    float sc[GP];
    if (valid) {
      if (coded && !MK) {
        // Ordinals come from caller memory: clamp so a corrupt cache can never
        // address outside the reference arrays.
        rk = min((int)load_idx(a.idx, sK * sh.Nc + u, sh.idx_bytes), sh.R - 1);
        rv = min((int)load_idx(a.idx, sV * sh.Nc + u, sh.idx_bytes), sh.R - 1);
      } else if (!coded) {
        rk = rv = u;
      }
      if constexpr (MK) {
        rvs[0] = rv;
#pragma unroll
        for (int j = 1; j < KM; ++j) rvs[j] = 0;
      }
      if (coded && MK) {
        const int t = slot_to_pos(u, sh.s);
        nref = min(sh.K, t / sh.s + 1);
        const size_t ib = (sK * sh.Nc + u) * sh.K, jb = (sV * sh.Nc + u) * sh.K;
        float ssum[GP];
#pragma unroll
        for (int g = 0; g < GP; ++g) ssum[g] = 0.f;
#pragma unroll
        for (int j = 0; j < KM; ++j) {
          if (j < nref) {
            const int kj = min((int)load_idx(a.idx, ib + j, sh.idx_bytes), sh.R - 1);
            rvs[j] = min((int)load_idx(a.idx, jb + j, sh.idx_bytes), sh.R - 1);
#pragma unroll
            for (int g = 0; g < GP; ++g) ssum[g] += g < G ? score[(size_t)kj * Gs + g] : 0.f;
          }
        }
        const float inv = 1.0f / (float)nref;
#pragma unroll
        for (int g = 0; g < GP; ++g) sc[g] = g < G ? ssum[g] * inv : -INFINITY;
      } else {
#pragma unroll
        for (int g = 0; g < GP; ++g) sc[g] = g < G ? score[(size_t)rk * Gs + g] : -INFINITY;
      }
      if (coded) {
        if constexpr (Q4) {
          const uint32_t* row = (const uint32_t*)(qK + (size_t)u * (dc / 2));
          const float scl = ld<S>(a.scales, sK * sh.Nc + u);
          float cd[GP];
#pragma unroll
          for (int g = 0; g < GP; ++g) cd[g] = 0.f;
          for (int w = 0; w < dc / 8; ++w) {
            const uint32_t word = row[w];
#pragma unroll
            for (int k2 = 0; k2 < 8; ++k2) {
              const float cj = q4_at(word, k2);
#pragma unroll
              for (int g = 0; g < GP; ++g) cd[g] = fmaf(qp_l[g][8 * w + k2], cj, cd[g]);
            }
          }
#pragma unroll
          for (int g = 0; g < GP; ++g) sc[g] = fmaf(scl, cd[g], sc[g]);
        } else {
          for (int j = 0; j < dc; ++j) {
            const float cj = S::load(codesK[(size_t)u * dc + j]);
#pragma unroll
            for (int g = 0; g < GP; ++g) sc[g] = fmaf(qp_l[g][j], cj, sc[g]);
          }
        }
      }
    } else {
#pragma unroll
      for (int g = 0; g < GP; ++g) sc[g] = -INFINITY;
    }
    float p[GP];
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      if (g >= G) { p[g] = 0.f; continue; }
      const float mn = fmaxf(m[g], wave_max(sc[g]));
      const float alpha = exp2f(m[g] - mn);   // m = -inf on the first chunk -> 0
      p[g] = exp2f(sc[g] - mn);
      m[g] = mn;
      lsum[g] = lsum[g] * alpha + p[g];
#pragma unroll
      for (int e = 0; e < RPL; ++e) accr[g][e] *= alpha;
      accc[g][0] *= alpha;
      accc[g][1] *= alpha;
    }
    for (int k = 0; k < cnt; ++k) {
      float xr[RPL];
      if constexpr (MK) {
        // the mean of the token's value references
        const int nk = __builtin_amdgcn_readlane(nref, k);
#pragma unroll
        for (int e = 0; e < RPL; ++e) xr[e] = 0.f;
#pragma unroll
        for (int j = 0; j < KM; ++j) {
          if (j < nk) {
            const int r = __builtin_amdgcn_readlane(rvs[j], k);
#pragma unroll
            for (int e = 0; e < RPL; ++e) xr[e] += S::load(refsV[(size_t)r * D + lane * RPL + e]);
          }
        }
        const float inv = 1.0f / (float)nk;
#pragma unroll
        for (int e = 0; e < RPL; ++e) xr[e] = nk > 1 ? xr[e] * inv : xr[e];
      } else {
        const int r = __builtin_amdgcn_readlane(rv, k);
#pragma unroll
        for (int e = 0; e < RPL; ++e) xr[e] = S::load(refsV[(size_t)r * D + lane * RPL + e]);
      }
      float c0 = 0.f, c1 = 0.f;
      if (coded) {
        if constexpr (Q4) {
          const uint8_t* row = qV + (size_t)(base + k) * (dc / 2);
          const float scl = ld<S>(a.scales, sV * sh.Nc + base + k);
          if (lane < dc) c0 = scl * (float)((int32_t)((uint32_t)row[lane >> 1] << (24 + 4 * (1 - (lane & 1)))) >> 28);
          if (lane + 64 < dc)
            c1 = scl * (float)((int32_t)((uint32_t)row[(lane + 64) >> 1] << (24 + 4 * (1 - (lane & 1)))) >> 28);
        } else {
          const size_t row = (size_t)(base + k) * dc;
          if (lane < dc) c0 = S::load(codesV[row + lane]);
          if (lane + 64 < dc) c1 = S::load(codesV[row + lane + 64]);
        }
      }
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        if (g >= G) continue;   // continue, not break: a loop with a break is not unrolled
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p[g]), k));
#pragma unroll
        for (int e = 0; e < RPL; ++e) accr[g][e] = fmaf(w, xr[e], accr[g][e]);
        accc[g][0] = fmaf(w, c0, accc[g][0]);
        accc[g][1] = fmaf(w, c1, accc[g][1]);
      }
    }
  }

  // Merge the four waves in a fixed order.
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    lsum[g] = wave_sum(lsum[g]);
    if (lane == 0) mw[wave][g] = m[g];
  }
  __syncthreads();
  float mb[GP], wgt[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    mb[g] = fmaxf(fmaxf(mw[0][g], mw[1][g]), fmaxf(mw[2][g], mw[3][g]));
    wgt[g] = m[g] == -INFINITY ? 0.f : exp2f(m[g] - mb[g]);
  }
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int e = 0; e < RPL; ++e) {
          const int i = lane * RPL + e;
          const float v = accr[g][e] * wgt[g];
          merge[g][i] = w == 0 ? v : merge[g][i] + v;
        }
        if (lane < dc) merge[g][D + lane] = (w == 0 ? 0.f : merge[g][D + lane]) + accc[g][0] * wgt[g];
        if (lane + 64 < dc) merge[g][D + lane + 64] = (w == 0 ? 0.f : merge[g][D + lane + 64]) + accc[g][1] * wgt[g];
        if (lane == 0) merge[g][2 * D] = (w == 0 ? 0.f : merge[g][2 * D]) + lsum[g] * wgt[g];
      }
    }
    __syncthreads();
  }
  const int rec = partial_rec(sh);
  float* out = a.part + ((size_t)bh * a.splits + sp) * G * rec;
  for (int p = threadIdx.x; p < G * rec; p += 256) {
    const int g = p / rec, f = p % rec;
    float v = 0.f;
    if (f == 0) {
      v = fmaxf(fmaxf(mw[0][g], mw[1][g]), fmaxf(mw[2][g], mw[3][g]));
    } else if (f == 1) {
      v = merge[g][2 * D];
    } else if (f < 2 + dc) {
      v = merge[g][D + f - 2];
    } else if (f < 2 + dc + D) {
      v = merge[g][f - 2 - dc];
    }
    out[p] = v;
  }
}

// ---------------------------------------------------------------------------
// split over a token list (selective decode): one block per (split, b, h);
// the split takes list entries [i0, i1) of sequence b, and its 4 waves take
// 64-entry chunks in turn.  Score phase: lane = entry, whose position t is
// either a reference (t mod s = 0: row t / s, no code) or coded row
// t - t/s - 1; entries at or past T score -inf.  Accumulate phase as in
// k_split_valu, eight entries at a time so that their value rows are loaded
// together.  Partials have the k_split_valu layout.
// ---------------------------------------------------------------------------

// Zeros standing in for the code and ordinal rows of streams that hold no
// coded token, so that the loads of k_split_sel need no condition.
__device__ const uint32_t kZeroRow[64] __attribute__((aligned(16))) = {0u};

// n consecutive storage elements as floats (n = 1 or 2).
template <class S, int N>
__device__ __forceinline__ void load_cols(const typename S::T* p, float (&v)[N]) {
  if constexpr (N == 2 && sizeof(typename S::T) == 2) {
    const uint32_t w = *(const __attribute__((address_space(1))) uint32_t*)p;
    v[0] = __uint_as_float(w << 16);
    v[1] = __uint_as_float(w & 0xFFFF0000u);
  } else if constexpr (N == 2) {
    const u32x2 w = *(const __attribute__((address_space(1))) u32x2*)p;
    v[0] = __uint_as_float(w[0]);
    v[1] = __uint_as_float(w[1]);
  } else {
    v[0] = S::load(*(const __attribute__((address_space(1))) typename S::T*)p);
  }
}

template <class S, int D, int GP, typename IdxT, bool Q4, bool MK>
__global__ __launch_bounds__(256) void k_split_sel(DecodeArgs a, Shape sh) {
  constexpr int RPL = D / 64;            // head-dim columns per lane
  constexpr int UN = MK ? 8 : 16;        // entries per accumulate step
  constexpr int KM = MK ? 8 : 1;         // ordinals held per lane (MK: top_k > 1)
  typedef typename S::T T;
  __shared__ float qp_l[GP][128];
  __shared__ float mw[4][GP];
  __shared__ float merge[GP][2 * D + 1];   // acc_r | acc_c | l
  const int sp = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / sh.H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int G = a.G, dc = sh.dc;
  const int i0 = (int)((int64_t)a.n_sel * sp / a.splits), i1 = (int)((int64_t)a.n_sel * (sp + 1) / a.splits);
  const uint32_t* sel = a.sel + (size_t)b * a.n_sel;

  // q' of the head's query heads; zero past d_c and past G.
  for (int p = threadIdx.x; p < GP * 128; p += 256) {
    const int g = p >> 7, j = p & 127;
    qp_l[g][j] = g < G && j < dc ? a.qp[((size_t)bh * G + g) * dc + j] : 0.f;
  }
  __syncthreads();

  const size_t sK = (size_t)bh * 2, sV = sK + 1;
  const int Gs = score_cols(G);
  const float* score = a.score + (size_t)bh * sh.R * Gs;
  const T* refsV = (const T*)a.refs + sV * sh.Rc * D;
  // Without coded tokens every entry is a reference: codes and ordinals come
  // from the zero row (row 0, stride 0).
  const bool has_codes = sh.N > 0;
  const int cstride = has_codes ? dc : 0;
  const T* codesK = has_codes ? (const T*)a.codes + sK * sh.Nc * dc : (const T*)kZeroRow;
  const T* codesV = has_codes ? (const T*)a.codes + sV * sh.Nc * dc : (const T*)kZeroRow;
  const IdxT* idxK = has_codes ? (const IdxT*)a.idx + sK * sh.Nc * sh.K : (const IdxT*)kZeroRow;
  const IdxT* idxV = has_codes ? (const IdxT*)a.idx + sV * sh.Nc * sh.K : (const IdxT*)kZeroRow;
  // 4-bit codes: rows of d_c / 2 bytes (stride 0 on the zero row) and scales.
  const int qstride = has_codes ? dc / 2 : 0;
  const uint8_t* qK = has_codes ? (const uint8_t*)a.codes + sK * sh.Nc * (dc / 2) : (const uint8_t*)kZeroRow;
  const uint8_t* qV = has_codes ? (const uint8_t*)a.codes + sV * sh.Nc * (dc / 2) : (const uint8_t*)kZeroRow;
  const T* sclK = has_codes && Q4 ? (const T*)a.scales + sK * sh.Nc : (const T*)kZeroRow;
  const T* sclV = has_codes && Q4 ? (const T*)a.scales + sV * sh.Nc : (const T*)kZeroRow;

  float m[GP], lsum[GP], accr[GP][RPL], accc[GP][2];
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    m[g] = -INFINITY; lsum[g] = 0.f;
#pragma unroll
    for (int e = 0; e < RPL; ++e) accr[g][e] = 0.f;
    accc[g][0] = accc[g][1] = 0.f;
  }

  const int cl0 = min(lane, dc - 1), cl1 = min(lane + 64, dc - 1);
  const int nchunks = (i1 - i0 + 63) / 64;
  for (int c = wave; c < nchunks; c += 4) {
    const int base = i0 + c * 64;
    const int cnt = min(64, i1 - base);
    // ---- scores: lane = entry ----
    const uint32_t t = sel[base + min(lane, cnt - 1)];
    const bool valid = lane < cnt && t < (uint32_t)sh.T;
    const int tt = valid ? (int)t : 0;
    const int r = tt / sh.s;
    const bool coded = valid && tt - r * sh.s != 0;
    const int u = coded ? tt - r - 1 : 0;     // coded row (0 when unused)
    // Ordinals come from caller memory: clamp so a corrupt cache can never
    // address outside the reference arrays.
    const int KK = MK ? sh.K : 1;
    const int nref = coded && MK ? min(sh.K, tt / sh.s + 1) : 1;
    int iks[KM], ivs[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      iks[j] = min((int)idxK[(size_t)u * KK + (j < nref ? j : 0)], sh.R - 1);
      ivs[j] = min((int)idxV[(size_t)u * KK + (j < nref ? j : 0)], sh.R - 1);
    }
    const int ik = iks[0], iv = ivs[0];
    float cd[GP];
#pragma unroll
    for (int g = 0; g < GP; ++g) cd[g] = 0.f;
    // Key-code dot products, 32 columns per trip: four 8-column loads go out
    // together (column blocks past d_c re-read the last block and meet the
    // zero q' columns).
    for (int j0 = 0; j0 < dc; j0 += 32) {
      float cv[4][8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int jj = has_codes ? min(j0 + 8 * q, dc - 8) : 0;
        if constexpr (Q4) {
          const uint32_t word = *(const __attribute__((address_space(1))) uint32_t*)(qK + (size_t)u * qstride + jj / 2);
#pragma unroll
          for (int i = 0; i < 8; ++i) cv[q][i] = q4_at(word, i);
        } else {
          load8<S>(codesK + (size_t)u * cstride + jj, cv[q]);
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int g = 0; g < GP; ++g)
#pragma unroll
          for (int i = 0; i < 8; ++i) cd[g] = fmaf(qp_l[g][j0 + 8 * q + i], cv[q][i], cd[g]);
    }
    if constexpr (Q4) {
      const float scl = S::load(sclK[u]);
#pragma unroll
      for (int g = 0; g < GP; ++g) cd[g] *= scl;
    }
    const int rk = coded ? ik : r, rv = coded ? iv : r;
    // The entry's S row, four columns per 16-byte load (rows hold Gs >= 4
    // columns; blocks past Gs re-read the last block, unused).
    constexpr int NQ = (GP + 3) / 4;
    f32x4 srow[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      srow[q] = *(const __attribute__((address_space(1))) f32x4*)(score + (size_t)rk * Gs + min(4 * q, Gs - 4));
    if constexpr (MK) {   // the mean of the entry's S rows
#pragma unroll
      for (int j = 1; j < KM; ++j) {
        if (j < nref) {
#pragma unroll
          for (int q = 0; q < NQ; ++q)
            srow[q] += *(const __attribute__((address_space(1))) f32x4*)(score + (size_t)iks[j] * Gs +
                                                                         min(4 * q, Gs - 4));
        }
      }
      const float inv = 1.0f / (float)nref;
#pragma unroll
      for (int q = 0; q < NQ; ++q) srow[q] = nref > 1 ? srow[q] * inv : srow[q];
    }
    float sc[GP];
#pragma unroll
    for (int g = 0; g < GP; ++g)
      sc[g] = valid && g < G ? srow[g >> 2][g & 3] + (coded ? cd[g] : 0.f) : -INFINITY;

    float p[GP];
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      if (g >= G) { p[g] = 0.f; continue; }
      const float mn = fmaxf(m[g], wave_max(sc[g]));
      if (mn == -INFINITY) { p[g] = 0.f; continue; }   // nothing valid yet
      const float alpha = exp2f(m[g] - mn);           // m = -inf on the first valid chunk -> 0
      p[g] = exp2f(sc[g] - mn);
      m[g] = mn;
      lsum[g] = lsum[g] * alpha + p[g];
#pragma unroll
      for (int e = 0; e < RPL; ++e) accr[g][e] *= alpha;
      accc[g][0] *= alpha;
      accc[g][1] *= alpha;
    }
    const int ucol = coded ? u : -1;   // coded row, or -1 for a reference entry

    // ---- accumulate: the wave walks the chunk's entries, UN at a time ----
    for (int k0 = 0; k0 < cnt; k0 += UN) {
      float xr[UN][RPL], c0[UN], c1[UN];
#pragma unroll
      for (int i = 0; i < UN; ++i) {
        const int k = min(k0 + i, cnt - 1);
        const int rr = __builtin_amdgcn_readlane(rv, k);
        const int uu = max(__builtin_amdgcn_readlane(ucol, k), 0);
        load_cols<S, RPL>(refsV + (size_t)rr * D + lane * RPL, xr[i]);
        if constexpr (MK) {   // the mean of the entry's value references
          const int nk = __builtin_amdgcn_readlane(nref, k);
#pragma unroll
          for (int j = 1; j < KM; ++j) {
            if (j < nk) {
              float xj[RPL];
              load_cols<S, RPL>(refsV + (size_t)__builtin_amdgcn_readlane(ivs[j], k) * D + lane * RPL, xj);
#pragma unroll
              for (int e = 0; e < RPL; ++e) xr[i][e] += xj[e];
            }
          }
          const float inv = 1.0f / (float)nk;
#pragma unroll
          for (int e = 0; e < RPL; ++e) xr[i][e] = nk > 1 ? xr[i][e] * inv : xr[i][e];
        }
        if constexpr (Q4) {
          const uint8_t* row = qV + (size_t)uu * qstride;
          const float scl = S::load(sclV[uu]);
          const uint32_t b0 = has_codes ? row[cl0 >> 1] : 0u, b1 = has_codes ? row[cl1 >> 1] : 0u;
          c0[i] = scl * (float)((int32_t)(b0 << (24 + 4 * (1 - (cl0 & 1)))) >> 28);
          c1[i] = scl * (float)((int32_t)(b1 << (24 + 4 * (1 - (cl1 & 1)))) >> 28);
        } else {
          float t0[1], t1[1];
          load_cols<S, 1>(codesV + (size_t)uu * cstride + (has_codes ? cl0 : 0), t0);
          load_cols<S, 1>(codesV + (size_t)uu * cstride + (has_codes ? cl1 : 0), t1);
          c0[i] = t0[0];
          c1[i] = t1[0];
        }
      }
#pragma unroll
      for (int i = 0; i < UN; ++i) {
        const int k = k0 + i;
        if (k >= cnt) break;
        const bool ck = __builtin_amdgcn_readlane(ucol, k) >= 0;
        const float v0 = ck && lane < dc ? c0[i] : 0.f;
        const float v1 = ck && lane + 64 < dc ? c1[i] : 0.f;
#pragma unroll
        for (int g = 0; g < GP; ++g) {
          if (g >= G) continue;
          const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p[g]), k));
#pragma unroll
          for (int e = 0; e < RPL; ++e) accr[g][e] = fmaf(w, xr[i][e], accr[g][e]);
          accc[g][0] = fmaf(w, v0, accc[g][0]);
          accc[g][1] = fmaf(w, v1, accc[g][1]);
        }
      }
    }
  }

  // Merge the four waves in a fixed order.
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    lsum[g] = wave_sum(lsum[g]);
    if (lane == 0) mw[wave][g] = m[g];
  }
  __syncthreads();
  float mb[GP], wgt[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    mb[g] = fmaxf(fmaxf(mw[0][g], mw[1][g]), fmaxf(mw[2][g], mw[3][g]));
    wgt[g] = m[g] == -INFINITY ? 0.f : exp2f(m[g] - mb[g]);
  }
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int e = 0; e < RPL; ++e) {
          const int i = lane * RPL + e;
          const float v = accr[g][e] * wgt[g];
          merge[g][i] = w == 0 ? v : merge[g][i] + v;
        }
        if (lane < dc) merge[g][D + lane] = (w == 0 ? 0.f : merge[g][D + lane]) + accc[g][0] * wgt[g];
        if (lane + 64 < dc) merge[g][D + lane + 64] = (w == 0 ? 0.f : merge[g][D + lane + 64]) + accc[g][1] * wgt[g];
        if (lane == 0) merge[g][2 * D] = (w == 0 ? 0.f : merge[g][2 * D]) + lsum[g] * wgt[g];
      }
    }
    __syncthreads();
  }
  const int rec = partial_rec(sh);
  float* out = a.part + ((size_t)bh * a.splits + sp) * G * rec;
  for (int p = threadIdx.x; p < G * rec; p += 256) {
    const int g = p / rec, f = p % rec;
    float v = 0.f;
    if (f == 0) {
      v = fmaxf(fmaxf(mw[0][g], mw[1][g]), fmaxf(mw[2][g], mw[3][g]));
    } else if (f == 1) {
      v = merge[g][2 * D];
    } else if (f < 2 + dc) {
      v = merge[g][D + f - 2];
    } else if (f < 2 + dc + D) {
      v = merge[g][f - 2 - dc];
    }
    out[p] = v;
  }
}

// ---------------------------------------------------------------------------
// combine: one block per (b, query head); merges the splits, then
// out = mu_V + (acc_r + W_up_V acc_c) / l.  grid B*Hq, block 128.
// ---------------------------------------------------------------------------

template <class S, int D>
__global__ __launch_bounds__(128) void k_combine(DecodeArgs a, Shape sh) {
  __shared__ float accc[128];
  __shared__ float mx_s, l_s;
  const int bq = blockIdx.x;
  const int b = bq / a.Hq, gq = bq % a.Hq;
  const int h = gq / a.G, g = gq % a.G;
  const int bh = b * sh.H + h;
  const int rec = partial_rec(sh);
  const int dc = sh.dc;
  const float* part = a.part + (size_t)bh * a.splits * a.G * rec + (size_t)g * rec;
  const size_t pstride = (size_t)a.G * rec;
  if (threadIdx.x == 0) {
    float mx = -INFINITY;
    for (int s = 0; s < a.splits; ++s) mx = fmaxf(mx, part[s * pstride]);
    float l = 0.f;
    for (int s = 0; s < a.splits; ++s) {
      const float ms = part[s * pstride];
      if (ms != -INFINITY) l += exp2f(ms - mx) * part[s * pstride + 1];
    }
    mx_s = mx;
    l_s = l;
  }
  __syncthreads();
  // l = 0 only when a selective decode attended no token: the output is 0.
  const float mx = mx_s, inv_l = l_s > 0.f ? 1.0f / l_s : 0.f;
  const int i = threadIdx.x;
  if (i < dc) {
    float c = 0.f;
    for (int s = 0; s < a.splits; ++s) {
      const float ms = part[s * pstride];
      if (ms != -INFINITY) c = fmaf(exp2f(ms - mx), part[s * pstride + 2 + i], c);
    }
    accc[i] = c;
  }
  __syncthreads();
  if (i < D) {
    float r = 0.f;
    for (int s = 0; s < a.splits; ++s) {
      const float ms = part[s * pstride];
      if (ms != -INFINITY) r = fmaf(exp2f(ms - mx), part[s * pstride + 2 + dc + i], r);
    }
    const typename S::T* wu = (const typename S::T*)a.wuv + (size_t)h * a.w_hs;
    float u = 0.f;
    for (int j = 0; j < dc; ++j) u = fmaf(S::load(wu[(size_t)i * dc + j]), accc[j], u);
    const float muv = ld<S>(a.mu, ((size_t)bh * 2 + 1) * D + i);
    a.out[((size_t)b * a.Hq + gq) * D + i] = l_s > 0.f ? muv + (r + u) * inv_l : 0.f;
  }
}

template <class S, int D, int GP>
hipError_t launch_split(const Shape& sh, const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(a.splits, sh.B * sh.H);
  const hipEvent_t e0 = ev_start(a.events, 1), e1 = ev_stop(a.events, 1);
  if (sh.K > 1)
    return sh.q4 ? launch(k_split_valu<S, D, GP, true, true>, grid, 256, st, e0, e1, a, sh)
                 : launch(k_split_valu<S, D, GP, false, true>, grid, 256, st, e0, e1, a, sh);
  return sh.q4 ? launch(k_split_valu<S, D, GP, true, false>, grid, 256, st, e0, e1, a, sh)
               : launch(k_split_valu<S, D, GP, false, false>, grid, 256, st, e0, e1, a, sh);
}

template <class S, int D>
hipError_t launch_decode_sd(const Shape& sh, const DecodeArgs& a, hipStream_t st) {
  const bool mfma = mfma_side_kernels_supported(sh, a.G, a.splits);
  hipError_t e = mfma ? launch_refscore_mfma(sh, a, st)
                      : launch(k_refscore<S, D>, dim3((sh.R + 63) / 64, sh.B * sh.H), 256, st,
                               ev_start(a.events, 0), ev_stop(a.events, 0), a, sh);
  if (e != hipSuccess) return e;
  if (a.G <= 1) e = launch_split<S, D, 1>(sh, a, st);
  else if (a.G <= 2) e = launch_split<S, D, 2>(sh, a, st);
  else if (a.G <= 4) e = launch_split<S, D, 4>(sh, a, st);
  else if (a.G <= 8) e = launch_split<S, D, 8>(sh, a, st);
  else e = launch_split<S, D, 16>(sh, a, st);
  if (e != hipSuccess) return e;
  if (mfma) return launch_combine_mfma(sh, a, st);
  return launch(k_combine<S, D>, dim3(sh.B * a.Hq), 128, st, ev_start(a.events, 2), ev_stop(a.events, 2), a, sh);
}

template <class S, int D, typename IdxT, bool Q4, bool MK>
hipError_t launch_split_sel_q(const Shape& sh, const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(a.splits, sh.B * sh.H);
  const hipEvent_t e0 = ev_start(a.events, 1), e1 = ev_stop(a.events, 1);
  if (a.G <= 1) return launch(k_split_sel<S, D, 1, IdxT, Q4, MK>, grid, 256, st, e0, e1, a, sh);
  if (a.G <= 2) return launch(k_split_sel<S, D, 2, IdxT, Q4, MK>, grid, 256, st, e0, e1, a, sh);
  if (a.G <= 4) return launch(k_split_sel<S, D, 4, IdxT, Q4, MK>, grid, 256, st, e0, e1, a, sh);
  if (a.G <= 8) return launch(k_split_sel<S, D, 8, IdxT, Q4, MK>, grid, 256, st, e0, e1, a, sh);
  return launch(k_split_sel<S, D, 16, IdxT, Q4, MK>, grid, 256, st, e0, e1, a, sh);
}

template <class S, int D, typename IdxT>
hipError_t launch_split_sel(const Shape& sh, const DecodeArgs& a, hipStream_t st) {
  if (sh.K > 1)
    return sh.q4 ? launch_split_sel_q<S, D, IdxT, true, true>(sh, a, st)
                 : launch_split_sel_q<S, D, IdxT, false, true>(sh, a, st);
  return sh.q4 ? launch_split_sel_q<S, D, IdxT, true, false>(sh, a, st)
               : launch_split_sel_q<S, D, IdxT, false, false>(sh, a, st);
}

template <class S, int D>
hipError_t launch_decode_sel_sd(const Shape& sh, const DecodeArgs& a, hipStream_t st) {
  const bool mfma = mfma_side_kernels_supported(sh, a.G, a.splits);
  hipError_t e = mfma ? launch_refscore_mfma(sh, a, st)
                      : launch(k_refscore<S, D>, dim3((sh.R + 63) / 64, sh.B * sh.H), 256, st,
                               ev_start(a.events, 0), ev_stop(a.events, 0), a, sh);
  if (e != hipSuccess) return e;
  e = sh.idx_bytes == 2 ? launch_split_sel<S, D, uint16_t>(sh, a, st) : launch_split_sel<S, D, uint32_t>(sh, a, st);
  if (e != hipSuccess) return e;
  if (mfma) return launch_combine_mfma(sh, a, st);
  return launch(k_combine<S, D>, dim3(sh.B * a.Hq), 128, st, ev_start(a.events, 2), ev_stop(a.events, 2), a, sh);
}

}  // namespace

hipError_t launch_decode_sel(const Shape& sh, const DecodeArgs& a, hipStream_t st) {
  if (decode_sel_fused_supported(sh, a.G, a.splits)) return launch_decode_sel_fused(sh, a, st);
  if (sh.bf16)
    return sh.d == 128 ? launch_decode_sel_sd<BF16, 128>(sh, a, st) : launch_decode_sel_sd<BF16, 64>(sh, a, st);
  return sh.d == 128 ? launch_decode_sel_sd<F32, 128>(sh, a, st) : launch_decode_sel_sd<F32, 64>(sh, a, st);
}

hipError_t launch_decode(const Shape& sh, const DecodeArgs& a, hipStream_t st) {
  if (decode_fused_supported(sh, a.G, a.splits)) return launch_decode_fused(sh, a, st);
  if (sh.bf16) return sh.d == 128 ? launch_decode_sd<BF16, 128>(sh, a, st) : launch_decode_sd<BF16, 64>(sh, a, st);
  return sh.d == 128 ? launch_decode_sd<F32, 128>(sh, a, st) : launch_decode_sd<F32, 64>(sh, a, st);
}

}  // namespace dkv
