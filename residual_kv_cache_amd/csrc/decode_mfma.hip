// DeltaKV decode attention, fused MFMA kernel (bfloat16 storage, head dim
// 128, up to 4 query heads per KV head, code dim 16..48).
//
// Two kernels per decode step (split, combine).  Attention of query head g over every cached
// token t as if it were reconstructed, k^_t = mu + ref + W_up code (DeltaKV
// explainer, English page, Technical Summary §3 "Reconstruction"):
//
//   score(t) = scale * (q_g . refs_K[ref_K(t)] + (W_up_K^T q_g) . code_K(t))
//   out_g    = mu_V + (sum_t p_t refs_V[ref_V(t)] + W_up_V sum_t p_t code_V(t)) / sum_t p_t
//
// (q_g . mu_K is the same for every token and cancels in the softmax.)  A
// reference token r is a token whose reference is itself and whose code is 0.
//
// Work split: the B*H (sequence, KV head) pairs are split along the sequence
// into `splits` pieces; a 512-thread block (8 waves) owns one piece, each wave
// a contiguous run of 16-token tiles.  Blocks of head bh run on XCD bh % 8
// (workgroups are dispatched to the eight XCDs round-robin), so the gathered
// key and value reference rows of a head stay in one L2.  Each block writes
// an online-softmax partial (max, sum, code and reference accumulators per
// query head); the last block of a head to finish (an atomic arrival count)
// merges the partials and writes the output, then rearms the count.
//
// Per 16-token tile, three MFMA 16x16x32 (bf16 in, fp32 accumulate) chains
// keep every operand lane-local (lane l: n16 = l % 16, q4 = l / 16):
//   scores  C[token][(g, e)]: A = key reference row / key code row of token
//           n16, B = q_g (exact bf16) / q'_g split into bf16 hi + lo;
//           lane l ends with the scores of query head (l%16)/4 for tokens
//           4*q4 + i, i = 0..3 (replicated over e = l % 4)
//   values  C[(g, e)][n] += sum_k P[(g, e)][k] X[k][n], k = (token, e'),
//           P[(g, e)][(token, e')] = p_g(token) if e == e' else 0,
//           X[(token, e')][n] = row(token)[4n + e'] (+ column offset):
//           the weights a lane holds are the ones it feeds (A), and B is
//           whole 8-byte row segments; lane l accumulates query head l/16.
// Softmax weights go in as bf16 hi + lo parts (about 16 significant bits);
// their sum comes from a spare value-code column set to 1.0, so the
// normaliser uses exactly the weights the accumulators used.  The running
// max is raised lazily: only when a score exceeds it by kTau.

#include "dkv_device.h"
#include "dkv_internal.h"

namespace dkv {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kTau = 8.0f;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kD = 128;
constexpr int kMaxDc = 48;

typedef uint32_t Frag __attribute__((ext_vector_type(4)));
typedef uint32_t U32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma16(Frag a, Frag b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
}

// Two floats -> packed bf16 pair, round to nearest even (one instruction).
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

template <typename T>
__device__ __forceinline__ T ldg(const void* base, uint32_t byte_off) {
  return *reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + byte_off);
}

// Reference ordinals of one 16-token tile, loaded one step ahead of the
// tile's data so that the data loads never wait on them.  Coded tiles and
// reference tiles are separate instantiations, so that the loop bodies have
// no control flow (a branch merge would make the compiler drain every
// outstanding load).
struct TileIdx {
  int base, cnt;   // first token (coded row or reference ordinal); valid tokens (0 = dead tile)
  int rkA;         // key reference of score row n16
  int rv[4];       // value references of tokens 4*q4 + i
};

struct Tile {
  Frag kr[4];      // score A: key reference row of token n16, K-steps 0..3
  Frag ck[2];      // score A: key code row of token n16 (coded tiles)
  Frag xv[2][2];   // value B [group][half]: tokens 4*q4 + 2*group + {0,1}
  Frag bc[2];      // value-code B [group] (+ the 1.0 column)
  int cnt;
};

struct Args {
  // per (b, h) stream bases
  const uint16_t* refsK;
  const uint16_t* refsV;
  const uint16_t* codesK;
  const uint16_t* codesV;
  const void* idxK;       // uint16_t or uint32_t ordinals
  const void* idxV;
};

// Tile tt of a run [t0, t1) of 16-token tiles starting at token `first`
// and ending at token `last` (exclusive).  Tiles past t1 are dead: they
// repeat the run's last tile with cnt = 0.
template <bool CODED, typename IdxT>
__device__ __forceinline__ void load_idx(const Args& p, int tt, int t1, int first, int last, int n16, int q4,
                                         TileIdx& ti) {
  const bool live = tt < t1;
  tt = min(tt, t1 - 1);
  const int base = first + tt * 16;
  const int cnt = min(16, last - base);
  ti.base = base;
  ti.cnt = live ? cnt : 0;
  const int ua = base + min(n16, cnt - 1);
  if (CODED) {
    const IdxT* ik = (const IdxT*)p.idxK;
    const IdxT* iv = (const IdxT*)p.idxV;
    ti.rkA = (int)ik[ua];
#pragma unroll
    for (int i = 0; i < 4; ++i) ti.rv[i] = (int)iv[base + min(q4 * 4 + i, cnt - 1)];
  } else {
    ti.rkA = ua;
#pragma unroll
    for (int i = 0; i < 4; ++i) ti.rv[i] = base + min(q4 * 4 + i, cnt - 1);
  }
}

template <bool CODED, int DCK>
__device__ __forceinline__ void load_data(const Args& p, const Shape& sh, const TileIdx& ti, int n16, int q4,
                                          Tile& td) {
  const int dc = sh.dc;
  td.cnt = ti.cnt;
  // Ordinals come from caller memory: clamp so that a corrupt cache can never
  // address outside the reference arrays.
  const uint32_t rkA = (uint32_t)min(ti.rkA, sh.R - 1);
  uint32_t rv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) rv[i] = (uint32_t)min(ti.rv[i], sh.R - 1);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) td.kr[ks] = ldg<Frag>(p.refsK, (rkA * kD + ks * 32 + q4 * 8) * 2u);
#pragma unroll
  for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const U32x2 a = ldg<U32x2>(p.refsV, (rv[2 * g2] * kD + n16 * 8 + hh * 4) * 2u);
      const U32x2 b = ldg<U32x2>(p.refsV, (rv[2 * g2 + 1] * kD + n16 * 8 + hh * 4) * 2u);
      td.xv[g2][hh] = Frag{a.x, a.y, b.x, b.y};
    }
  // Spare value-code column (the first past d_c) accumulates the weights.
  const bool ones = n16 * 4 == dc;
  const Frag one_col = Frag{ones ? 0x3F80u : 0u, 0u, ones ? 0x3F80u : 0u, 0u};
  if (CODED) {
    const int cnt = max(ti.cnt, 1);
    const uint32_t ua = ti.base + min(n16, cnt - 1);
#pragma unroll
    for (int ks = 0; ks < DCK; ++ks) {
      // Columns past d_c (only when d_c is not a multiple of 32) read the
      // row's own first columns and are zeroed after the load.
      const int c = ks * 32 + q4 * 8;
      const Frag v = ldg<Frag>(p.codesK, (ua * dc + (c < dc ? c : 0)) * 2u);
      td.ck[ks] = c < dc ? v : Frag{0u, 0u, 0u, 0u};
    }
    const int cc = n16 * 4 < dc ? n16 * 4 : 0;
#pragma unroll
    for (int g2 = 0; g2 < 2; ++g2) {
      const uint32_t u0 = ti.base + min(q4 * 4 + 2 * g2, cnt - 1);
      const uint32_t u1 = ti.base + min(q4 * 4 + 2 * g2 + 1, cnt - 1);
      const U32x2 a = ldg<U32x2>(p.codesV, (u0 * dc + cc) * 2u);
      const U32x2 b = ldg<U32x2>(p.codesV, (u1 * dc + cc) * 2u);
      td.bc[g2] = n16 * 4 < dc ? Frag{a.x, a.y, b.x, b.y} : one_col;
    }
  } else {
    td.bc[0] = td.bc[1] = one_col;
  }
}

struct State {
  float m;         // running max (base-2 units) of query head (l%16)/4
  f32x4 accr[2];   // value-reference accumulators of query head l/16
  f32x4 accc;      // value-code accumulators (+ weight sum column)
};

template <bool CODED, int DCK>
__device__ __forceinline__ void compute_tile(const Tile& td, const Frag* qk, const Frag* qh, const Frag* ql, float cs,
                                             int q4, const uint32_t* sel, State& st) {
  f32x4 sr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) sr = mfma16(td.kr[ks], qk[ks], sr);
  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
  if (CODED) {
#pragma unroll
    for (int ks = 0; ks < DCK; ++ks) {
      sc = mfma16(td.ck[ks], qh[ks], sc);
      sc = mfma16(td.ck[ks], ql[ks], sc);
    }
  }
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = q4 * 4 + i < td.cnt ? fmaf(sr[i], cs, sc[i]) : -INFINITY;
  const float tmax = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  if (__ballot(tmax > st.m + kTau) != 0ull) {
    float t2 = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    t2 = fmaxf(t2, __shfl_xor(t2, 32, 64));
    const float mn = fmaxf(st.m, t2);
    const float alpha = st.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.m - mn);
    st.m = mn;
    const float aa = __shfl(alpha, q4 * 4, 64);   // accumulators hold query head q4
    st.accr[0] *= aa;
    st.accr[1] *= aa;
    st.accc *= aa;
  }
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(s[i] - st.m);
  const uint32_t h01 = pk_bf16(p[0], p[1]), h23 = pk_bf16(p[2], p[3]);
  const uint32_t l01 = pk_bf16(p[0] - __uint_as_float(h01 << 16), p[1] - __uint_as_float(h01 & 0xFFFF0000u));
  const uint32_t l23 = pk_bf16(p[2] - __uint_as_float(h23 << 16), p[3] - __uint_as_float(h23 & 0xFFFF0000u));
#pragma unroll
  for (int g2 = 0; g2 < 2; ++g2) {
    const uint32_t hp = g2 ? h23 : h01, lp = g2 ? l23 : l01;
    const Frag ah = Frag{__builtin_amdgcn_perm(hp, hp, sel[0]), __builtin_amdgcn_perm(hp, hp, sel[1]),
                         __builtin_amdgcn_perm(hp, hp, sel[2]), __builtin_amdgcn_perm(hp, hp, sel[3])};
    const Frag al = Frag{__builtin_amdgcn_perm(lp, lp, sel[0]), __builtin_amdgcn_perm(lp, lp, sel[1]),
                         __builtin_amdgcn_perm(lp, lp, sel[2]), __builtin_amdgcn_perm(lp, lp, sel[3])};
    st.accr[0] = mfma16(ah, td.xv[g2][0], st.accr[0]);
    st.accr[0] = mfma16(al, td.xv[g2][0], st.accr[0]);
    st.accr[1] = mfma16(ah, td.xv[g2][1], st.accr[1]);
    st.accr[1] = mfma16(al, td.xv[g2][1], st.accr[1]);
    st.accc = mfma16(ah, td.bc[g2], st.accc);
    st.accc = mfma16(al, td.bc[g2], st.accc);
  }
}

// One run of tiles of a wave: software pipeline, two tiles per trip
// (buffers A and B); the ordinals of tile t+2 and the data of tile t+1 are
// in flight while tile t computes.  Dead tiles (past the run) are masked.
template <bool CODED, int DCK, typename IdxT>
__device__ __forceinline__ void run_tiles(const Args& p, const Shape& sh, int t0, int t1, int first, int last,
                                          int n16, int q4, const Frag* qk, const Frag* qh, const Frag* ql, float cs,
                                          const uint32_t* sel, State& st) {
  if (t0 >= t1) return;
  TileIdx ia, ib;
  Tile da, db;
  load_idx<CODED, IdxT>(p, t0, t1, first, last, n16, q4, ia);
  load_idx<CODED, IdxT>(p, t0 + 1, t1, first, last, n16, q4, ib);
  load_data<CODED, DCK>(p, sh, ia, n16, q4, da);
  for (int tt = t0; tt < t1; tt += 2) {
    load_idx<CODED, IdxT>(p, tt + 2, t1, first, last, n16, q4, ia);
    load_data<CODED, DCK>(p, sh, ib, n16, q4, db);
    compute_tile<CODED, DCK>(da, qk, qh, ql, cs, q4, sel, st);
    load_idx<CODED, IdxT>(p, tt + 3, t1, first, last, n16, q4, ib);
    load_data<CODED, DCK>(p, sh, ia, n16, q4, da);
    compute_tile<CODED, DCK>(db, qk, qh, ql, cs, q4, sel, st);
  }
}

// Split boundaries (coded rows on 16-row boundaries).
__device__ __forceinline__ int split_lo(int n, int sp, int splits, int align) {
  int64_t x = (int64_t)n * sp / splits;
  return sp == splits ? n : (int)(x / align * align);
}

template <int DCK, typename IdxT>
__global__ __launch_bounds__(kThreads) void k_decode_mfma(DecodeArgs a, Shape sh) {
  __shared__ __attribute__((aligned(16))) uint16_t w_lds[kD * kMaxDc];
  __shared__ float q_lds[4][kD];
  __shared__ float qp4[4][4 * kMaxDc];
  __shared__ float qp_lds[4][kMaxDc];
  __shared__ float red_m[kWaves][4];
  __shared__ float red_acc[kWaves][4][kD + 64];

  const int BH = sh.B * sh.H;
  const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
  const int bh = xcd + 8 * (kx / a.splits), sp = kx % a.splits;
  if (bh >= BH) return;
  const int b = bh / sh.H, h = bh % sh.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int gl = n16 >> 2, el = lane & 3;   // score layout: query head, e
  const int G = a.G, dc = sh.dc;
  const float cs = a.scale * kLog2e;

  const int n0 = split_lo(sh.N, sp, a.splits, 16), n1 = split_lo(sh.N, sp + 1, a.splits, 16);
  const int r0 = split_lo(sh.R, sp, a.splits, 1), r1 = split_lo(sh.R, sp + 1, a.splits, 1);
  const int nct = (n1 - n0 + 15) / 16, nrt = (r1 - r0 + 15) / 16;
  const int nt = nct + nrt;
  const int t_beg = (int)((int64_t)nt * wave / kWaves), t_end = (int)((int64_t)nt * (wave + 1) / kWaves);

  Args p;
  const size_t sK = (size_t)bh * 2, sV = sK + 1;
  p.refsK = (const uint16_t*)a.refs + sK * sh.R * kD;
  p.refsV = (const uint16_t*)a.refs + sV * sh.R * kD;
  p.codesK = (const uint16_t*)a.codes + sK * sh.N * dc;
  p.codesV = (const uint16_t*)a.codes + sV * sh.N * dc;
  p.idxK = (const IdxT*)a.idx + sK * sh.N;
  p.idxV = (const IdxT*)a.idx + sV * sh.N;

  // ---- q'_g = scale * log2e * W_up_K^T q_g, through LDS ----
  const uint16_t* q = (const uint16_t*)a.q + ((size_t)b * a.Hq + h * G) * kD;
  {
    const uint16_t* wu = (const uint16_t*)a.wuk + (size_t)h * a.w_hs;
    for (int i = tid; i < kD * dc / 8; i += kThreads)
      *reinterpret_cast<uint4*>(&w_lds[i * 8]) = *reinterpret_cast<const uint4*>(wu + (size_t)i * 8);
    for (int i = tid; i < G * kD; i += kThreads) q_lds[i / kD][i % kD] = bf2f(q[i]);
  }
  // The score B operands of the key references: q_g itself (exact bf16).
  Frag qk[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qk[ks] = gl < G ? ldg<Frag>(q, ((uint32_t)gl * kD + ks * 32 + q4 * 8) * 2u) : Frag{0u, 0u, 0u, 0u};
  __syncthreads();
  for (int i = tid; i < 4 * G * dc; i += kThreads) {
    const int qt = i / (G * dc), r = i % (G * dc), g = r / dc, j = r % dc;
    float acc = 0.f;
#pragma unroll 8
    for (int k = qt * (kD / 4); k < (qt + 1) * (kD / 4); ++k) acc = fmaf(q_lds[g][k], bf2f(w_lds[k * dc + j]), acc);
    qp4[qt][r] = acc;
  }
  __syncthreads();
  for (int i = tid; i < G * dc; i += kThreads)
    qp_lds[i / dc][i % dc] = (qp4[0][i] + qp4[1][i] + qp4[2][i] + qp4[3][i]) * cs;
  __syncthreads();
  Frag qh[DCK], ql[DCK];
#pragma unroll
  for (int ks = 0; ks < DCK; ++ks) {
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      const int j = ks * 32 + q4 * 8 + k2 * 2;
      const float v0 = (gl < G && j < dc) ? qp_lds[gl][j] : 0.f;
      const float v1 = (gl < G && j + 1 < dc) ? qp_lds[gl][j + 1] : 0.f;
      const uint32_t hp = pk_bf16(v0, v1);
      qh[ks][k2] = hp;
      ql[ks][k2] = pk_bf16(v0 - __uint_as_float(hp << 16), v1 - __uint_as_float(hp & 0xFFFF0000u));
    }
  }
  // v_perm selectors that place a packed pair (p_a low, p_b high) at
  // positions e and 4 + e of an 8 x bf16 A operand (zeros elsewhere).
  uint32_t sel[4];
  {
    const uint32_t lo_a = (el & 1) ? 0x01000c0cu : 0x0c0c0100u;  // p_a into half e&1
    const uint32_t lo_b = (el & 1) ? 0x03020c0cu : 0x0c0c0302u;  // p_b into half e&1
    const int dw = el >> 1;
    sel[0] = dw == 0 ? lo_a : 0x0c0c0c0cu;
    sel[1] = dw == 1 ? lo_a : 0x0c0c0c0cu;
    sel[2] = dw == 0 ? lo_b : 0x0c0c0c0cu;
    sel[3] = dw == 1 ? lo_b : 0x0c0c0c0cu;
  }

  State st;
  st.m = -INFINITY;
  st.accr[0] = st.accr[1] = st.accc = f32x4{0.f, 0.f, 0.f, 0.f};
  // The wave's tiles: coded tiles [0, nct) then reference tiles [nct, nt).
  run_tiles<true, DCK, IdxT>(p, sh, t_beg, min(t_end, nct), n0, n1, n16, q4, qk, qh, ql, cs, sel, st);
  run_tiles<false, DCK, IdxT>(p, sh, max(t_beg, nct) - nct, t_end - nct, r0, r1, n16, q4, qk, qh, ql, cs, sel, st);

  // ---- merge the block's waves (fixed order) ----
  if (lane < 16 && el == 0) red_m[wave][gl] = st.m;
  __syncthreads();
  float mb = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) mb = fmaxf(mb, red_m[w][q4]);
  const float mw = red_m[wave][q4];
  const float wgt = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - mb);
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int i = 0; i < 4; ++i) red_acc[wave][q4][n16 * 8 + hh * 4 + i] = st.accr[hh][i] * wgt;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (n16 * 4 + i <= dc) red_acc[wave][q4][kD + n16 * 4 + i] = st.accc[i] * wgt;
  __syncthreads();
  // Partial record per query head: [max, sum, code acc[dc], reference acc[d]].
  const int rec = partial_rec(sh);
  float* part = a.part + (size_t)bh * a.splits * G * rec;
  float* mine = part + (size_t)sp * G * rec;
  for (int i = tid; i < G * rec; i += kThreads) {
    const int g = i / rec, f = i % rec;
    float v = 0.f;
    if (f == 0) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v = w == 0 ? red_m[0][g] : fmaxf(v, red_m[w][g]);
    } else if (f == 1) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += red_acc[w][g][kD + dc];
    } else if (f < 2 + dc) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += red_acc[w][g][kD + f - 2];
    } else if (f < 2 + dc + kD) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += red_acc[w][g][f - 2 - dc];
    }
    mine[i] = v;
  }

}

// combine: merges the splits of one (b, query head) and applies mu_V and
// W_up_V.  grid B*Hq, block 256: thread t owns column t of the partial
// records (code columns, then head-dim columns) and issues its loads of 32
// splits at once, together with the split maxima and sums, so the records
// (written by blocks on several XCDs) arrive in few round trips.
constexpr int kCombineBatch = 32;

__global__ __launch_bounds__(256) void k_combine(DecodeArgs a, Shape sh) {
  __shared__ float mls[2][kMfmaMaxSplits];
  __shared__ float accc[kMaxDc];
  __shared__ float red[1];
  const int bq = blockIdx.x;
  const int b = bq / a.Hq, gq = bq % a.Hq;
  const int h = gq / a.G, g = gq % a.G;
  const int bh = b * sh.H + h;
  const int rec = partial_rec(sh), dc = sh.dc, ns = a.splits;
  const size_t pstride = (size_t)a.G * rec;
  const float* part = a.part + (size_t)bh * ns * pstride + (size_t)g * rec;
  const int t = threadIdx.x;
  const bool has_col = t < dc + kD;
  const float* pc = part + 2 + (has_col ? t : 0);
  // W_up_V row of this thread's output column, loaded early.
  const int i_out = t - dc;
  const uint16_t* wuv = (const uint16_t*)a.wuv + (size_t)h * a.w_hs;
  U32x2 wrow[kMaxDc / 4];
#pragma unroll
  for (int j = 0; j < kMaxDc / 4; ++j)
    wrow[j] = (i_out >= 0 && has_col && j * 4 < dc) ? ldg<U32x2>(wuv, ((uint32_t)i_out * dc + j * 4) * 2u)
                                                      : U32x2{0u, 0u};
  float v[kCombineBatch];
#pragma unroll
  for (int k = 0; k < kCombineBatch; ++k) v[k] = (has_col && k < ns) ? pc[(size_t)k * pstride] : 0.f;
  for (int s2 = t; s2 < ns; s2 += 256) {
    mls[0][s2] = part[s2 * pstride];
    mls[1][s2] = part[s2 * pstride + 1];
  }
  __syncthreads();
  if (t < 64) {
    float mx = -INFINITY;
    for (int s2 = t; s2 < ns; s2 += 64) mx = fmaxf(mx, mls[0][s2]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    float l = 0.f;
    for (int s2 = t; s2 < ns; s2 += 64) {
      const float ms = mls[0][s2];
      const float w = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - mx);
      mls[0][s2] = w;
      l = fmaf(w, mls[1][s2], l);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
    if (t == 0) red[0] = l;
  }
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < kCombineBatch; ++k)
    if (k < ns) acc = fmaf(mls[0][k], v[k], acc);
  for (int s0 = kCombineBatch; s0 < ns; s0 += kCombineBatch) {
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k) v[k] = (has_col && s0 + k < ns) ? pc[(size_t)(s0 + k) * pstride] : 0.f;
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k)
      if (s0 + k < ns) acc = fmaf(mls[0][s0 + k], v[k], acc);
  }
  if (t < dc) accc[t] = acc;
  __syncthreads();
  if (i_out >= 0 && has_col) {
    float u = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxDc / 4; ++j) {
      if (j * 4 >= dc) break;
      u = fmaf(__uint_as_float(wrow[j].x << 16), accc[j * 4 + 0], u);
      u = fmaf(__uint_as_float(wrow[j].x & 0xFFFF0000u), accc[j * 4 + 1], u);
      u = fmaf(__uint_as_float(wrow[j].y << 16), accc[j * 4 + 2], u);
      u = fmaf(__uint_as_float(wrow[j].y & 0xFFFF0000u), accc[j * 4 + 3], u);
    }
    const float muv = bf2f(((const uint16_t*)a.mu)[((size_t)bh * 2 + 1) * kD + i_out]);
    a.out[((size_t)b * a.Hq + gq) * kD + i_out] = muv + (acc + u) / red[0];
  }
}

}  // namespace

bool decode_fused_supported(const Shape& sh, int G, int splits) {
  return sh.bf16 && sh.d == kD && G <= 4 && sh.dc <= kMaxDc && splits <= kMfmaMaxSplits;
}

int decode_fused_auto_splits(const Shape& sh) {
  const int64_t heads_per_xcd = (sh.B * sh.H + 7) / 8;
  int64_t s = (512 + 8 * heads_per_xcd - 1) / (8 * heads_per_xcd);
  const int64_t by_len = (sh.T + 511) / 512;
  if (s > by_len) s = by_len;
  if (s < 1) s = 1;
  if (s > kMfmaMaxSplits) s = kMfmaMaxSplits;
  return (int)s;
}

hipError_t launch_decode_fused(const Shape& sh, const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(8 * ((sh.B * sh.H + 7) / 8) * a.splits);
  const bool i16 = sh.idx_bytes == 2;
  hipError_t e;
  hipEvent_t e0 = ev_start(a.events, 1), e1 = ev_stop(a.events, 1);
  if (sh.dc <= 32)
    e = i16 ? launch(k_decode_mfma<1, uint16_t>, grid, kThreads, st, e0, e1, a, sh)
            : launch(k_decode_mfma<1, uint32_t>, grid, kThreads, st, e0, e1, a, sh);
  else
    e = i16 ? launch(k_decode_mfma<2, uint16_t>, grid, kThreads, st, e0, e1, a, sh)
            : launch(k_decode_mfma<2, uint32_t>, grid, kThreads, st, e0, e1, a, sh);
  if (e != hipSuccess) return e;
  e = launch(k_combine, dim3(sh.B * a.Hq), 256, st, ev_start(a.events, 2), ev_stop(a.events, 2), a, sh);
  if (e != hipSuccess || !a.events) return e;
  // The reference scores are computed inside the split kernel: an empty stage.
  if ((e = hipEventRecord(ev_start(a.events, 0), st)) != hipSuccess) return e;
  return hipEventRecord(ev_stop(a.events, 0), st);
}

}  // namespace dkv
