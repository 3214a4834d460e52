// DeltaKV decode attention, MFMA path (bfloat16 storage, head dim 128, up to
// 4 query heads per KV head, code dim 16..48).
//
// Attention of query head g over every cached token t as if it were
// reconstructed, k^_t = mu + ref + W_up code (DeltaKV explainer, English
// page, Technical Summary §3 "Reconstruction"):
//
//   score(t) = S[ref_K(t)][g] + q'_g . code_K(t),
//              S[r][g] = c * q_g . refs_K[r],  q'_g = c * W_up_K^T q_g,  c = scale * log2 e
//   out_g    = mu_V + (sum_t p_t refs_V[ref_V(t)] + W_up_V sum_t p_t code_V(t)) / sum_t p_t
//
// (q_g . mu_K is the same for every token and cancels in the softmax; a
// reference token r is a token whose reference is itself and whose code is
// 0.)  Three kernels per decode step:
//
//   refscore  S for every key reference (one MFMA chain per 16 references)
//             and q' (16 lanes per output element);
//   split     the token stream: the B*H (sequence, KV head) pairs are split
//             along the sequence; a 512-thread block (8 waves) owns one
//             piece, each wave a contiguous run of 16-token tiles.  The
//             head's S table sits in LDS, so a token's key reference costs
//             one LDS read instead of a 256-byte row gather.  Each block
//             applies W_up_V to its own value-code sums, so its record per
//             query head is [max, sum, d output columns];
//   combine   merges the splits of each query head and adds mu_V (one wave
//             per 64 columns, no LDS, no barrier).
//
// Blocks of head bh run on XCD bh % 8 (workgroups are dispatched to the
// eight XCDs round-robin), so the value reference rows a head gathers stay
// in one L2.
//
// Per 16-token tile a wave issues one MFMA 16x16x32 (bf16 in, fp32
// accumulate) chain for the code part of the scores and three for the value
// side, every operand lane-local (lane l: n16 = l % 16, q4 = l / 16):
//   scores  C[token][(g, e)] = code_K(token) . q'_g: A = key code rows
//           (token n16), B = q'_g split into bf16 hi + lo parts, replicated
//           over e; lane l ends with the scores of query head n16 / 4 for
//           tokens 4 q4 + i, i = 0..3, and adds S[ref_K(token)][g] from LDS;
//   values  C[(g, e)][n] += sum_k P[(g, e)][k] X[k][n], k = (token, e'),
//           P[(g, e)][(token, e')] = p_g(token) if e == e' else 0,
//           X[(token, e')][n] = row(token)[8n + e' (+4)] (value reference
//           rows) or [4n + e'] (value code rows): the weights a lane holds
//           are the ones it feeds (A), B is whole row segments as loaded,
//           and lane l accumulates query head q4.
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
constexpr int kRsRefs = 64;                              // references per refscore block
constexpr int kRedFloats = kWaves * 4 * (kD + 64);       // wave-merge buffer of the split kernel
constexpr size_t kSplitLdsMax = 160 * 1024 - 1024;       // dynamic LDS of one split block

typedef uint32_t Frag __attribute__((ext_vector_type(4)));
typedef uint32_t U32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(1))) char* GPtr;

__device__ __forceinline__ f32x4 mfma16(Frag a, Frag b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
}

// Two floats -> packed bf16 pair, round to nearest even (one instruction).
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// a where the bits of m are set, b elsewhere (one bitfield select, never a
// branch).
__device__ __forceinline__ float bsel(uint32_t m, float a, float b) {
  return __uint_as_float((__float_as_uint(a) & m) | (__float_as_uint(b) & ~m));
}

// v[i] of a four-entry register array for a run-time i in 0..3, by bitfield
// selects (the array stays in registers, and a lane-dependent i makes no
// divergent branch).
__device__ __forceinline__ float pick4(float v0, float v1, float v2, float v3, int i) {
  const uint32_t m1 = 0u - (uint32_t)(i & 1), m2 = 0u - (uint32_t)((i >> 1) & 1);
  return bsel(m2, bsel(m1, v3, v2), bsel(m1, v1, v0));
}
__device__ __forceinline__ float pick4(const float (&v)[4], int i) { return pick4(v[0], v[1], v[2], v[3], i); }

// DPP move of a float with control C (every lane has a valid source).
template <int C>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), C, 0xF, 0xF, true));
}

// Sum over the wave, the same value in every lane: quads (quad_perm 1,0,3,2
// and 2,3,0,1), eights (row_half_mirror) and rows of 16 (row_mirror) by DPP,
// each step adding two equal partial sums in either order, then the four
// row sums by readlane, added in a fixed order.
__device__ __forceinline__ float wave_sum(float v) {
  v += dppf<0xB1>(v);
  v += dppf<0x4E>(v);
  v += dppf<0x141>(v);
  v += dppf<0x140>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Maximum over the wave, the same value in every lane (as wave_sum).
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dppf<0xB1>(v));
  v = fmaxf(v, dppf<0x4E>(v));
  v = fmaxf(v, dppf<0x141>(v));
  v = fmaxf(v, dppf<0x140>(v));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Global-memory load at a byte offset (the address space is explicit so that
// selected base pointers still compile to global, not flat, loads).
template <typename T>
__device__ __forceinline__ T ldg(const void* base, uint32_t byte_off) {
  return *(const __attribute__((address_space(1))) T*)((GPtr)base + byte_off);
}

// bf16 {1, 0, 0, 0}: value-code operand of the weight-sum column (read by
// lanes past the code columns; 16 bytes so that 16-byte loads may read it).
__device__ const uint16_t kOnePair[8] __attribute__((aligned(16))) = {0x3F80u, 0u, 0u, 0u, 0x3F80u, 0u, 0u, 0u};

// ---------------------------------------------------------------------------
// refscore.  Block (bh, chunk) of 256 threads: S rows of kRsRefs references
// (wave w: references chunk*64 + 16w + n16; A = q_g, B = reference rows read
// from LDS, where the block's rows arrive by buffer loads straight into LDS,
// one contiguous KB per wave instruction; lane (n16, q4 = 0) ends with
// S[r][0..3]); wave 0 also computes q' outputs
// 4 (chunk + chunks m), m = 0, 1, ...: four consecutive code columns of one
// query head, lane l taking rows l and l + 64 of W_up (8 contiguous bytes
// each), summed over the wave by wave_sum.  The first group's
// loads go out with the S loads, so a block takes one round trip.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_refscore_mfma(DecodeArgs a, Shape sh, int chunks) {
  const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
  const int bh = xcd + 8 * (kx / chunks), c = kx % chunks;
  if (bh >= sh.B * sh.H) return;
  const int b = bh / sh.H, h = bh % sh.H;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15, q4 = lane >> 4;
  const int G = a.G, dc = sh.dc;
  const float cs = a.scale * kLog2e;
  const uint16_t* q = (const uint16_t*)a.q + ((size_t)b * a.Hq + h * G) * kD;

  const int r = c * kRsRefs + wave * 16 + n16;
  const uint16_t* refsK = (const uint16_t*)a.refs + (size_t)bh * 2 * sh.Rc * kD;
  // q' group of this block (wave 0): outputs o0 .. o0 + 3 (clamped when the
  // block has none; the stores are masked).
  const int no = G * dc;
  const uint16_t* wu = (const uint16_t*)a.wuk + (size_t)h * a.w_hs;
  auto qp_loads = [&](int o0, U32x2 (&w)[2], uint16_t (&qx)[2]) {
    const int oc = min(o0, no - 4);
    const int g = oc / dc, j = oc % dc;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const uint32_t row = (uint32_t)(lane + 64 * hh);
      w[hh] = ldg<U32x2>(wu, (row * dc + (uint32_t)j) * 2u);
      qx[hh] = ldg<uint16_t>(q, ((uint32_t)g * kD + row) * 2u);
    }
  };
  auto qp_out = [&](int o0, const U32x2 (&w)[2], const uint16_t (&qx)[2]) {
    float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const float qf = bf2f(qx[hh]);
      v[0] = fmaf(qf, __uint_as_float(w[hh].x << 16), v[0]);
      v[1] = fmaf(qf, __uint_as_float(w[hh].x & 0xFFFF0000u), v[1]);
      v[2] = fmaf(qf, __uint_as_float(w[hh].y << 16), v[2]);
      v[3] = fmaf(qf, __uint_as_float(w[hh].y & 0xFFFF0000u), v[3]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = wave_sum(v[e]);
    if (lane < 4 && o0 < no) {
      const int g = o0 / dc, j = o0 % dc + lane;
      a.qp[((size_t)bh * G + g) * dc + j] = pick4(v, lane) * cs;
    }
  };
  // Every wave issues the first group's loads (a branch around them would
  // make the compiler wait for them at its end); wave 0 uses them.
  const bool qp_wave = wave == 0 && 4 * c < no;
  U32x2 w0[2];
  uint16_t q0[2];
  qp_loads(4 * c, w0, q0);
  // The block's 64 reference rows go straight into LDS, each wave
  // instruction one contiguous KB (rows past R read as zeros); piece p of row
  // w lands at slot p ^ (w & 15), so the B-fragment reads below hit distinct
  // banks.  The query rows come through registers.
  __shared__ __attribute__((aligned(16))) uint16_t rl[kRsRefs * kD];
  {
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(refsK + (size_t)c * kRsRefs * kD,
                                                  (uint32_t)max(sh.R - c * kRsRefs, 0) * kD * 2u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int qi = (wave * 4 + j) * 64 + lane;   // 16-byte slot in LDS order
      const int row = qi >> 4, slot = qi & 15;
      const uint32_t voff = (uint32_t)(row * kD + ((slot ^ (row & 15)) << 3)) * 2u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(rl + (wave * 4 + j) * 512),
                                               16, voff, 0, 0, 0);
    }
  }
  Frag aq[4], br[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint32_t col = ks * 32 + q4 * 8;
    aq[ks] = ldg<Frag>(q, ((uint32_t)min(n16, G - 1) * kD + col) * 2u);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the LDS rows have landed
  __syncthreads();
  {
    const int row = wave * 16 + n16;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int piece = ks * 4 + q4;
      br[ks] = *reinterpret_cast<const Frag*>(&rl[row * kD + ((piece ^ (row & 15)) << 3)]);
    }
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const Frag a0 = n16 < G ? aq[ks] : Frag{0u, 0u, 0u, 0u};
    acc = mfma16(a0, br[ks], acc);
  }
  if (q4 == 0 && r < sh.R)
    *reinterpret_cast<f32x4*>(a.score + ((size_t)bh * sh.R + r) * 4) = acc * cs;
  if (qp_wave) {
    qp_out(4 * c, w0, q0);
    // Further groups of this block (only when G d_c > 4 chunks).
    for (int o0 = 4 * (c + chunks); o0 < no; o0 += 4 * chunks) {
      U32x2 w[2];
      uint16_t qx[2];
      qp_loads(o0, w, qx);
      qp_out(o0, w, qx);
    }
  }
}

// ---------------------------------------------------------------------------
// split.
// ---------------------------------------------------------------------------

// One 16-token tile.  Lane (n16, q4) with n16 < 4 holds the key ordinal of
// token 4 q4 + n16, with 4 <= n16 < 8 the value ordinal of token
// 4 q4 + n16 - 4; a row broadcast hands every lane of row q4 the ordinals of
// its four tokens.  Ordinals are loaded a step ahead of the tile's data.
// Coded tiles and reference tiles are separate instantiations, so that the
// loop bodies have no control flow (a branch merge would make the compiler
// drain every outstanding load).
struct TileIdx {
  int base, cnt;   // first token (coded row or reference ordinal); valid tokens (0 = dead tile);
                   // token lists: cnt is the tile's validity mask (bit j = token j)
  int raw;
  // Token lists only: the ordinal of a reference or invalid position (used
  // instead of raw when use_alt), and the code rows of the lane's key-code
  // and value-code tokens (-1: zero row).
  int alt, use_alt, rb, rc;
  // k references per token (KT > 1): the lane's token's ordinals 1 .. KT - 1
  // (ordinal 0 is raw).
  int rk[kTopMax];
};

struct Tile {
  float sb[4];     // S[ref_K(token 4 q4 + i)][n16 / 4]
  Frag ck[2];      // score A: key code row of token n16 (coded tiles)
  Frag xv[2][2];   // value B [group][half]: tokens 4 q4 + 2 group + {0, 1}
  Frag bc[2];      // value-code B [group] (+ the 1.0 column); d_c > 32
  Frag cv;         // d_c <= 32: the tile's value codes, one 16-byte load per lane
  uint32_t ckq;    // 4-bit codes: the key code nibbles of token n16 (columns 8 q4 ..)
  uint32_t cvq;    // 4-bit codes: the value code nibbles the lane would load as cv
  uint32_t scl;    // 4-bit codes: bits of the key scale of token 4 q4 + n16 % 4 (token lists: n16)
  uint32_t sclv;   // 4-bit codes: bits of the value scale of the token of cvq
  int cnt;
  // k references per token (KT > 1): value ordinals 1 .. KT - 1 of the lane's
  // broadcast token, the reference counts of tokens 4 q4 + j (4 bits each),
  // and their reciprocals.
  int rk[kTopMax];
  uint32_t cnt4;
  float invc[4];
};

struct Args {
  // per (b, h) stream bases
  const uint16_t* refsV;
  const uint16_t* codesK;
  const uint16_t* codesV;
  const uint8_t* qK;      // 4-bit codes: rows of d_c / 2 bytes
  const uint8_t* qV;
  const uint16_t* sclK;   // 4-bit codes: per-row scales
  const uint16_t* sclV;
  const void* idxK;       // uint16_t or uint32_t ordinals
  const void* idxV;
  const float* score;     // S rows of this (b, h), 4 floats each
  const uint32_t* list;   // token lists: the positions of sequence b
  uint32_t magic;         // token lists: floor((2^32 - 1) / s)
};

// 256 zero bytes: the code row of a reference position in a token list.
__device__ const uint32_t kZeroCodes[64] __attribute__((aligned(16))) = {0u};

// floor(t / s) from magic = floor((2^32 - 1) / s): the high product is
// floor(t / s) or one less, and one correction step fixes it.
__device__ __forceinline__ uint32_t div_s(uint32_t t, uint32_t s, uint32_t magic) {
  const uint32_t q = __umulhi(t, magic);
  return q + (uint32_t)(t - q * s >= s);
}

// Lane k of each 16-lane row, broadcast over the row.  Every lane has a
// valid source in these DPP patterns, so no "old" value is needed (plain DPP
// moves with bound_ctrl: no initialising copy of the destination).
template <int K>
__device__ __forceinline__ int row_bcast(int v) {
  return __builtin_amdgcn_mov_dpp(v, 0x150 + K, 0xF, 0xF, true);
}

// Tile tt of a run [t0, t1) of 16-token tiles starting at token `first`
// and ending at token `last` (exclusive).  Tiles past t1 are dead: they
// repeat the run's last tile with cnt = 0.
template <bool CODED, typename IdxT, int KT = 1>
__device__ __forceinline__ void load_idx(const Args& p, int tt, int t1, int first, int last, int n16, int q4,
                                         TileIdx& ti, int K = 1) {
  const bool live = tt < t1;
  tt = min(tt, t1 - 1);
  const int base = first + tt * 16;
  const int cnt = min(16, last - base);
  ti.base = base;
  ti.cnt = live ? cnt : 0;
  const int u = base + min(q4 * 4 + (n16 & 3), cnt - 1);
  if (CODED && KT > 1) {
    // Rows of K ordinals; slots past K repeat the last one (never used).
    const IdxT* src = (const IdxT*)(n16 < 4 ? p.idxK : p.idxV) + (size_t)u * K;
    ti.raw = (int)src[0];
#pragma unroll
    for (int k = 1; k < KT; ++k) ti.rk[k] = (int)src[min(k, K - 1)];
  } else if (CODED) {
    const IdxT* src = (const IdxT*)(n16 < 4 ? p.idxK : p.idxV);
    ti.raw = (int)src[u];
  } else {
    ti.raw = u;
  }
}

// Token-list mode: tile tt of the list entries [first, last) of the block.
// A lane reads the positions of three of the tile's tokens: j_a, whose
// ordinal it contributes to the row broadcast (lanes n16 < 8: key ordinal of
// token 4 q4 + n16, value ordinal of token 4 q4 + n16 - 4), j_b = n16 (its
// key-code row) and j_c (its value-code row, the token load_data pairs it
// with).  A reference position acts as a coded token with a zero code row and
// its own ordinal in both streams, so its score is S[t / s] and its value the
// reference row; a position at or past T is cleared by the validity mask.
template <typename IdxT>
__device__ __forceinline__ void load_idx_sel(const Args& p, const Shape& sh, int tt, int t1, int first, int last,
                                             int n16, int q4, TileIdx& ti) {
  const bool live = tt < t1;
  tt = min(tt, t1 - 1);
  const int base = first + tt * 16;
  const int cnt = min(16, last - base);
  const int ja = q4 * 4 + (n16 & 3), jb = n16, jc = q4 * 4 + 2 * (n16 >> 3) + (n16 & 1);
  const uint32_t pa = p.list[base + min(ja, cnt - 1)];
  const uint32_t pb = p.list[base + min(jb, cnt - 1)];
  const uint32_t pc = p.list[base + min(jc, cnt - 1)];
  const uint32_t T = (uint32_t)sh.T, s = (uint32_t)sh.s;
  const uint32_t qa = div_s(pa, s, p.magic), qb = div_s(pb, s, p.magic), qc = div_s(pc, s, p.magic);
  const bool coded_a = pa < T && pa != qa * s;
  const bool coded_b = pb < T && pb != qb * s;
  const bool coded_c = pc < T && pc != qc * s;
  // Not coded: read the zero row (a layout may hold no coded rows at all).
  const IdxT* src = coded_a ? (const IdxT*)(n16 < 4 ? p.idxK : p.idxV) + (pa - qa - 1) : (const IdxT*)kZeroCodes;
  ti.raw = (int)ldg<IdxT>(src, 0u);
  ti.alt = pa < T ? (int)qa : 0;
  ti.use_alt = !coded_a;
  ti.rb = coded_b ? (int)(pb - qb - 1) : -1;
  ti.rc = coded_c ? (int)(pc - qc - 1) : -1;
  const uint64_t vb = __ballot(live && jb < cnt && pb < T);
  ti.cnt = (int)(vb & 0xFFFFull);
  ti.base = 0;
}

template <bool CODED, bool SEL, typename IdxT, int KT = 1>
__device__ __forceinline__ void load_tile_idx(const Args& p, const Shape& sh, int tt, int t1, int first, int last,
                                              int n16, int q4, TileIdx& ti) {
  if constexpr (SEL)
    load_idx_sel<IdxT>(p, sh, tt, t1, first, last, n16, q4, ti);
  else
    load_idx<CODED, IdxT, KT>(p, tt, t1, first, last, n16, q4, ti, sh.K);
}

template <int I, bool SLDS>
__device__ __forceinline__ float s_lookup(const Args& p, const float* s_lds, int raw, int R, int gl) {
  const uint32_t rk = (uint32_t)min(row_bcast<I>(raw), R - 1);
  return SLDS ? s_lds[rk * 4 + gl] : ldg<float>(p.score, (rk * 4 + gl) * 4u);
}

template <bool CODED, int DCK, bool SLDS, bool Q4, bool SEL = false, int KT = 1>
__device__ __forceinline__ void load_data(const Args& p, const Shape& sh, const float* s_lds, const TileIdx& ti,
                                          int n16, int q4, Tile& td) {
  const int dc = sh.dc;
  const int gl = n16 >> 2;
  td.cnt = ti.cnt;
  const int raw = SEL ? (ti.use_alt ? ti.alt : ti.raw) : ti.raw;
  // Ordinals come from caller memory: clamp so that a corrupt cache can never
  // address outside the reference arrays or the S table.
  td.sb[0] = s_lookup<0, SLDS>(p, s_lds, raw, sh.R, gl);
  td.sb[1] = s_lookup<1, SLDS>(p, s_lds, raw, sh.R, gl);
  td.sb[2] = s_lookup<2, SLDS>(p, s_lds, raw, sh.R, gl);
  td.sb[3] = s_lookup<3, SLDS>(p, s_lds, raw, sh.R, gl);
  if constexpr (CODED && KT > 1) {
    // Token 4 q4 + j (coded row n) averages cnt = min(K, n / (s - 1) + 1)
    // references: its position t has t / s = n / (s - 1) earlier references
    // besides its own block's.  The key score takes the mean of their S rows.
    const int s1 = sh.s - 1;
    uint32_t cnt4 = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = ti.base + q4 * 4 + j;
      int c = 1;
#pragma unroll
      for (int k = 1; k < KT; ++k) c += (k < sh.K && n >= k * s1) ? 1 : 0;
      cnt4 |= (uint32_t)c << (4 * j);
      td.invc[j] = 1.0f / (float)c;
    }
    td.cnt4 = cnt4;
#pragma unroll
    for (int k = 1; k < KT; ++k) {
      td.rk[k] = ti.rk[k];
      const float s0 = s_lookup<0, SLDS>(p, s_lds, ti.rk[k], sh.R, gl);
      const float s1v = s_lookup<1, SLDS>(p, s_lds, ti.rk[k], sh.R, gl);
      const float s2 = s_lookup<2, SLDS>(p, s_lds, ti.rk[k], sh.R, gl);
      const float s3 = s_lookup<3, SLDS>(p, s_lds, ti.rk[k], sh.R, gl);
      td.sb[0] += k < (int)(cnt4 & 15u) ? s0 : 0.f;
      td.sb[1] += k < (int)((cnt4 >> 4) & 15u) ? s1v : 0.f;
      td.sb[2] += k < (int)((cnt4 >> 8) & 15u) ? s2 : 0.f;
      td.sb[3] += k < (int)((cnt4 >> 12) & 15u) ? s3 : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) td.sb[j] *= td.invc[j];
  }
  const uint32_t rv0 = (uint32_t)min(row_bcast<4>(raw), sh.R - 1);
  const uint32_t rv1 = (uint32_t)min(row_bcast<5>(raw), sh.R - 1);
  const uint32_t rv2 = (uint32_t)min(row_bcast<6>(raw), sh.R - 1);
  const uint32_t rv3 = (uint32_t)min(row_bcast<7>(raw), sh.R - 1);
  {
    const Frag a = ldg<Frag>(p.refsV, (rv0 * kD + n16 * 8) * 2u);
    const Frag b = ldg<Frag>(p.refsV, (rv1 * kD + n16 * 8) * 2u);
    td.xv[0][0] = Frag{a.x, a.y, b.x, b.y};
    td.xv[0][1] = Frag{a.z, a.w, b.z, b.w};
  }
  {
    const Frag a = ldg<Frag>(p.refsV, (rv2 * kD + n16 * 8) * 2u);
    const Frag b = ldg<Frag>(p.refsV, (rv3 * kD + n16 * 8) * 2u);
    td.xv[1][0] = Frag{a.x, a.y, b.x, b.y};
    td.xv[1][1] = Frag{a.z, a.w, b.z, b.w};
  }
  if (CODED && Q4 && SEL) {
    // Token lists: rows from the list; a reference position reads zeros.
    const int c = q4 * 8;
    const int col = 4 * ((n16 & 7) & ~1);
    const bool kb = ti.rb >= 0, vb = ti.rc >= 0;
    const uint32_t ua = (uint32_t)ti.rb, u = (uint32_t)ti.rc;
    td.ckq = ldg<uint32_t>(kb ? (const void*)p.qK : (const void*)kZeroCodes,
                           kb ? ua * (uint32_t)(dc / 2) + (uint32_t)(c < dc ? c : 0) / 2u : 0u);
    td.scl = ldg<uint16_t>(kb ? (const void*)p.sclK : (const void*)kOnePair, kb ? ua * 2u : 0u);
    td.cvq = ldg<uint32_t>(vb ? (const void*)p.qV : (const void*)kZeroCodes,
                           vb ? u * (uint32_t)(dc / 2) + (uint32_t)(col < dc ? col : 0) / 2u : 0u);
    td.sclv = ldg<uint16_t>(vb ? (const void*)p.sclV : (const void*)kOnePair, vb ? u * 2u : 0u);
  } else if (CODED && SEL) {
    const int c = q4 * 8;
    const bool kb = ti.rb >= 0;
    td.ck[0] = ldg<Frag>(kb ? (const void*)p.codesK : (const void*)kZeroCodes,
                         kb ? ((uint32_t)ti.rb * dc + (c < dc ? c : 0)) * 2u : 0u);
    const int cc = n16 & 7;
    const int col = 4 * (cc & ~1);
    const bool in_code = col < dc, vb = ti.rc >= 0;
    const void* vbase = in_code ? (vb ? (const void*)p.codesV : (const void*)kZeroCodes) : (const void*)kOnePair;
    td.cv = ldg<Frag>(vbase, in_code && vb ? ((uint32_t)ti.rc * dc + col) * 2u : 0u);
  } else if (CODED && Q4) {
    // 4-bit codes (d_c <= 32): raw nibbles and the token's scale; the
    // operands are built in compute_tile, once the words have arrived.
    const int cnt = max(ti.cnt, 1);
    const uint32_t ua = ti.base + min(n16, cnt - 1);
    const int c = q4 * 8;
    td.ckq = ldg<uint32_t>(p.qK, ua * (uint32_t)(dc / 2) + (uint32_t)(c < dc ? c : 0) / 2u);
    // Key scale of token 4 q4 + n16 % 4: compute_tile hands lane i's to the
    // whole row by a DPP row broadcast.
    td.scl = ldg<uint16_t>(p.sclK, (ti.base + (uint32_t)min(q4 * 4 + (n16 & 3), cnt - 1)) * 2u);
    const int g2 = n16 >> 3, cc = n16 & 7;
    const int col = 4 * (cc & ~1);
    const uint32_t u = ti.base + min(q4 * 4 + 2 * g2 + (cc & 1), cnt - 1);
    td.cvq = ldg<uint32_t>(p.qV, u * (uint32_t)(dc / 2) + (uint32_t)(col < dc ? col : 0) / 2u);
    td.sclv = ldg<uint16_t>(p.sclV, u * 2u);
  } else if (CODED) {
    const int cnt = max(ti.cnt, 1);
    const uint32_t ua = ti.base + min(n16, cnt - 1);
#pragma unroll
    for (int ks = 0; ks < DCK; ++ks) {
      // Columns past d_c (only when d_c is not a multiple of 32) read the
      // row's own first columns; q' is zero there.
      const int c = ks * 32 + q4 * 8;
      td.ck[ks] = ldg<Frag>(p.codesK, (ua * dc + (c < dc ? c : 0)) * 2u);
    }
    if (DCK == 1) {
      // One 16-byte load per lane covers the tile's value codes: lanes
      // n16 < 8 load group 0, lanes n16 >= 8 group 1; within a group, lane
      // c = n16 % 8 loads token 4 q4 + 2 group + (c & 1) at columns
      // 4 (c & ~1) .. + 7 (compute_tile pairs the lanes up).
      const int g2 = n16 >> 3, c = n16 & 7;
      const int col = 4 * (c & ~1);
      const uint32_t u = ti.base + min(q4 * 4 + 2 * g2 + (c & 1), cnt - 1);
      const bool in_code = col < dc;
      td.cv = ldg<Frag>(in_code ? p.codesV : kOnePair, in_code ? (u * dc + col) * 2u : 0u);
    } else {
      // Lanes past the code columns read the 1.0 pair (the lane at column
      // d_c accumulates the weight sum; the others are never read).
      const bool in_code = n16 * 4 < dc;
      const uint16_t* vb = in_code ? p.codesV : kOnePair;
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) {
        const uint32_t u0 = ti.base + min(q4 * 4 + 2 * g2, cnt - 1);
        const uint32_t u1 = ti.base + min(q4 * 4 + 2 * g2 + 1, cnt - 1);
        const U32x2 a = ldg<U32x2>(vb, in_code ? (u0 * dc + n16 * 4) * 2u : 0u);
        const U32x2 b = ldg<U32x2>(vb, in_code ? (u1 * dc + n16 * 4) * 2u : 0u);
        td.bc[g2] = Frag{a.x, a.y, b.x, b.y};
      }
    }
  } else {
    const bool ones = n16 * 4 == dc;
    td.bc[0] = td.bc[1] = Frag{ones ? 0x3F80u : 0u, 0u, ones ? 0x3F80u : 0u, 0u};
  }
}

struct State {
  float m;         // running max (base-2 units) of query head n16 / 4
  f32x4 accr[2];   // value-reference accumulators of query head q4
  f32x4 accc;      // value-code accumulators (+ weight sum column)
};

// DPP lane moves within 16-lane rows: swap neighbours (quad_perm 1,0,3,2)
// and rotate by 8.
__device__ __forceinline__ uint32_t swap_pairs(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t ror8(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, true);
}

// Value-code B operands of both groups from the one 16-byte load per lane
// (d_c <= 32): a lane pair (c even, c + 1) holds tokens (a, b) at columns
// 4c .. 4c + 7; swapping halves gives lane c columns 4c .. 4c + 3 and lane
// c + 1 columns 4c + 4 .. 4c + 7 of both tokens, and group 1 sits 8 lanes
// up.  Lanes at or past column d_c get the 1.0 column (only the lane at d_c
// is read).
__device__ __forceinline__ void value_code_operands(const Frag& x, int n16, int dc, Frag* bc,
                                                    uint32_t one_bits = 0x3F80u) {
  const bool odd = n16 & 1;
  const uint32_t r0 = swap_pairs(odd ? x.x : x.z), r1 = swap_pairs(odd ? x.y : x.w);
  const Frag mine = odd ? Frag{r0, r1, x.z, x.w} : Frag{x.x, x.y, r0, r1};
  const Frag up = Frag{ror8(mine.x), ror8(mine.y), ror8(mine.z), ror8(mine.w)};
  const bool data = n16 * 4 < dc;
  const uint32_t one = n16 * 4 == dc ? one_bits : 0u;
  const Frag ones = Frag{one, 0u, one, 0u};
  bc[0] = data ? mine : ones;
  bc[1] = data ? up : ones;
}

// 4-bit codes: elements 2j and 2j + 1 of a nibble word as a bf16 pair
// (small integers are exact in bf16: the top half of their fp32 bits).
__device__ __forceinline__ uint32_t q4_pair_bf16(uint32_t w, int j) {
  const float a = (float)((int32_t)(w << (28 - 8 * j)) >> 28);
  const float b = (float)((int32_t)(w << (24 - 8 * j)) >> 28);
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
}

// k references per token: value rows of reference slot k of the tile's
// tokens 4 q4 + 2 G2 + {0, 1}, as the B operands of group G2 (a slot past a
// token's count reads the zero row).
template <int G2>
__device__ __forceinline__ void gather_refs(const Args& p, int R, const Tile& td, int k, int n16, Frag* x) {
  const int ca = (int)((td.cnt4 >> (8 * G2)) & 15u), cb = (int)((td.cnt4 >> (8 * G2 + 4)) & 15u);
  const int rw = k == 0 ? 0 : td.rk[k];
  const uint32_t ra = (uint32_t)min(row_bcast<4 + 2 * G2>(rw), R - 1);
  const uint32_t rb = (uint32_t)min(row_bcast<5 + 2 * G2>(rw), R - 1);
  const bool va = k < ca, vb = k < cb;
  const Frag a = ldg<Frag>(va ? (const void*)p.refsV : (const void*)kZeroCodes, va ? (ra * kD + n16 * 8) * 2u : n16 * 16u);
  const Frag b = ldg<Frag>(vb ? (const void*)p.refsV : (const void*)kZeroCodes, vb ? (rb * kD + n16 * 8) * 2u : n16 * 16u);
  x[0] = Frag{a.x, a.y, b.x, b.y};
  x[1] = Frag{a.z, a.w, b.z, b.w};
}

template <bool CODED, int DCK, bool Q4, bool SEL = false, int KT = 1>
__device__ __forceinline__ void compute_tile(const Tile& td, const Frag* qh, const Frag* ql, int n16, int q4, int dc,
                                             const uint32_t* sel, State& st, const Args& pa, int R) {
  float s[4] = {td.sb[0], td.sb[1], td.sb[2], td.sb[3]};
  if (CODED && Q4) {
    // Key codes: integer values as the A operand, the token's scale applied
    // to the fp32 product (exact operands, one rounding).
    const Frag ck = Frag{q4_pair_bf16(td.ckq, 0), q4_pair_bf16(td.ckq, 1), q4_pair_bf16(td.ckq, 2),
                         q4_pair_bf16(td.ckq, 3)};
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
    c = mfma16(ck, qh[0], c);
    c = mfma16(ck, ql[0], c);
    if constexpr (SEL) {
      // Token lists: the lane's scale is its key-code token's (n16).
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] += bf2f((uint16_t)__shfl((int)td.scl, 4 * q4 + i, 64)) * c[i];
    } else {
      s[0] += bf2f((uint16_t)row_bcast<0>((int)td.scl)) * c[0];
      s[1] += bf2f((uint16_t)row_bcast<1>((int)td.scl)) * c[1];
      s[2] += bf2f((uint16_t)row_bcast<2>((int)td.scl)) * c[2];
      s[3] += bf2f((uint16_t)row_bcast<3>((int)td.scl)) * c[3];
    }
  } else if (CODED) {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DCK; ++ks) {
      c = mfma16(td.ck[ks], qh[ks], c);
      c = mfma16(td.ck[ks], ql[ks], c);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] += c[i];
  }
  if constexpr (SEL) {
    const uint32_t vm = (uint32_t)td.cnt >> (q4 * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = (vm >> i) & 1u ? s[i] : -INFINITY;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = q4 * 4 + i < td.cnt ? s[i] : -INFINITY;
  }
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
  Frag bc[2] = {td.bc[0], td.bc[1]};
  Frag bl[2];   // 4-bit codes: low bf16 parts of the dequantized value codes
  if (CODED && Q4) {
    // Value codes scale * q (at most 12 significant bits) as exact bf16
    // hi + lo parts; the weight-sum column rides on the hi operand only.
    const float sv = bf2f((uint16_t)td.sclv);
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = sv * (float)((int32_t)(td.cvq << (28 - 8 * j)) >> 28);
      const float b = sv * (float)((int32_t)(td.cvq << (24 - 8 * j)) >> 28);
      hw[j] = pk_bf16(a, b);
      lw[j] = pk_bf16(a - __uint_as_float(hw[j] << 16), b - __uint_as_float(hw[j] & 0xFFFF0000u));
    }
    value_code_operands(Frag{hw[0], hw[1], hw[2], hw[3]}, n16, dc, bc);
    value_code_operands(Frag{lw[0], lw[1], lw[2], lw[3]}, n16, dc, bl, 0u);
  } else if (CODED && DCK == 1) {
    value_code_operands(td.cv, n16, dc, bc);
  }
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(s[i] - st.m);
  const uint32_t h01 = pk_bf16(p[0], p[1]), h23 = pk_bf16(p[2], p[3]);
  const uint32_t l01 = pk_bf16(p[0] - __uint_as_float(h01 << 16), p[1] - __uint_as_float(h01 & 0xFFFF0000u));
  const uint32_t l23 = pk_bf16(p[2] - __uint_as_float(h23 << 16), p[3] - __uint_as_float(h23 & 0xFFFF0000u));
  constexpr bool MK = CODED && KT > 1;
  Frag ahk[2], alk[2];   // MK: A operands of the weights p / cnt (reference part)
#pragma unroll
  for (int g2 = 0; g2 < 2; ++g2) {
    const uint32_t hp = g2 ? h23 : h01, lp = g2 ? l23 : l01;
    const Frag ah = Frag{__builtin_amdgcn_perm(hp, hp, sel[0]), __builtin_amdgcn_perm(hp, hp, sel[1]),
                         __builtin_amdgcn_perm(hp, hp, sel[2]), __builtin_amdgcn_perm(hp, hp, sel[3])};
    const Frag al = Frag{__builtin_amdgcn_perm(lp, lp, sel[0]), __builtin_amdgcn_perm(lp, lp, sel[1]),
                         __builtin_amdgcn_perm(lp, lp, sel[2]), __builtin_amdgcn_perm(lp, lp, sel[3])};
    if constexpr (!MK) {
      st.accr[0] = mfma16(ah, td.xv[g2][0], st.accr[0]);
      st.accr[0] = mfma16(al, td.xv[g2][0], st.accr[0]);
      st.accr[1] = mfma16(ah, td.xv[g2][1], st.accr[1]);
      st.accr[1] = mfma16(al, td.xv[g2][1], st.accr[1]);
    }
    st.accc = mfma16(ah, bc[g2], st.accc);
    st.accc = mfma16(al, bc[g2], st.accc);
    if (CODED && Q4) st.accc = mfma16(ah, bl[g2], st.accc);
  }
  if constexpr (MK) {
    // The reference part averages each token's references: weights p / cnt,
    // one pass of value-reference MFMAs per reference slot, the next slot's
    // rows gathered before the current slot's products.
    float q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = p[i] * td.invc[i];
    const uint32_t k01 = pk_bf16(q[0], q[1]), k23 = pk_bf16(q[2], q[3]);
    const uint32_t m01 = pk_bf16(q[0] - __uint_as_float(k01 << 16), q[1] - __uint_as_float(k01 & 0xFFFF0000u));
    const uint32_t m23 = pk_bf16(q[2] - __uint_as_float(k23 << 16), q[3] - __uint_as_float(k23 & 0xFFFF0000u));
#pragma unroll
    for (int g2 = 0; g2 < 2; ++g2) {
      const uint32_t hp = g2 ? k23 : k01, lp = g2 ? m23 : m01;
      ahk[g2] = Frag{__builtin_amdgcn_perm(hp, hp, sel[0]), __builtin_amdgcn_perm(hp, hp, sel[1]),
                     __builtin_amdgcn_perm(hp, hp, sel[2]), __builtin_amdgcn_perm(hp, hp, sel[3])};
      alk[g2] = Frag{__builtin_amdgcn_perm(lp, lp, sel[0]), __builtin_amdgcn_perm(lp, lp, sel[1]),
                     __builtin_amdgcn_perm(lp, lp, sel[2]), __builtin_amdgcn_perm(lp, lp, sel[3])};
    }
    Frag cur[2][2] = {{td.xv[0][0], td.xv[0][1]}, {td.xv[1][0], td.xv[1][1]}};
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      Frag nxt[2][2];
      if (k + 1 < KT) {
        gather_refs<0>(pa, R, td, k + 1, n16, nxt[0]);
        gather_refs<1>(pa, R, td, k + 1, n16, nxt[1]);
      }
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) {
        st.accr[0] = mfma16(ahk[g2], cur[g2][0], st.accr[0]);
        st.accr[0] = mfma16(alk[g2], cur[g2][0], st.accr[0]);
        st.accr[1] = mfma16(ahk[g2], cur[g2][1], st.accr[1]);
        st.accr[1] = mfma16(alk[g2], cur[g2][1], st.accr[1]);
      }
      if (k + 1 < KT) {
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
          cur[g2][0] = nxt[g2][0];
          cur[g2][1] = nxt[g2][1];
        }
      }
    }
  }
}

// One run of tiles of a wave: software pipeline, two tiles per trip
// (buffers A and B); the ordinals of tile t+2 and the data of tile t+1 are
// in flight while tile t computes.  The scheduling barriers keep the
// compiler from hoisting a tile's arithmetic above the next tile's loads.
// The ordinals of the first two tiles (ia, ib) come from the caller, which
// issues them early.
template <bool CODED, int DCK, typename IdxT, bool SLDS, bool Q4, bool SEL, int KT = 1>
__device__ __forceinline__ void run_tiles(const Args& p, const Shape& sh, const float* s_lds, int t0, int t1,
                                          int first, int last, int n16, int q4, const Frag* qh, const Frag* ql,
                                          const uint32_t* sel, TileIdx ia, TileIdx ib, State& st) {
  if (t0 >= t1) return;
  Tile da, db;
  load_data<CODED, DCK, SLDS, Q4, SEL, KT>(p, sh, s_lds, ia, n16, q4, da);
  for (int tt = t0; tt < t1; tt += 2) {
    load_tile_idx<CODED, SEL, IdxT, KT>(p, sh, tt + 2, t1, first, last, n16, q4, ia);
    load_data<CODED, DCK, SLDS, Q4, SEL, KT>(p, sh, s_lds, ib, n16, q4, db);
    __builtin_amdgcn_sched_barrier(0);
    compute_tile<CODED, DCK, Q4, SEL, KT>(da, qh, ql, n16, q4, sh.dc, sel, st, p, sh.R);
    __builtin_amdgcn_sched_barrier(0);
    load_tile_idx<CODED, SEL, IdxT, KT>(p, sh, tt + 3, t1, first, last, n16, q4, ib);
    load_data<CODED, DCK, SLDS, Q4, SEL, KT>(p, sh, s_lds, ia, n16, q4, da);
    __builtin_amdgcn_sched_barrier(0);
    compute_tile<CODED, DCK, Q4, SEL, KT>(db, qh, ql, n16, q4, sh.dc, sel, st, p, sh.R);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// W_up_V row i = tid % d of head bh % H (the output column that thread tid
// writes in store_partials), as 16-byte pieces; pieces past d_c repeat the
// last one and are never used.
__device__ __forceinline__ void load_wup_row(const DecodeArgs& a, const Shape& sh, int bh, int tid,
                                             Frag (&wr)[kMaxDc / 8]) {
  const int dc = sh.dc;
  const uint16_t* row = (const uint16_t*)a.wuv + (size_t)(bh % sh.H) * a.w_hs + (size_t)(tid % kD) * dc;
#pragma unroll
  for (int j = 0; j < kMaxDc / 8; ++j) wr[j] = ldg<Frag>(row, (uint32_t)min(j * 8, dc - 8) * 2u);
}

// Partial record of each query head g of a split block: [max, sum, out[d]],
// out = the block's value-reference sum plus W_up_V times its value-code
// sums, both weighted against the block's maximum, so the combine only
// merges splits.  red_acc [NW][4][d + 64] holds each wave's head-dim columns,
// then its code columns and the weight-sum column (at d_c); threads
// tid < G (d_c + 1) first sum the code columns over the waves into cs, then
// thread (g, i) = (tid / d, tid % d) writes out[i] with its row wr of W_up_V
// (load_wup_row).
template <int NW>
__device__ __forceinline__ void store_partials(const DecodeArgs& a, const Shape& sh, int bh, int sp, int tid,
                                               const float (*red_m)[4], const float* red_acc, float* cs,
                                               const Frag (&wr)[kMaxDc / 8]) {
  const int G = a.G, dc = sh.dc;
  if (tid < G * (dc + 1)) {
    const int g = tid / (dc + 1), j = tid % (dc + 1);
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += red_acc[(w * 4 + g) * (kD + 64) + kD + j];
    cs[g * (kMaxDc + 1) + j] = v;
  }
  __syncthreads();
  if (tid < G * kD) {
    const int g = tid / kD, i = tid % kD;
    float r = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) r += red_acc[(w * 4 + g) * (kD + 64) + i];
    const float* c = cs + g * (kMaxDc + 1);
    float u = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxDc / 8; ++j) {
      if (j * 8 < dc) {
        const Frag w = wr[j];
        u = fmaf(__uint_as_float(w.x << 16), c[8 * j + 0], u);
        u = fmaf(__uint_as_float(w.x & 0xFFFF0000u), c[8 * j + 1], u);
        u = fmaf(__uint_as_float(w.y << 16), c[8 * j + 2], u);
        u = fmaf(__uint_as_float(w.y & 0xFFFF0000u), c[8 * j + 3], u);
        u = fmaf(__uint_as_float(w.z << 16), c[8 * j + 4], u);
        u = fmaf(__uint_as_float(w.z & 0xFFFF0000u), c[8 * j + 5], u);
        u = fmaf(__uint_as_float(w.w << 16), c[8 * j + 6], u);
        u = fmaf(__uint_as_float(w.w & 0xFFFF0000u), c[8 * j + 7], u);
      }
    }
    float* part = a.part + (((size_t)bh * a.splits + sp) * G + g) * partial_rec(sh);
    part[2 + i] = r + u;
    if (i == 0) {
      float mx = red_m[0][g];
#pragma unroll
      for (int w = 1; w < NW; ++w) mx = fmaxf(mx, red_m[w][g]);
      part[0] = mx;
      part[1] = c[dc];
    }
  }
}

// Split boundaries (coded rows on 16-row boundaries).
__device__ __forceinline__ int split_lo(int n, int sp, int splits, int align) {
  int64_t x = (int64_t)n * sp / splits;
  return sp == splits ? n : (int)(x / align * align);
}

// Dynamic LDS: the S table (SLDS) and, after the tile loop, the wave-merge
// buffer in the same bytes.  SEL: the block's tiles are 16-entry runs of the
// sequence's token list (a.sel) instead of coded rows and references.
template <int DCK, typename IdxT, bool SLDS, bool Q4, bool SEL, int KT = 1>
__global__ __launch_bounds__(kThreads) void k_split_mfma(DecodeArgs a, Shape sh) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  __shared__ float red_m[kWaves][4];
  __shared__ float csum[4 * (kMaxDc + 1)];

  const int BH = sh.B * sh.H;
  const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
  const int bh = xcd + 8 * (kx / a.splits), sp = kx % a.splits;
  if (bh >= BH) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: tile ranges and bases stay scalar
  const int n16 = lane & 15, q4 = lane >> 4;
  const int G = a.G, dc = sh.dc;

  // Coded rows [n0, n1) and references [r0, r1); token lists: entries [n0, n1).
  const int nrow = SEL ? a.n_sel : sh.N;
  const int n0 = split_lo(nrow, sp, a.splits, 16), n1 = split_lo(nrow, sp + 1, a.splits, 16);
  const int r0 = SEL ? 0 : split_lo(sh.R, sp, a.splits, 1), r1 = SEL ? 0 : split_lo(sh.R, sp + 1, a.splits, 1);
  const int nct = (n1 - n0 + 15) / 16, nrt = (r1 - r0 + 15) / 16;
  const int nt = nct + nrt;
  const int t_beg = (int)((int64_t)nt * wave / kWaves), t_end = (int)((int64_t)nt * (wave + 1) / kWaves);

  Args p;
  const size_t sK = (size_t)bh * 2, sV = sK + 1;
  p.refsV = (const uint16_t*)a.refs + sV * sh.Rc * kD;
  p.codesK = (const uint16_t*)a.codes + sK * sh.Nc * dc;
  p.codesV = (const uint16_t*)a.codes + sV * sh.Nc * dc;
  p.idxK = (const IdxT*)a.idx + sK * sh.Nc * sh.K;   // rows of K ordinals
  p.idxV = (const IdxT*)a.idx + sV * sh.Nc * sh.K;
  p.score = a.score + (size_t)bh * sh.R * 4;
  p.qK = (const uint8_t*)a.codes + sK * sh.Nc * (dc / 2);
  p.qV = (const uint8_t*)a.codes + sV * sh.Nc * (dc / 2);
  p.sclK = Q4 ? (const uint16_t*)a.scales + sK * sh.Nc : kOnePair;
  p.sclV = Q4 ? (const uint16_t*)a.scales + sV * sh.Nc : kOnePair;
  p.list = SEL ? a.sel + (size_t)(bh / sh.H) * a.n_sel : nullptr;
  p.magic = SEL ? 0xFFFFFFFFu / (uint32_t)sh.s : 0u;

  // q'_g (g = n16 / 4) for the score B operands: loaded first and
  // unconditionally (clamped column, masked later by a 0/1 factor), so that
  // this load, the first ordinals and the S-table copy share one round trip.
  f32x4 qv[DCK][2];
  {
    const float* qp = a.qp + ((size_t)bh * G + min(n16 >> 2, G - 1)) * dc;
#pragma unroll
    for (int ks = 0; ks < DCK; ++ks) {
      const int k0 = min(ks * 32 + q4 * 8, dc - 8);
      qv[ks][0] = *reinterpret_cast<const f32x4*>(qp + k0);
      qv[ks][1] = *reinterpret_cast<const f32x4*>(qp + k0 + 4);
    }
  }
  // Ordinals of the wave's first two coded tiles: issued first, so that
  // their HBM round trip overlaps the S-table copy.
  const int c1 = min(t_end, nct);
  TileIdx ia = {0, 0, 0, 0, 0, 0, 0}, ib = {0, 0, 0, 0, 0, 0, 0};
  if (t_beg < c1) {
    load_tile_idx<true, SEL, IdxT, KT>(p, sh, t_beg, c1, n0, n1, n16, q4, ia);
    load_tile_idx<true, SEL, IdxT, KT>(p, sh, t_beg + 1, c1, n0, n1, n16, q4, ib);
  }
  // The head's S table into LDS, four rows per thread in flight at once.
  if (SLDS) {
    const f32x4* src = reinterpret_cast<const f32x4*>(p.score);
    f32x4* dst = reinterpret_cast<f32x4*>(lds);
    int i = tid;
    for (; i + 3 * kThreads < sh.R; i += 4 * kThreads) {
      const f32x4 v0 = src[i], v1 = src[i + kThreads], v2 = src[i + 2 * kThreads], v3 = src[i + 3 * kThreads];
      dst[i] = v0;
      dst[i + kThreads] = v1;
      dst[i + 2 * kThreads] = v2;
      dst[i + 3 * kThreads] = v3;
    }
    for (; i < sh.R; i += kThreads) dst[i] = src[i];
  }
  // Score B operands: q' split into bf16 hi + lo parts.
  Frag qh[DCK], ql[DCK];
#pragma unroll
  for (int ks = 0; ks < DCK; ++ks) {
    const float on = ((n16 >> 2) < G && ks * 32 + q4 * 8 < dc) ? 1.f : 0.f;
    const f32x4 v0 = qv[ks][0] * on, v1 = qv[ks][1] * on;
    const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      const uint32_t hp = pk_bf16(v[2 * k2], v[2 * k2 + 1]);
      qh[ks][k2] = hp;
      ql[ks][k2] = pk_bf16(v[2 * k2] - __uint_as_float(hp << 16), v[2 * k2 + 1] - __uint_as_float(hp & 0xFFFF0000u));
    }
  }
  // v_perm selectors that place a packed pair (p_a low, p_b high) at
  // positions e and 4 + e of an 8 x bf16 A operand (zeros elsewhere),
  // e = n16 % 4.
  uint32_t sel[4];
  {
    const int el = n16 & 3;
    const uint32_t lo_a = (el & 1) ? 0x01000c0cu : 0x0c0c0100u;  // p_a into half e&1
    const uint32_t lo_b = (el & 1) ? 0x03020c0cu : 0x0c0c0302u;  // p_b into half e&1
    const int dw = el >> 1;
    sel[0] = dw == 0 ? lo_a : 0x0c0c0c0cu;
    sel[1] = dw == 1 ? lo_a : 0x0c0c0c0cu;
    sel[2] = dw == 0 ? lo_b : 0x0c0c0c0cu;
    sel[3] = dw == 1 ? lo_b : 0x0c0c0c0cu;
  }
  if (SLDS) __syncthreads();

  State st;
  // Token lists may leave a wave (or a whole split) with no valid token: a
  // finite initial maximum keeps every weight 2^(s - m) at 0 rather than NaN
  // there, and is replaced by the first real score.
  st.m = SEL ? -3.0e38f : -INFINITY;
  st.accr[0] = st.accr[1] = st.accc = f32x4{0.f, 0.f, 0.f, 0.f};
  // The wave's tiles: coded tiles [0, nct) then reference tiles [nct, nt).
  run_tiles<true, DCK, IdxT, SLDS, Q4, SEL, KT>(p, sh, lds, t_beg, c1, n0, n1, n16, q4, qh, ql, sel, ia, ib, st);
  if (!SEL) {
    const int rt0 = max(t_beg, nct) - nct, rt1 = t_end - nct;
    TileIdx ra = {0, 0, 0, 0, 0, 0, 0}, rb = {0, 0, 0, 0, 0, 0, 0};
    if (rt0 < rt1) {
      load_idx<false, IdxT>(p, rt0, rt1, r0, r1, n16, q4, ra);
      load_idx<false, IdxT>(p, rt0 + 1, rt1, r0, r1, n16, q4, rb);
    }
    run_tiles<false, DCK, IdxT, SLDS, Q4, false>(p, sh, lds, rt0, rt1, r0, r1, n16, q4, qh, ql, sel, ra, rb, st);
  }

  Frag wr[kMaxDc / 8];
  load_wup_row(a, sh, bh, tid, wr);

  // ---- merge the block's waves (fixed order) ----
  if (lane < 16 && (n16 & 3) == 0) red_m[wave][n16 >> 2] = st.m;
  __syncthreads();  // also: every wave is done with the S table
  float* red_acc = lds;  // [kWaves][4][kD + 64]
  float mb = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) mb = fmaxf(mb, red_m[w][q4]);
  const float mw = red_m[wave][q4];
  const float wgt = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - mb);
  float* mine_acc = red_acc + (wave * 4 + q4) * (kD + 64);
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int i = 0; i < 4; ++i) mine_acc[n16 * 8 + hh * 4 + i] = st.accr[hh][i] * wgt;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (n16 * 4 + i <= dc) mine_acc[kD + n16 * 4 + i] = st.accc[i] * wgt;
  __syncthreads();
  store_partials<kWaves>(a, sh, bh, sp, tid, red_m, red_acc, csum, wr);
}

// ---------------------------------------------------------------------------
// split, histogram form, for splits that hold many more tokens than the head
// has references (batched decode: a few long splits per head).  The value
// side sum_t p_t x~V[ref(t)] equals sum_r w_r x~V[r] with w_r the summed
// weights of the tokens whose value reference is r, so each token adds its
// weight to an LDS histogram instead of gathering its reference row, and
// every reference row is read once at the end.
//
// All waves must then weight against one maximum per query head: the block
// works through its tiles in chunks of kHistTiles per wave.  Pass A scores a
// chunk (its ordinals and codes were loaded one chunk ahead) and publishes
// each wave's maxima; after a barrier every thread forms the same block
// maxima, and when one grew by more than kTau the histogram and the code
// accumulators are rescaled by the same factor; pass B then adds the weights
// 2^(s - M) to the histogram and runs the value-code MFMAs (with the weight
// sum column), as the token-tile split does.  The block's own reference
// positions are tokens with a zero code row and their own ordinal in both
// streams.  The histogram holds 64-bit fixed-point weights (scale 2^32,
// added with integer LDS atomics, so the sums do not depend on the order of
// the additions and the output stays deterministic).  A dense pass over the
// references then applies the weights with the token-tile split's
// value-reference MFMAs.
//
// The score MFMA's 16 output columns hold each query head four times (the
// four lanes of a quad).  Those four lanes split the chunk instead: lane e
// of a quad takes tile e, so the S lookups, masks, exponentials and
// histogram adds after the score MFMA run once per (token, query head).  The
// value-code MFMA of tile k, which spreads the weights over the quad's
// lanes, takes them from lane k of the quad by a DPP broadcast.
// ---------------------------------------------------------------------------

constexpr int kHistTiles = 4;   // tiles per wave per chunk: one per lane of a quad


// Lane K of each quad (four consecutive lanes), broadcast over the quad.
template <int K>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, K * 0x55, 0xF, 0xF, true);
}

// Maximum over each quad (quad_perm 1,0,3,2 then 2,3,0,1).
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true)));
  return fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true)));
}

struct HChunk {
  int ldk[4];             // K and V ordinal rows of tokens 4 q4 + i of the lane's own
  int ldv[4];             //   tile (tile n16 & 3 of the chunk), as loaded
  Frag ck[kHistTiles];    // key-code A operand rows (zero rows for references)
  Frag cv[kHistTiles];    // value-code pieces, as Tile::cv
};

// p (0 <= p <= 2^kTau) as a fixed-point integer at scale 2^32, truncated:
// floor(p) in the high word and floor(fract(p) 2^32) in the low one (the
// fraction and the power-of-two product are exact).
__device__ __forceinline__ unsigned long long fix32(float p) {
  const uint32_t hi = (uint32_t)p;
  const uint32_t lo = (uint32_t)(__builtin_amdgcn_fractf(p) * 4294967296.0f);
  return ((unsigned long long)hi << 32) | lo;
}

size_t hist_lds_bytes(const Shape& sh) {
  const size_t front = (size_t)sh.R * 4 * sizeof(float);
  const size_t red = (size_t)kRedFloats * sizeof(float);
  return (front > red ? front : red) + (size_t)4 * sh.R * sizeof(unsigned long long);
}

template <typename IdxT>
__global__ __launch_bounds__(kThreads) void k_split_hist(DecodeArgs a, Shape sh) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  __shared__ __attribute__((aligned(16))) float red_m[kWaves][4];
  __shared__ __attribute__((aligned(16))) float chunk_m[2][kWaves][4];   // by chunk parity
  __shared__ float csum[4 * (kMaxDc + 1)];

  const int BH = sh.B * sh.H;
  const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
  const int bh = xcd + 8 * (kx / a.splits), sp = kx % a.splits;
  if (bh >= BH) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: tile bases stay scalar
  const int n16 = lane & 15, q4 = lane >> 4;
  const int G = a.G, dc = sh.dc, R = sh.R;
  const int gl = n16 >> 2, e4 = n16 & 3;

  const int n0 = split_lo(sh.N, sp, a.splits, 16), n1 = split_lo(sh.N, sp + 1, a.splits, 16);
  const int r0 = split_lo(sh.R, sp, a.splits, 1), r1 = split_lo(sh.R, sp + 1, a.splits, 1);
  const int nct = (n1 - n0 + 15) / 16, nrt = (r1 - r0 + 15) / 16;
  const int nt = nct + nrt;
  const int t_beg = (int)((int64_t)nt * wave / kWaves), t_end = (int)((int64_t)nt * (wave + 1) / kWaves);
  const int nchunk = ((nt + kWaves - 1) / kWaves + kHistTiles - 1) / kHistTiles;

  Args p;
  const size_t sK = (size_t)bh * 2, sV = sK + 1;
  p.refsV = (const uint16_t*)a.refs + sV * sh.Rc * kD;
  p.codesK = (const uint16_t*)a.codes + sK * sh.Nc * dc;
  p.codesV = (const uint16_t*)a.codes + sV * sh.Nc * dc;
  p.idxK = (const IdxT*)a.idx + sK * sh.Nc;
  p.idxV = (const IdxT*)a.idx + sV * sh.Nc;
  p.score = a.score + (size_t)bh * sh.R * 4;

  float* s_tab = lds;   // [R][4]; the wave-merge buffer after the dense pass
  unsigned long long* hist = (unsigned long long*)(lds + max(R * 4, kRedFloats));   // [4][R]

  // Chunk loads: the wave's tile t = t_beg + kHistTiles c + k (clamped to a
  // tile of the block, masked when past the wave's range).
  auto tile_of = [&](int c, int k, int& tb, int& cnt, bool& coded, bool& live) {
    const int t = t_beg + c * kHistTiles + k;
    live = t < t_end;
    const int tc = min(t, nt - 1);
    coded = tc < nct;
    tb = coded ? n0 + 16 * tc : r0 + 16 * (tc - nct);
    cnt = coded ? min(16, n1 - tb) : min(16, r1 - tb);
  };
  // Loads through buffer descriptors whose range ends at the stream's last
  // coded row, so that rows past it (capacity rows, whatever they hold) read
  // as zeros without a clamp.  Per tile the base is a scalar; the lanes'
  // offsets are the same for every tile.  A reference tile reads through an
  // empty range: zero code rows.
  const uint32_t row_bytes = (uint32_t)dc * 2u;
  const int g2l = n16 >> 3, c7 = n16 & 7, colv = 4 * (c7 & ~1);
  const uint32_t voff_ck = ((uint32_t)n16 * dc + (q4 * 8 < dc ? q4 * 8 : 0)) * 2u;
  // Lanes past the code columns read nothing (their value-code operand is
  // the constant weight-sum column, formed from no loaded data).
  const uint32_t voff_cv = colv < dc ? ((uint32_t)(q4 * 4 + 2 * g2l + (c7 & 1)) * dc + colv) * 2u : 0x80000000u;
  const __amdgpu_buffer_rsrc_t r_idxK = buffer_rsrc(p.idxK, (uint32_t)sh.N * sizeof(IdxT));
  const __amdgpu_buffer_rsrc_t r_idxV = buffer_rsrc(p.idxV, (uint32_t)sh.N * sizeof(IdxT));
  auto issue = [&](int c, HChunk& L) {
#pragma unroll
    for (int k = 0; k < kHistTiles; ++k) {
      int tb, cnt;
      bool coded, live;
      tile_of(c, k, tb, cnt, coded, live);
      const uint32_t bytes = coded ? (uint32_t)(sh.N - tb) * row_bytes : 0u;
      L.ck[k] = __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(
                                             buffer_rsrc(p.codesK + (size_t)tb * dc, bytes), voff_ck, 0, 0));
      L.cv[k] = __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(
                                             buffer_rsrc(p.codesV + (size_t)tb * dc, bytes), voff_cv, 0, 0));
    }
    // The lane's own tile: the K and V ordinals of its four tokens.  A
    // reference tile uses its positions instead; its rows, below R <= N, are
    // read all the same, so the loads take no lane-dependent branch.
    int tb, cnt;
    bool coded, live;
    tile_of(c, e4, tb, cnt, coded, live);
    const uint32_t vo = (uint32_t)(tb + q4 * 4) * (uint32_t)sizeof(IdxT);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // Each ordinal its own load: an opaque offset keeps the compiler from
      // merging neighbours into one wider load, whose unpacking it could
      // then schedule ahead of the consuming chunk.
      uint32_t o = vo + (uint32_t)sizeof(IdxT) * i;
      asm("" : "+v"(o));
      if constexpr (sizeof(IdxT) == 2) {
        L.ldk[i] = (int)__builtin_amdgcn_raw_buffer_load_b16(r_idxK, o, 0, 0);
        L.ldv[i] = (int)__builtin_amdgcn_raw_buffer_load_b16(r_idxV, o, 0, 0);
      } else {
        L.ldk[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(r_idxK, o, 0, 0);
        L.ldv[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(r_idxV, o, 0, 0);
      }
    }
  };

  HChunk LA, LB;
  if (nchunk > 0) issue(0, LA);

  // S table into LDS; histogram cleared.
  {
    const f32x4* src = reinterpret_cast<const f32x4*>(p.score);
    f32x4* dst = reinterpret_cast<f32x4*>(s_tab);
    int i = tid;
    for (; i + 3 * kThreads < R; i += 4 * kThreads) {
      const f32x4 v0 = src[i], v1 = src[i + kThreads], v2 = src[i + 2 * kThreads], v3 = src[i + 3 * kThreads];
      dst[i] = v0;
      dst[i + kThreads] = v1;
      dst[i + 2 * kThreads] = v2;
      dst[i + 3 * kThreads] = v3;
    }
    for (; i < R; i += kThreads) dst[i] = src[i];
    for (int j = tid; j < 4 * R; j += kThreads) hist[j] = 0ull;
  }
  Frag qh[1], ql[1];
  {
    const int g = n16 >> 2;
    const float* qp = a.qp + ((size_t)bh * G + min(g, G - 1)) * dc;
    const int k0 = q4 * 8;
    const bool live = g < G && k0 < dc;
    const f32x4 v0 = live ? *reinterpret_cast<const f32x4*>(qp + k0) : f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x4 v1 = live ? *reinterpret_cast<const f32x4*>(qp + k0 + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
    const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      const uint32_t hp = pk_bf16(v[2 * k2], v[2 * k2 + 1]);
      qh[0][k2] = hp;
      ql[0][k2] = pk_bf16(v[2 * k2] - __uint_as_float(hp << 16), v[2 * k2 + 1] - __uint_as_float(hp & 0xFFFF0000u));
    }
  }
  uint32_t sel[4];
  {
    const int el = n16 & 3;
    const uint32_t lo_a = (el & 1) ? 0x01000c0cu : 0x0c0c0100u;
    const uint32_t lo_b = (el & 1) ? 0x03020c0cu : 0x0c0c0302u;
    const int dw = el >> 1;
    sel[0] = dw == 0 ? lo_a : 0x0c0c0c0cu;
    sel[1] = dw == 1 ? lo_a : 0x0c0c0c0cu;
    sel[2] = dw == 0 ? lo_b : 0x0c0c0c0cu;
    sel[3] = dw == 1 ? lo_b : 0x0c0c0c0cu;
  }
  __syncthreads();

  float M[4] = {-3.0e38f, -3.0e38f, -3.0e38f, -3.0e38f};   // block maxima per query head (base 2)
  f32x4 accc = {0.f, 0.f, 0.f, 0.f};                         // value codes + weight sum, query head q4

  auto chunk = [&](int c, HChunk& L, HChunk& Lnext) {
    // This chunk's loaded registers become usable here, after the previous
    // chunk's barrier (empty asm, ordered with the barrier): otherwise the
    // scheduler may hoist their first uses into the previous chunk, whose
    // wait would then also cover the loads it had just issued.
#pragma unroll
    for (int k = 0; k < kHistTiles; ++k) asm volatile("" : "+v"(L.ck[k]), "+v"(L.cv[k]));
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(L.ldk[i]), "+v"(L.ldv[i]));
    // ---- pass A: scores of the lane's own tile ----
    f32x4 cs4[kHistTiles];
#pragma unroll
    for (int k = 0; k < kHistTiles; ++k) {
      f32x4 cs = {0.f, 0.f, 0.f, 0.f};
      cs = mfma16(L.ck[k], qh[0], cs);
      cs4[k] = mfma16(L.ck[k], ql[0], cs);
    }
    int tb, cnt;
    bool coded, live;
    tile_of(c, e4, tb, cnt, coded, live);
    const int vm = live ? cnt : 0;
    float sc[4], sb[4];
    int rv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pos = tb + q4 * 4 + i;
      const int rk = min(coded ? L.ldk[i] : pos, R - 1);
      rv[i] = min(coded ? L.ldv[i] : pos, R - 1);
      sb[i] = s_tab[(uint32_t)rk * 4 + gl];
    }
    float wmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float csi = pick4(cs4[0][i], cs4[1][i], cs4[2][i], cs4[3][i], e4);
      // All ones when token 4 q4 + i is valid (a sign shift, so that no
      // branch forms around the score).
      const uint32_t valid = (uint32_t)((q4 * 4 + i - vm) >> 31);
      const float sv = bsel(valid, sb[i] + csi, -INFINITY);
      sc[i] = sv;
      wmax = fmaxf(wmax, sv);
    }
    // The next chunk's loads fly through the barriers and pass B (issued
    // once this chunk's ordinals and key codes are consumed).  They are
    // issued after the last chunk too (its tiles clamped into the block):
    // with the loads unconditional, the compiler can count exactly which are
    // still in flight, so pass B waits only for this chunk's value codes.
    issue(c + 1, Lnext);
    wmax = quad_max(wmax);
    wmax = fmaxf(wmax, __shfl_xor(wmax, 16, 64));
    wmax = fmaxf(wmax, __shfl_xor(wmax, 32, 64));
    // Maxima slots alternate with the chunk's parity: a wave may write the
    // next chunk's while a slower one still reads these.
    if (lane < 16 && e4 == 0) chunk_m[c & 1][wave][gl] = wmax;
    __syncthreads();
    // ---- block maxima and lazy rescale (the same decision in every thread) ----
    f32x4 mx4 = {M[0], M[1], M[2], M[3]};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(&chunk_m[c & 1][w][0]);
#pragma unroll
      for (int g = 0; g < 4; ++g) mx4[g] = fmaxf(mx4[g], v[g]);
    }
    float alpha[4];
    bool grow_any = false;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const bool grow = mx4[g] > M[g] + kTau;
      alpha[g] = grow ? __builtin_amdgcn_exp2f(M[g] - mx4[g]) : 1.f;
      M[g] = grow ? mx4[g] : M[g];
      grow_any |= grow;
    }
    // Block-uniform (every thread computed the same maxima).  The barrier
    // above already follows every wave's adds of the earlier chunks.
    if (grow_any) {
      for (int j = tid; j < 4 * R; j += kThreads) {
        const float al = pick4(alpha, j / R);
        hist[j] = (unsigned long long)((double)hist[j] * (double)al);
      }
      accc *= pick4(alpha, q4);
      __syncthreads();
    }
    // ---- pass B: histogram weights of the own tile, then each tile's
    // value-code MFMAs with its weights from the quad's lane ----
    const float mg = pick4(M, gl);
    float pw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pw[i] = __builtin_amdgcn_exp2f(sc[i] - mg);
    // Every lane adds (the histogram has rows for all four query-head
    // slots; the dense pass reads only those of real heads).
    {
      unsigned long long* hg = hist + (size_t)gl * R;
#pragma unroll
      for (int i = 0; i < 4; ++i) atomicAdd(hg + rv[i], fix32(pw[i]));
    }
    const uint32_t h01 = pk_bf16(pw[0], pw[1]), h23 = pk_bf16(pw[2], pw[3]);
    const uint32_t l01 = pk_bf16(pw[0] - __uint_as_float(h01 << 16), pw[1] - __uint_as_float(h01 & 0xFFFF0000u));
    const uint32_t l23 = pk_bf16(pw[2] - __uint_as_float(h23 << 16), pw[3] - __uint_as_float(h23 & 0xFFFF0000u));
#pragma unroll
    for (int k = 0; k < kHistTiles; ++k) {
      Frag bc[2];
      value_code_operands(L.cv[k], n16, dc, bc);
      const uint32_t kh01 = k == 0 ? quad_bcast<0>(h01) : k == 1 ? quad_bcast<1>(h01) : k == 2 ? quad_bcast<2>(h01) : quad_bcast<3>(h01);
      const uint32_t kh23 = k == 0 ? quad_bcast<0>(h23) : k == 1 ? quad_bcast<1>(h23) : k == 2 ? quad_bcast<2>(h23) : quad_bcast<3>(h23);
      const uint32_t kl01 = k == 0 ? quad_bcast<0>(l01) : k == 1 ? quad_bcast<1>(l01) : k == 2 ? quad_bcast<2>(l01) : quad_bcast<3>(l01);
      const uint32_t kl23 = k == 0 ? quad_bcast<0>(l23) : k == 1 ? quad_bcast<1>(l23) : k == 2 ? quad_bcast<2>(l23) : quad_bcast<3>(l23);
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) {
        const uint32_t hp = g2 ? kh23 : kh01, lp = g2 ? kl23 : kl01;
        const Frag ah = Frag{__builtin_amdgcn_perm(hp, hp, sel[0]), __builtin_amdgcn_perm(hp, hp, sel[1]),
                             __builtin_amdgcn_perm(hp, hp, sel[2]), __builtin_amdgcn_perm(hp, hp, sel[3])};
        const Frag al = Frag{__builtin_amdgcn_perm(lp, lp, sel[0]), __builtin_amdgcn_perm(lp, lp, sel[1]),
                             __builtin_amdgcn_perm(lp, lp, sel[2]), __builtin_amdgcn_perm(lp, lp, sel[3])};
        accc = mfma16(ah, bc[g2], accc);
        accc = mfma16(al, bc[g2], accc);
      }
    }
  };
  for (int c = 0; c < nchunk; c += 2) {
    chunk(c, LA, LB);
    if (c + 1 < nchunk) chunk(c + 1, LB, LA);
  }
  __syncthreads();   // every weight is in the histogram

  // ---- dense pass: the reference part from the weighted rows ----
  f32x4 accr[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  {
    const int rt = (R + 15) / 16;
    const int rt0 = (int)((int64_t)rt * wave / kWaves), rt1 = (int)((int64_t)rt * (wave + 1) / kWaves);
    auto load_rows = [&](int t, Frag (&x)[2][2]) {
      const int base = 16 * min(t, rt - 1) + 4 * q4;
      const uint32_t ra = (uint32_t)min(base + 0, R - 1), rb = (uint32_t)min(base + 1, R - 1);
      const uint32_t rc = (uint32_t)min(base + 2, R - 1), rd = (uint32_t)min(base + 3, R - 1);
      const Frag fa = ldg<Frag>(p.refsV, (ra * kD + n16 * 8) * 2u), fb = ldg<Frag>(p.refsV, (rb * kD + n16 * 8) * 2u);
      const Frag fc = ldg<Frag>(p.refsV, (rc * kD + n16 * 8) * 2u), fd = ldg<Frag>(p.refsV, (rd * kD + n16 * 8) * 2u);
      x[0][0] = Frag{fa.x, fa.y, fb.x, fb.y};
      x[0][1] = Frag{fa.z, fa.w, fb.z, fb.w};
      x[1][0] = Frag{fc.x, fc.y, fd.x, fd.y};
      x[1][1] = Frag{fc.z, fc.w, fd.z, fd.w};
    };
    // One reference tile: weights of references 16 t + 4 q4 + i for query
    // head gl (zero past R, past the wave's range, or for unused heads).
    auto dense_tile = [&](int t, const Frag (&x)[2][2]) {
      const int base = 16 * t + 4 * q4;
      float w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = min(base + i, R - 1);
        const float v = (float)((double)hist[(size_t)min(gl, 3) * R + r] * 0x1p-32);
        w[i] = t < rt1 && base + i < R && gl < G ? v : 0.f;
      }
      const uint32_t h01 = pk_bf16(w[0], w[1]), h23 = pk_bf16(w[2], w[3]);
      const uint32_t l01 = pk_bf16(w[0] - __uint_as_float(h01 << 16), w[1] - __uint_as_float(h01 & 0xFFFF0000u));
      const uint32_t l23 = pk_bf16(w[2] - __uint_as_float(h23 << 16), w[3] - __uint_as_float(h23 & 0xFFFF0000u));
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) {
        const uint32_t hp = g2 ? h23 : h01, lp = g2 ? l23 : l01;
        const Frag ah = Frag{__builtin_amdgcn_perm(hp, hp, sel[0]), __builtin_amdgcn_perm(hp, hp, sel[1]),
                             __builtin_amdgcn_perm(hp, hp, sel[2]), __builtin_amdgcn_perm(hp, hp, sel[3])};
        const Frag al = Frag{__builtin_amdgcn_perm(lp, lp, sel[0]), __builtin_amdgcn_perm(lp, lp, sel[1]),
                             __builtin_amdgcn_perm(lp, lp, sel[2]), __builtin_amdgcn_perm(lp, lp, sel[3])};
        accr[0] = mfma16(ah, x[g2][0], accr[0]);
        accr[0] = mfma16(al, x[g2][0], accr[0]);
        accr[1] = mfma16(ah, x[g2][1], accr[1]);
        accr[1] = mfma16(al, x[g2][1], accr[1]);
      }
    };
    // Two row buffers in turn; loads past the range are clamped and their
    // weights are zero, so the loop body has no branch.
    Frag xa[2][2], xb[2][2];
    if (rt0 < rt1) load_rows(rt0, xa);
    for (int t = rt0; t < rt1; t += 2) {
      load_rows(min(t + 1, rt1 - 1), xb);
      dense_tile(t, xa);
      load_rows(min(t + 2, rt1 - 1), xa);
      dense_tile(t + 1, xb);
    }
  }

  Frag wr[kMaxDc / 8];
  load_wup_row(a, sh, bh, tid, wr);

  // ---- merge the block's waves: one maximum per query head, plain sums ----
  if (lane < 16 && (n16 & 3) == 0) red_m[wave][gl] = pick4(M, gl);
  __syncthreads();   // also: the S table is no longer read
  float* red_acc = lds;
  float* mine_acc = red_acc + (wave * 4 + q4) * (kD + 64);
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int i = 0; i < 4; ++i) mine_acc[n16 * 8 + hh * 4 + i] = accr[hh][i];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (n16 * 4 + i <= dc) mine_acc[kD + n16 * 4 + i] = accc[i];
  __syncthreads();
  store_partials<kWaves>(a, sh, bh, sp, tid, red_m, red_acc, csum, wr);
}

// combine of the general (VALU) split kernels, whose records hold
// [max, sum, code acc[d_c], reference acc[d]]: merges the splits of one
// (b, query head) and applies mu_V and W_up_V (the token-tile and histogram
// splits apply W_up_V themselves; k_combine_out merges theirs).
// Block L (256 threads) runs on XCD L % 8, the XCD of its head's
// split blocks; thread t owns column t of the partial records (code columns,
// then head-dim columns) and issues its loads of 32 splits at once, together
// with the split maxima and sums, so the records arrive in few round trips.
constexpr int kCombineBatch = 32;

__global__ __launch_bounds__(256) void k_combine(DecodeArgs a, Shape sh) {
  __shared__ float mls[2][kMfmaMaxSplits];
  __shared__ float accc[kMaxDc];
  __shared__ float red[1];
  const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
  const int bh = xcd + 8 * (kx / a.G), g = kx % a.G;
  if (bh >= sh.B * sh.H) return;
  const int b = bh / sh.H, h = bh % sh.H;
  const int gq = h * a.G + g;
  const int rec = partial_rec(sh), dc = sh.dc, ns = a.splits;
  const size_t pstride = (size_t)a.G * rec;
  const float* part = a.part + (size_t)bh * ns * pstride + (size_t)g * rec;
  const int t = threadIdx.x;
  const bool has_col = t < dc + kD;
  const float* pc = part + 2 + (has_col ? t : 0);
  // W_up_V row and mu_V of this thread's output column, loaded early.
  const int i_out = t - dc;
  const bool is_out = i_out >= 0 && has_col;
  const uint16_t* wuv = (const uint16_t*)a.wuv + (size_t)h * a.w_hs;
  // Every load is unconditional (clamped addresses) and masked afterwards
  // with arithmetic, so the compiler cannot turn a select into a branch that
  // waits: the W_up row, mu_V and the first 32 records arrive in one round
  // trip.
  const uint32_t io = is_out ? (uint32_t)i_out : 0u;
  U32x2 wrow[kMaxDc / 4];
#pragma unroll
  for (int j = 0; j < kMaxDc / 4; ++j)
    wrow[j] = ldg<U32x2>(wuv, (io * dc + (uint32_t)min(j * 4, dc - 4)) * 2u);
  const uint16_t mu_bits = ldg<uint16_t>(a.mu, ((uint32_t)(bh * 2 + 1) * kD + io) * 2u);
  // Records past the split count are not loaded (a uniform condition).
  float v[kCombineBatch];
#pragma unroll
  for (int k = 0; k < kCombineBatch; ++k) v[k] = k < ns ? pc[(size_t)k * pstride] : 0.f;
  const float col_on = has_col ? 1.f : 0.f;
#pragma unroll
  for (int k = 0; k < kCombineBatch; ++k) v[k] *= col_on;
#pragma unroll
  for (int j = 0; j < kMaxDc / 4; ++j) {
    const uint32_t m = 0u - (uint32_t)(is_out && j * 4 < dc);
    wrow[j] = U32x2{wrow[j].x & m, wrow[j].y & m};
  }
  const float muv = is_out ? bf2f(mu_bits) : 0.f;
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
  if (is_out) {
    float u = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxDc / 4; ++j) {
      if (j * 4 >= dc) break;
      u = fmaf(__uint_as_float(wrow[j].x << 16), accc[j * 4 + 0], u);
      u = fmaf(__uint_as_float(wrow[j].x & 0xFFFF0000u), accc[j * 4 + 1], u);
      u = fmaf(__uint_as_float(wrow[j].y << 16), accc[j * 4 + 2], u);
      u = fmaf(__uint_as_float(wrow[j].y & 0xFFFF0000u), accc[j * 4 + 3], u);
    }
    // l = 0 only when a selective decode attended no token: the output is 0.
    // A bit mask rather than a select keeps the compiler from branching (a
    // branch merge would wait for every load in flight).
    const float res = muv + (acc + u) / red[0];
    const uint32_t keep = 0u - (uint32_t)(red[0] > 0.f);
    a.out[((size_t)b * a.Hq + gq) * kD + i_out] = __uint_as_float(__float_as_uint(res) & keep);
  }
}

// combine of the token-tile and histogram splits, whose records hold
// [max, sum, out[d]] (store_partials).  Block L is one wave on XCD L % 8, the
// XCD of its head's split blocks, and owns 64 output columns of one
// (b, query head).  Per batch of 32 splits, lane j loads the (max, sum) pair
// of split j and every lane loads its column of each split at once; lane j
// forms split j's weight against the running maximum (wave reductions give
// the maximum and the weighted sum), and the weights reach every lane by
// readlane, so the merge needs no LDS and no barrier.  Columns add the
// splits in fixed order.
__global__ __launch_bounds__(64) void k_combine_out(DecodeArgs a, Shape sh) {
  const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
  const int per = 2 * a.G;
  const int bh = xcd + 8 * (kx / per), g = (kx % per) >> 1, half = kx & 1;
  if (bh >= sh.B * sh.H) return;
  const int b = bh / sh.H, h = bh % sh.H;
  const int rec = partial_rec(sh), ns = a.splits;
  const size_t pstride = (size_t)a.G * rec;
  const float* part = a.part + (size_t)bh * ns * pstride + (size_t)g * rec;
  const int lane = threadIdx.x, col = half * 64 + lane;
  const float muv = bf2f(ldg<uint16_t>(a.mu, ((uint32_t)(bh * 2 + 1) * kD + (uint32_t)col) * 2u));
  float M = -INFINITY, L = 0.f, acc = 0.f;
  for (int s0 = 0; s0 < ns; s0 += kCombineBatch) {
    const f32x2 ml = *reinterpret_cast<const f32x2*>(part + (size_t)min(s0 + (lane & 31), ns - 1) * pstride);
    float v[kCombineBatch];
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k) v[k] = part[(size_t)min(s0 + k, ns - 1) * pstride + 2 + col];
    // Lane j < 32: split s0 + j (lanes past the batch or the split count
    // hold no split).
    const float mj = lane < kCombineBatch && s0 + lane < ns ? ml.x : -INFINITY;
    const float bm = fmaxf(M, wave_max(mj));
    // What is summed so far, to the new maximum (nothing when M = -inf;
    // a factor of exactly 1 when the maximum stays).
    const float r = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - bm);
    M = bm;
    const float w = mj == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mj - M);
    L = fmaf(L, r, wave_sum(w * ml.y));
    acc *= r;
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j)
      acc = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j)), v[j], acc);
  }
  // L = 0 only when a selective decode attended no token: the output is 0.
  const float res = muv + acc / L;
  const uint32_t keep = 0u - (uint32_t)(L > 0.f);
  a.out[((size_t)b * a.Hq + h * a.G + g) * kD + col] = __uint_as_float(__float_as_uint(res) & keep);
}

size_t split_lds_bytes(const Shape& sh, bool slds) {
  const size_t red = (size_t)kRedFloats * sizeof(float);
  const size_t s = slds ? (size_t)sh.R * 4 * sizeof(float) : 0;
  return s > red ? s : red;
}

template <int DCK, typename IdxT, bool SLDS, bool SEL>
hipError_t launch_split(const Shape& sh, const DecodeArgs& a, hipStream_t st, dim3 grid) {
  // gfx950 gives a workgroup up to 160 KB of LDS; dynamic sizes above 64 KB
  // need no opt-in attribute on this runtime.  4-bit codes and token lists:
  // d_c <= 32 only.
  if (DCK == 1 && sh.q4)
    return launch_lds(k_split_mfma<1, IdxT, SLDS, true, SEL>, grid, kThreads, split_lds_bytes(sh, SLDS), st,
                      ev_start(a.events, 1), ev_stop(a.events, 1), a, sh);
  return launch_lds(k_split_mfma<DCK, IdxT, SLDS, false, SEL && DCK == 1>, grid, kThreads,
                    split_lds_bytes(sh, SLDS), st, ev_start(a.events, 1), ev_stop(a.events, 1), a, sh);
}

template <int DCK, typename IdxT, bool SEL = false>
hipError_t launch_split_s(const Shape& sh, const DecodeArgs& a, hipStream_t st, dim3 grid) {
  return split_lds_bytes(sh, true) <= kSplitLdsMax ? launch_split<DCK, IdxT, true, SEL>(sh, a, st, grid)
                                                   : launch_split<DCK, IdxT, false, SEL>(sh, a, st, grid);
}

// k references per token (storage-dtype codes, d_c <= 32): KT = 4 serves
// k <= 4, KT = 8 the rest.
template <typename IdxT, bool SLDS>
hipError_t launch_split_topk(const Shape& sh, const DecodeArgs& a, hipStream_t st, dim3 grid) {
  const size_t lds = split_lds_bytes(sh, SLDS);
  if (sh.K <= 4)
    return launch_lds(k_split_mfma<1, IdxT, SLDS, false, false, 4>, grid, kThreads, lds, st, ev_start(a.events, 1),
                      ev_stop(a.events, 1), a, sh);
  return launch_lds(k_split_mfma<1, IdxT, SLDS, false, false, 8>, grid, kThreads, lds, st, ev_start(a.events, 1),
                    ev_stop(a.events, 1), a, sh);
}

template <typename IdxT>
hipError_t launch_split_topk_s(const Shape& sh, const DecodeArgs& a, hipStream_t st, dim3 grid) {
  return split_lds_bytes(sh, true) <= kSplitLdsMax ? launch_split_topk<IdxT, true>(sh, a, st, grid)
                                                   : launch_split_topk<IdxT, false>(sh, a, st, grid);
}

}  // namespace

bool mfma_side_kernels_supported(const Shape& sh, int G, int splits) {
  return sh.bf16 && sh.d == kD && G <= 4 && sh.dc <= kMaxDc && splits <= kMfmaMaxSplits;
}

bool decode_fused_supported(const Shape& sh, int G, int splits) {
  const bool codes_ok = sh.K == 1 ? (!sh.q4 || sh.dc <= 32) : (!sh.q4 && sh.dc <= 32);
  return codes_ok && mfma_side_kernels_supported(sh, G, splits);
}

// The histogram split serves storage-dtype codes with d_c <= 32 and one
// reference when each split holds at least four times as many coded tokens
// as the head has references (there the one pass over the references is far
// cheaper than a gather per token) and the S table and histogram fit in LDS.
bool decode_hist_supported(const Shape& sh, int G, int splits) {
  return sh.K == 1 && !sh.q4 && sh.dc <= 32 && mfma_side_kernels_supported(sh, G, splits) &&
         (int64_t)sh.N >= (int64_t)4 * sh.R * splits && hist_lds_bytes(sh) <= kSplitLdsMax;
}

bool decode_sel_fused_supported(const Shape& sh, int G, int splits) {
  return sh.K == 1 && sh.dc <= 32 && decode_fused_supported(sh, G, splits);
}

// The split kernel holds one 512-thread block per CU: about 256 blocks over
// the chip (32 per XCD), at least 512 tokens per split.
int decode_fused_auto_splits(const Shape& sh) {
  const int64_t heads_per_xcd = (sh.B * sh.H + 7) / 8;
  int64_t s = (32 + heads_per_xcd - 1) / heads_per_xcd;
  const int64_t by_len = (sh.T + 511) / 512;
  if (s > by_len) s = by_len;
  if (s < 1) s = 1;
  if (s > kMfmaMaxSplits) s = kMfmaMaxSplits;
  return (int)s;
}

hipError_t launch_refscore_mfma(const Shape& sh, const DecodeArgs& a, hipStream_t st) {
  const int BH8 = 8 * ((sh.B * sh.H + 7) / 8);
  const int chunks = (sh.R + kRsRefs - 1) / kRsRefs;
  return launch(k_refscore_mfma, dim3(BH8 * chunks), 256, st, ev_start(a.events, 0), ev_stop(a.events, 0), a, sh,
                chunks);
}

hipError_t launch_combine_mfma(const Shape& sh, const DecodeArgs& a, hipStream_t st) {
  const int BH8 = 8 * ((sh.B * sh.H + 7) / 8);
  return launch(k_combine, dim3(BH8 * a.G), 256, st, ev_start(a.events, 2), ev_stop(a.events, 2), a, sh);
}

hipError_t launch_decode_fused(const Shape& sh, const DecodeArgs& a, hipStream_t st) {
  const int BH8 = 8 * ((sh.B * sh.H + 7) / 8);
  hipError_t e = launch_refscore_mfma(sh, a, st);
  if (e != hipSuccess) return e;
  const dim3 grid(BH8 * a.splits);
  const bool i16 = sh.idx_bytes == 2;
  if (decode_hist_supported(sh, a.G, a.splits))
    e = i16 ? launch_lds(k_split_hist<uint16_t>, grid, kThreads, hist_lds_bytes(sh), st, ev_start(a.events, 1),
                         ev_stop(a.events, 1), a, sh)
            : launch_lds(k_split_hist<uint32_t>, grid, kThreads, hist_lds_bytes(sh), st, ev_start(a.events, 1),
                         ev_stop(a.events, 1), a, sh);
  else if (sh.K > 1)
    e = i16 ? launch_split_topk_s<uint16_t>(sh, a, st, grid) : launch_split_topk_s<uint32_t>(sh, a, st, grid);
  else if (sh.dc <= 32)
    e = i16 ? launch_split_s<1, uint16_t>(sh, a, st, grid) : launch_split_s<1, uint32_t>(sh, a, st, grid);
  else
    e = i16 ? launch_split_s<2, uint16_t>(sh, a, st, grid) : launch_split_s<2, uint32_t>(sh, a, st, grid);
  if (e != hipSuccess) return e;
  return launch(k_combine_out, dim3(BH8 * a.G * 2), 64, st, ev_start(a.events, 2), ev_stop(a.events, 2), a, sh);
}

hipError_t launch_decode_sel_fused(const Shape& sh, const DecodeArgs& a, hipStream_t st) {
  const int BH8 = 8 * ((sh.B * sh.H + 7) / 8);
  hipError_t e = launch_refscore_mfma(sh, a, st);
  if (e != hipSuccess) return e;
  const dim3 grid(BH8 * a.splits);
  e = sh.idx_bytes == 2 ? launch_split_s<1, uint16_t, true>(sh, a, st, grid)
                        : launch_split_s<1, uint32_t, true>(sh, a, st, grid);
  if (e != hipSuccess) return e;
  return launch(k_combine_out, dim3(BH8 * a.G * 2), 64, st, ev_start(a.events, 2), ev_stop(a.events, 2), a, sh);
}

}  // namespace dkv
