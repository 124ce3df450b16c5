// prefill_scores.hip -- lightning-indexer scores for many query tokens (the
// prefill chunk): S[t,s] = sum_h w[t,h] * max(q_idx[t,h,:] . k_idx[s,:], 0)
// for s <= p_t, -inf beyond ("Naive-N0.5-Flash: no full-attention layers, and
// a runtime built by AI", section "Inside a DSA layer: the lightning indexer").
//
// A [T*16 x 128] x [128 x Lk] contraction on the fp8 MFMA (16x16x128): the 16
// index heads of one token on M, 16 keys on N.  Workgroups take 32 tokens x
// 2048 keys in an XCD-aware order; each wave keeps its 8 tokens' operands in
// registers (its head weights in LDS) and streams 128 key blocks with 4 in
// flight.  Per block the eight MFMA tiles are issued first, then the
// ReLU-weighted sums; the row sums of four tokens share three permlane swaps
// and leave token r's score in lane row r.  Scores of a 64-key round are
// staged in LDS and leave as 16-byte stores.  The fp8 MFMA adds each group of
// 8 products after aligning them to the group's largest exponent, so its sums
// carry less precision than fp32 (measured and bounded in the tests).
//
// The candidate pass of the fused prefill top-k (kGemmCand) needs no scores,
// only a test against the row threshold with a proven margin, so it does the
// head sums on the bf16 matrix cores instead (gemm_block_cand): the VALU is
// what bounds the score modes (about 76 instructions per block of 8 MFMAs,
// issued while the matrix cores idle), and the candidate mode's blocks take
// 32.  Its candidates are recorded as per-lane bit masks over windows of 32
// blocks and emitted once per window, as key indices only.
//
// Built with MFMA results in VGPRs (no accumulation-register reads).
#include <type_traits>

#include "dsa_common.hpp"
#include "indexer.hpp"
#include "kernels.hpp"

namespace dsa {

namespace {

constexpr int kGemmTok = 32;     // tokens per workgroup (8 per wave)
constexpr int kGemmKeys = kPrefillTileKeys;  // keys per workgroup (128 blocks of 16)
constexpr int kGemmPF = 4;       // key blocks in flight per wave
constexpr int kGemmGroupT = 32;  // token tiles per L2 super-tile

constexpr int kRoundKeys = 16 * kGemmPF;            // keys per prefetch round
constexpr int kStageStride = kRoundKeys + 16;       // padded LDS row (one token)
static_assert(kRoundKeys == 16 * 4, "a round is 16 lanes x 4 keys of one stored row piece");

// one 16-key block against the wave's 8 tokens: 8 MFMAs, the ReLU-weighted
// head sums and the causal mask.  The block's keys are kk + step * c for
// c < 16; lane group g gets the scores of tokens g (x) and g + 4 (y) for key
// kk + step * (lane % 16).  Blocks at or beyond Lk (the tail of the last
// tile) compute on clamped keys; their scores are not used.  Blocks beyond
// every token of the wave are computed too and masked (a branch around them
// would cost every block a wait for all its loads; there are few such
// blocks).  The slot's next fragment is loaded (reload) once the MFMAs have
// read the current one, so the load can reuse the slot's registers: loaded
// into other registers, the ring of fragments would be copied back, and
// waited for, at every round.
template <class Reload>
__device__ __forceinline__ float2 gemm_block(const i32x8 (&a)[8], const float* wv, i32x8& slot, Reload reload,
                                             int64_t kk, int step, int t0, int64_t Lk, int T, int col, int grp) {
  const int64_t p0 = Lk - T + t0;                       // position of the wave's first token
  const i32x8 b = slot;
  f32x4 c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = mfma_f8_16x16x128(a[j], b, f32x4{0.f, 0.f, 0.f, 0.f});
  slot = reload();
  __builtin_amdgcn_sched_barrier(0);                    // all eight tiles in flight before the epilogue
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float4 w4 = *reinterpret_cast<const float4*>(wv + j * 16 + 4 * grp);
    const float ww[4] = {w4.x, w4.y, w4.z, w4.w};
    x[j] = relu_weighted_part(c[j], ww);
  }
  float lo = sum_rows4x4(x[0], x[1], x[2], x[3]);
  float hi = sum_rows4x4(x[4], x[5], x[6], x[7]);
  if (kk + 15 * step > p0) {                            // the block reaches the causal edge (wave-uniform)
    const int64_t key = kk + (int64_t)step * col;
    if (key > p0 + grp) lo = -INFINITY;
    if (key > p0 + grp + 4) hi = -INFINITY;
  }
  return make_float2(lo, hi);
}

// Candidate mode: the same 8 fp8 MFMA tiles, and the ReLU-weighted head sums
// on the matrix cores instead of the VALU.  The 32 logits a lane holds (heads
// 4 grp .. + 3 of its key for 8 tokens) are rounded to bf16 two at a time and
// clamped at zero as 16-bit integers (ReLU commutes with the rounding), which
// is exactly the B operand layout of a 16x16x32 bf16 MFMA whose k runs over
// (token pair, head); four such MFMAs against a block-diagonal weight operand
// (aw, fixed for the kernel) leave in lane (key, grp) the rows 4 grp + i:
// i = 0 / 1 the score of token grp / grp + 4, i = 2 / 3 the bound term
// sum_h |w_h| R_h of the same tokens (R_h the rounded ReLU logit).  Per block
// this takes 32 VALU instructions where the VALU epilogue takes 76, for four
// bf16 MFMAs; the bf16 rounding of R and w costs at most 2^-7 (1.012) of
// sum_h |w_h| R_h, which the candidate test adds to its margin.
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t relu_bf16x2(float a, float b) {
  const i16x2 v = __builtin_bit_cast(i16x2, f32x2_to_bf16x2_rne(a, b));
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(v, i16x2{0, 0}));
}

// The weight operands of the head-sum MFMAs: row m = 4 g + i holds the
// weights (i < 2) or their magnitudes (i >= 2) of token tm = g + 4 (i & 1),
// in MFMA tm / 2 and the k-half tm % 2 of its lane group's heads; every other
// entry is zero, so each output row sums one token's 16 heads exactly once.
__device__ __forceinline__ void cand_weight_operands(const float* w, int t0, int T, int col, int grp,
                                                     bf16x8 (&aw)[4]) {
  const int tm = (col >> 2) + 4 * (col & 1);
  const int t = t0 + tm < T ? t0 + tm : T - 1;
  const float* wp = w + (size_t)t * 16 + 4 * grp;
  uint32_t w01 = f32x2_to_bf16x2_rne(wp[0], wp[1]);
  uint32_t w23 = f32x2_to_bf16x2_rne(wp[2], wp[3]);
  if (col & 2) {
    w01 &= 0x7FFF7FFFu;
    w23 &= 0x7FFF7FFFu;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bool mine = q == (tm >> 1);
    const bool hi = (tm & 1) != 0;
    const u32x4 v = u32x4{mine && !hi ? w01 : 0u, mine && !hi ? w23 : 0u, mine && hi ? w01 : 0u,
                          mine && hi ? w23 : 0u};
    aw[q] = __builtin_bit_cast(bf16x8, v);
  }
}

template <class Reload>
__device__ __forceinline__ f32x4 gemm_block_cand(const i32x8 (&a)[8], const bf16x8 (&aw)[4], i32x8& slot,
                                                 Reload reload, int64_t kk, int t0, int64_t Lk, int T, int col,
                                                 int grp) {
  const int64_t p0 = Lk - T + t0;                       // position of the wave's first token
  const i32x8 b = slot;
  f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
  // two halves of four tokens: each half's logits feed two head-sum MFMAs,
  // so only four logit tiles are live at a time
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    f32x4 c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = mfma_f8_16x16x128(a[4 * hf + j], b, f32x4{0.f, 0.f, 0.f, 0.f});
    if (hf == 1) slot = reload();                       // the MFMAs have read the slot
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const u32x4 r = u32x4{relu_bf16x2(c[2 * q][0], c[2 * q][1]), relu_bf16x2(c[2 * q][2], c[2 * q][3]),
                            relu_bf16x2(c[2 * q + 1][0], c[2 * q + 1][1]),
                            relu_bf16x2(c[2 * q + 1][2], c[2 * q + 1][3])};
      d = mfma_bf16_16x16x32(aw[2 * hf + q], __builtin_bit_cast(bf16x8, r), d);
    }
  }
  if (kk + 15 > p0) {                                   // the block reaches the causal edge (wave-uniform)
    const int64_t key = kk + col;
    if (key > p0 + grp) d[0] = -INFINITY;
    if (key > p0 + grp + 4) d[1] = -INFINITY;
  }
  return d;
}

// A round's 8 x 64 scores, staged in the wave's LDS rows, leave as 16-byte
// stores: lane (c, g) writes columns 4c .. 4c+3 of tokens g and g + 4.  Rows
// that are not 16-byte aligned, the column tail and the token tail take
// 4-byte stores.
__device__ __forceinline__ void store_round(const float* st, int64_t rk, int t0, int64_t ncol, int T,
                                            float* __restrict__ scores, int64_t ld, int col, int grp) {
  const float4 v0 = *reinterpret_cast<const float4*>(st + grp * kStageStride + 4 * col);
  const float4 v1 = *reinterpret_cast<const float4*>(st + (grp + 4) * kStageStride + 4 * col);
  const int64_t key = rk + 4 * col;
  float* r0 = scores + (int64_t)(t0 + grp) * ld + key;
  float* r1 = scores + (int64_t)(t0 + grp + 4) * ld + key;
  const bool rows16 = (ld & 3) == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0;
  if (rows16 && rk + kRoundKeys <= ncol && t0 + 8 <= T) {   // wave-uniform
    // streaming stores: the score rows are read back only by a later kernel
    __builtin_nontemporal_store(f32x4{v0.x, v0.y, v0.z, v0.w}, reinterpret_cast<f32x4*>(r0));
    __builtin_nontemporal_store(f32x4{v1.x, v1.y, v1.z, v1.w}, reinterpret_cast<f32x4*>(r1));
    return;
  }
  const bool w0 = t0 + grp < T, w1 = t0 + grp + 4 < T;
  if (w0 && key < ncol) r0[0] = v0.x;
  if (w0 && key + 1 < ncol) r0[1] = v0.y;
  if (w0 && key + 2 < ncol) r0[2] = v0.z;
  if (w0 && key + 3 < ncol) r0[3] = v0.w;
  if (w1 && key < ncol) r1[0] = v1.x;
  if (w1 && key + 1 < ncol) r1[1] = v1.y;
  if (w1 && key + 2 < ncol) r1[2] = v1.z;
  if (w1 && key + 3 < ncol) r1[3] = v1.w;
}

// Candidate emission.  Each wave keeps, per token, up to kLocalCand
// candidates of its current tile in LDS and appends them to the row's global
// slots with one atomic add at the end of the tile.  A lane row (one token)
// finds its lanes' local positions from the ballot alone; a candidate past
// the local buffer goes straight to the global slots (one atomic per lane row
// and block).  Slots past cap are counted, not written.
constexpr int kLocalCand = 64;

__device__ __forceinline__ void emit_direct(bool ok, uint64_t mine, int lane, int t, uint32_t key, uint32_t s,
                                            const PrefillCand& pc) {
  uint32_t base = 0;
  const int leader = mine ? __builtin_ctzll(mine) : lane;
  if (mine && lane == leader) base = atomicAdd(pc.count + t, (uint32_t)__builtin_popcountll(mine));
  base = __shfl(base, leader, 64);
  if (ok) {
    const uint32_t pos = base + (uint32_t)__builtin_popcountll(mine & ((1ull << lane) - 1));
    if (pos < (uint32_t)pc.cap) pc.cand[(size_t)t * pc.cap + pos] = make_uint2(key, s);
  }
}

// lane row grp of a block: local position from the ballot, then LDS or (past
// the local buffer) the global slots
__device__ __forceinline__ void emit_local(bool ok, uint64_t m, int grp, int lane, uint32_t& cnt, uint2* lbuf,
                                           int t, uint32_t key, uint32_t s, const PrefillCand& pc) {
  const uint64_t mine = m & (0xFFFFull << (16 * grp));
  const uint32_t pos = cnt + (uint32_t)__builtin_popcountll(mine & ((1ull << lane) - 1));
  const uint32_t n = (uint32_t)__builtin_popcountll(mine);
  const bool spill = cnt + n > (uint32_t)kLocalCand;   // uniform in the lane row
  const uint64_t over = __ballot(ok && pos >= (uint32_t)kLocalCand) & (0xFFFFull << (16 * grp));
  if (ok && pos < (uint32_t)kLocalCand) lbuf[pos] = make_uint2(key, s);
  if (__ballot(spill)) emit_direct(ok && pos >= (uint32_t)kLocalCand, over, lane, t, key, s, pc);
  cnt = cnt + n < (uint32_t)kLocalCand ? cnt + n : (uint32_t)kLocalCand;
}

// end of a tile: every token's local candidates go to its global slots
__device__ __forceinline__ void flush_local(uint2* lb, const uint32_t* cnt_tok, int t0, int T, int lane,
                                            const PrefillCand& pc) {
#pragma unroll 1
  for (int j = 0; j < 8; ++j) {
    const uint32_t n = cnt_tok[j];                       // wave-uniform
    if (n == 0 || t0 + j >= T) continue;
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(pc.count + t0 + j, n);
    base = __shfl(base, 0, 64);
    if ((uint32_t)lane < n && base + lane < (uint32_t)pc.cap)
      pc.cand[(size_t)(t0 + j) * pc.cap + base + lane] = lb[j * kLocalCand + lane];
  }
}

// the float whose order key is u; order key 0 (every visible key) maps to the
// lowest finite float, which every finite score reaches and -inf does not
__device__ __forceinline__ float order_key_to_float(uint32_t u) {
  if (u == 0u) return -3.402823466e38f;
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// The candidate test of a row: score + cw * n_s >= the returned value, where
// cw * n_s bounds how far this contraction's score of key s can lie from the
// exact one.  The row's threshold is lowered by 2^-20 of its magnitude, which
// covers the float rounding of the test's product and sum.  No threshold
// (order key 0) gives the lowest finite float, which every finite score
// passes and a masked key (-inf) does not.
__device__ __forceinline__ float cand_threshold(uint32_t theta) {
  if (theta == 0u) return -3.402823466e38f;
  const float f = order_key_to_float(theta);
  return f - fabsf(f) * (1.0f / 1048576.0f);
}

enum GemmMode { kGemmScores = 0, kGemmSample = 1, kGemmCand = 2 };

// Candidate mode: margin factor for the bf16 head sums, applied to
// sum_h |w_h| R_h.  Rounding w and R to bf16 (unit roundoff 2^-8 each, both
// round to nearest even) moves a term w_h R_h by at most 2^-8 |w_h| R_h +
// 2^-8 |w_h| relu(l_h) <= 2^-7 (1 - 2^-8)^-2 |w~_h| R_h, the MFMA's exact
// products and fp32 sums add below 2^-19 of the same sum, and the computed
// sum of |w~_h| R_h is within 2^-19 of its exact value: 1/100 covers
// 2^-7 x 1.012 with a 26% margin.  The fp8 contraction's own error stays in
// the per-row factor cw (times the key norm bound).
constexpr float kCandRound = 0.01f;

struct GemmArgs {
  const float* cw;     // candidate mode: [T] per-row error factor (see PrefillCand)
  const float* knorm;  // candidate mode: [Lk] key norm bounds
  const uint8_t* q_idx;
  const float* w;
  const uint8_t* k_idx;
  int64_t Lk;
  int T;
  int step;            // key stride of the key space (1, or the sample stride)
  int64_t nkeys;       // keys of the key space: key j is key row j * step
  float* scores;       // score modes: [T][ld], column j = key j of the key space
  int64_t ld;
  PrefillCand cand;    // candidate mode
  SeqBatch sb;         // batch (score mode): grid dimension y is the sequence
  int64_t n_ttiles, n_ktiles, per_xcd;
};

// Waves per SIMD the launch bounds ask for, and key blocks in flight per wave.
// The candidate mode keeps more state per lane: with 4 blocks in flight it
// spills at 3 waves per SIMD (46.8 ms for the 8,192-token chunk's fused
// top-k), at 2 waves it takes 26.4 ms, with 2 blocks in flight at 3 waves
// 23.3 ms.
template <int kMode> struct GemmShape { static constexpr int waves = 3, pf = kGemmPF; };
template <> struct GemmShape<2> { static constexpr int waves = 3, pf = 2; };

template <int kMode>
__global__ __launch_bounds__(256, GemmShape<kMode>::waves) void idx_gemm_kernel(GemmArgs ga) {
  constexpr int PF = GemmShape<kMode>::pf;
  // XCD-aware order: workgroup b runs on XCD b % 8; give each XCD a contiguous
  // range of logical tiles, ordered so consecutive tiles share a key tile
  // and a group of token tiles stays resident in that XCD's L2.
  const int64_t bid = blockIdx.x;
  const int64_t logical = (bid & 7) * ga.per_xcd + (bid >> 3);
  const int64_t total = ga.n_ttiles * ga.n_ktiles;
  if (logical >= total) return;
  const int64_t gsz = kGemmGroupT * ga.n_ktiles;
  const int64_t g = logical / gsz;
  const int64_t rem = logical - g * gsz;
  const int64_t g_tiles = (g + 1) * kGemmGroupT <= ga.n_ttiles ? kGemmGroupT : ga.n_ttiles - g * kGemmGroupT;
  const int64_t ktile = rem / g_tiles;
  const int64_t ttile = g * kGemmGroupT + rem % g_tiles;

  const int T = ga.T;
  int64_t Lk = ga.Lk;
  const int step = kMode == kGemmSample ? ga.step : 1;
  if (kMode == kGemmScores && ga.sb.len) {
    const int b = blockIdx.y;
    int64_t first;
    Lk = seq_keys(ga.sb, b, &first);
    ga.q_idx += (size_t)b * T * 16 * 128;
    ga.w += (size_t)b * T * 16;
    ga.k_idx += first * 128;
    ga.scores += (size_t)b * T * ga.ld;
    ga.nkeys = Lk;
    if (Lk == 0) return;
  }
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int t0 = (int)(ttile * kGemmTok) + __builtin_amdgcn_readfirstlane(wave) * 8;   // wave-uniform
  const int64_t s0 = ktile * kGemmKeys;                // first key of the tile, in key-space units
  // candidate mode: the norm bounds of the tile's keys, staged in LDS once
  __shared__ float nsm[kMode == kGemmCand ? kGemmKeys : 1];
  if (kMode == kGemmCand) {
    for (int i = threadIdx.x; i < kGemmKeys; i += 256) {
      const int64_t key = s0 + i;
      nsm[i] = ga.knorm[key < Lk ? key : Lk - 1];
    }
    __syncthreads();
  }
  if (t0 >= T) return;                                 // wave-uniform

  // score modes: the wave's 8 x 16 head weights sit in LDS (registers go to
  // the operands); candidate mode: the head-sum MFMAs' weight operands
  constexpr bool kCand = kMode == kGemmCand;
  __shared__ __attribute__((aligned(16))) float wsm[kCand ? 1 : 4][kCand ? 1 : 8 * 16];
  const float* wv = wsm[kCand ? 0 : wave];
  bf16x8 aw[4];
  if constexpr (kCand) {
    cand_weight_operands(ga.w, t0, T, col, grp, aw);
  } else {
    const int j = lane >> 3, h = 2 * (lane & 7);
    const int t = t0 + j < T ? t0 + j : T - 1;
    wsm[wave][j * 16 + h] = ga.w[t * 16 + h];
    wsm[wave][j * 16 + h + 1] = ga.w[t * 16 + h + 1];
  }
  i32x8 a[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int t = t0 + j < T ? t0 + j : T - 1;
    a[j] = load_frag32_cached(ga.q_idx + (size_t)(t * 16 + col) * 128 + 32 * grp);
  }
  // key blocks beyond the key space are clamped into the cache (only the
  // last key tile has any: it runs a copy of the loop with the clamp, so the
  // loop body has no branch around its loads)
  const int64_t last = Lk - 1;
  const bool tail = (s0 + kGemmKeys) * step > Lk;      // wave-uniform
  const uint8_t* kp = ga.k_idx + (s0 + col) * step * 128 + 32 * grp;
  constexpr int NB = kGemmKeys / 16;
  static_assert(NB % PF == 0 && PF <= kGemmPF && 32 % PF == 0, "whole prefetch rounds and candidate windows");
  const int64_t end = ga.nkeys - s0 < kGemmKeys ? ga.nkeys - s0 : kGemmKeys;   // keys of this tile
  __shared__ __attribute__((aligned(16))) float stage[kMode == kGemmCand ? 1 : 4][8 * kStageStride];
  float* st = stage[kMode == kGemmCand ? 0 : wave];
  // candidate mode: the thresholds of this lane's two tokens, their local
  // candidate counts (uniform in a lane row) and the wave's LDS buffers
  float th0 = INFINITY, th1 = INFINITY;
  uint32_t c0 = 0, c1 = 0;
  __shared__ uint2 lcand[kMode == kGemmCand ? 4 : 1][kMode == kGemmCand ? 8 * kLocalCand : 1];
  __shared__ uint32_t lcnt[kMode == kGemmCand ? 4 : 1][8];
  float cw0 = 0.f, cw1 = 0.f;
  if (kMode == kGemmCand) {
    if (t0 + grp < T) {
      th0 = cand_threshold(ga.cand.theta[t0 + grp]);
      cw0 = ga.cw[t0 + grp];
    }
    if (t0 + grp + 4 < T) {
      th1 = cand_threshold(ga.cand.theta[t0 + grp + 4]);
      cw1 = ga.cw[t0 + grp + 4];
    }
  }

  auto main_loop = [&](auto tail_tag) {
    constexpr bool kTail = decltype(tail_tag)::value;
    auto load_b = [&](int kb) {
      if constexpr (!kTail) {
        return load_frag32_cached(kp + (int64_t)kb * 16 * step * 128);
      } else {
        const int64_t key = (s0 + kb * 16 + col) * step;
        return load_frag32_cached(ga.k_idx + (key < last ? key : last) * 128 + 32 * grp);
      }
    };
    i32x8 b[PF];
#pragma unroll
    for (int u = 0; u < PF; ++u) b[u] = load_b(u);
    // candidate mode: bit i of bm0 / bm1 marks block wb + i of the current
    // 32-block window as holding a candidate of token grp / grp + 4 in this
    // lane's key column; a window's keys are emitted together (the indices
    // only: the exact pass that follows rescores every candidate)
    uint32_t bm0 = 0, bm1 = 0;
    auto flush_window = [&](int wb) {
      uint2* lb = lcand[kCand ? wave : 0];
      for (;;) {
        const bool e0 = bm0 != 0u, e1 = bm1 != 0u;
        const uint64_t m0 = __ballot(e0), m1 = __ballot(e1);
        if (!(m0 | m1)) break;                           // wave-uniform
        const uint32_t key0 = (uint32_t)(s0 + (wb + (e0 ? __builtin_ctz(bm0) : 0)) * 16 + col);
        const uint32_t key1 = (uint32_t)(s0 + (wb + (e1 ? __builtin_ctz(bm1) : 0)) * 16 + col);
        bm0 &= bm0 - 1u;
        bm1 &= bm1 - 1u;
        if (m0) emit_local(e0, m0, grp, lane, c0, lb + grp * kLocalCand, t0 + grp, 0u, key0, ga.cand);
        if (m1) emit_local(e1, m1, grp, lane, c1, lb + (grp + 4) * kLocalCand, t0 + grp + 4, 0u, key1, ga.cand);
      }
    };
    int kb = 0;
#pragma unroll 1
    for (; kb < NB; kb += PF) {
      if ((int64_t)kb * 16 >= end) break;                // wave-uniform
      float nr[PF];                                      // candidate mode: the round's key norm bounds
      if constexpr (kCand) {
#pragma unroll
        for (int u = 0; u < PF; ++u) nr[u] = nsm[(kb + u) * 16 + col];
      }
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        const int nb = kb + PF + u;
        const int64_t kk = (s0 + (kb + u) * 16) * step;
        // the next fragment of this slot is loaded unconditionally (no branch around the load)
        auto next = [&] { return load_b(nb < NB ? nb : NB - 1); };
        if constexpr (kCand) {
          // a key is a candidate of token t when its score plus both error
          // margins reaches t's threshold: masked keys score -inf, which no
          // threshold admits, and tokens beyond T have threshold +inf
          const f32x4 d = gemm_block_cand(a, aw, b[u], next, kk, t0, Lk, T, col, grp);
          const bool ok0 = fmaf(kCandRound, d[2], fmaf(cw0, nr[u], d[0])) >= th0;
          const bool ok1 = fmaf(kCandRound, d[3], fmaf(cw1, nr[u], d[1])) >= th1;
          const uint32_t bit = 1u << ((kb + u) & 31);
          bm0 |= ok0 ? bit : 0u;
          bm1 |= ok1 ? bit : 0u;
        } else {
          const float2 v = gemm_block(a, wv, b[u], next, kk, step, t0, Lk, T, col, grp);
          st[grp * kStageStride + 16 * u + col] = v.x;
          st[(grp + 4) * kStageStride + 16 * u + col] = v.y;
        }
      }
      if constexpr (kCand) {
        if (((kb + PF) & 31) == 0) flush_window(kb + PF - 32);
      } else {
        store_round(st, s0 + kb * 16, t0, ga.nkeys, T, ga.scores, ga.ld, col, grp);
      }
    }
    if constexpr (kCand) flush_window(kb & ~31);         // a window cut short by the tile's end
  };
  if (tail)
    main_loop(std::true_type{});
  else
    main_loop(std::false_type{});
  if (kMode == kGemmCand) {
    // the lane rows' counts to LDS (one lane per row and token), then flush
    uint32_t* lc = lcnt[kMode == kGemmCand ? wave : 0];
    if (col == 0) {
      lc[grp] = c0;
      lc[grp + 4] = c1;
    }
    flush_local(lcand[kMode == kGemmCand ? wave : 0], lc, t0, T, lane, ga.cand);
  }
}

GemmArgs gemm_args(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t Lk, int T, int step) {
  GemmArgs ga{};
  ga.q_idx = q_idx;
  ga.w = w;
  ga.k_idx = k_idx;
  ga.Lk = Lk;
  ga.T = T;
  ga.step = step;
  ga.nkeys = cdiv(Lk, step);
  ga.n_ttiles = cdiv(T, kGemmTok);
  ga.n_ktiles = cdiv(ga.nkeys, kGemmKeys);
  ga.per_xcd = cdiv(ga.n_ttiles * ga.n_ktiles, 8);
  return ga;
}

template <int kMode>
hipError_t launch_gemm(const GemmArgs& ga, hipStream_t st, int batch = 1) {
  const int64_t nblocks = ga.per_xcd * 8;
  if (nblocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(idx_gemm_kernel<kMode>, dim3((unsigned)nblocks, (unsigned)batch), dim3(256), 0, st, ga);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_idx_gemm(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t Lk, int T,
                           float* scores, int64_t ld, hipStream_t st) {
  GemmArgs ga = gemm_args(q_idx, w, k_idx, Lk, T, 1);
  ga.scores = scores;
  ga.ld = ld;
  return launch_gemm<kGemmScores>(ga, st);
}

hipError_t launch_idx_gemm_batch(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, const SeqBatch& sb,
                                 int B, int T, float* scores, int64_t ld, hipStream_t st) {
  if (B < 1 || B > 65535 || ld < sb.max_len) return hipErrorInvalidValue;
  GemmArgs ga = gemm_args(q_idx, w, k_idx, sb.max_len, T, 1);
  ga.scores = scores;
  ga.ld = ld;
  ga.sb = sb;
  return launch_gemm<kGemmScores>(ga, st, B);
}

hipError_t launch_idx_gemm_sample(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t Lk, int T,
                                  int step, float* scores, int64_t ld, hipStream_t st) {
  if (step < 1 || ld < cdiv(Lk, step)) return hipErrorInvalidValue;
  GemmArgs ga = gemm_args(q_idx, w, k_idx, Lk, T, step);
  ga.scores = scores;
  ga.ld = ld;
  return launch_gemm<kGemmSample>(ga, st);
}

hipError_t launch_idx_gemm_cand(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t Lk, int T,
                                const PrefillCand& pc, hipStream_t st) {
  if (pc.cap < 1 || !pc.theta || !pc.count || !pc.cand || !pc.cw || !pc.knorm) return hipErrorInvalidValue;
  GemmArgs ga = gemm_args(q_idx, w, k_idx, Lk, T, 1);
  ga.cand = pc;
  ga.cw = pc.cw;
  ga.knorm = pc.knorm;
  return launch_gemm<kGemmCand>(ga, st);
}

}  // namespace dsa
