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

  // the wave's 8 x 16 head weights sit in LDS (registers go to the operands)
  __shared__ __attribute__((aligned(16))) float wsm[4][8 * 16];
  {
    const int j = lane >> 3, h = 2 * (lane & 7);
    const int t = t0 + j < T ? t0 + j : T - 1;
    wsm[wave][j * 16 + h] = ga.w[t * 16 + h];
    wsm[wave][j * 16 + h + 1] = ga.w[t * 16 + h + 1];
  }
  const float* wv = wsm[wave];
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
  static_assert(NB % PF == 0 && PF <= kGemmPF, "whole prefetch rounds");
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
#pragma unroll 1
    for (int kb = 0; kb < NB; kb += PF) {
      if ((int64_t)kb * 16 >= end) break;                // wave-uniform
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        const int nb = kb + PF + u;
        const int64_t kk = (s0 + (kb + u) * 16) * step;
        // the next fragment of this slot is loaded unconditionally (no branch around the load)
        const float2 v = gemm_block(a, wv, b[u], [&] { return load_b(nb < NB ? nb : NB - 1); }, kk, step, t0, Lk,
                                    T, col, grp);
        if (kMode == kGemmCand) {
          // a key is a candidate of token t when its score reaches t's
          // threshold: masked keys score -inf, which no threshold admits, and
          // tokens beyond T have threshold +inf
          const int64_t key = kk + col;
          const float ncur = nsm[(kb + u) * 16 + col];
          const bool ok0 = v.x + cw0 * ncur >= th0, ok1 = v.y + cw1 * ncur >= th1;
          const uint32_t k0 = order_key(v.x), k1 = order_key(v.y);
          const uint64_t m0 = __ballot(ok0), m1 = __ballot(ok1);
          if (m0 | m1) {                                 // wave-uniform
            uint2* lb = lcand[kMode == kGemmCand ? wave : 0];
            emit_local(ok0, m0, grp, lane, c0, lb + grp * kLocalCand, t0 + grp, k0, (uint32_t)key, ga.cand);
            emit_local(ok1, m1, grp, lane, c1, lb + (grp + 4) * kLocalCand, t0 + grp + 4, k1, (uint32_t)key,
                       ga.cand);
          }
        } else {
          st[grp * kStageStride + 16 * u + col] = v.x;
          st[(grp + 4) * kStageStride + 16 * u + col] = v.y;
        }
      }
      if (kMode != kGemmCand) store_round(st, s0 + kb * 16, t0, ga.nkeys, T, ga.scores, ga.ld, col, grp);
    }
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
