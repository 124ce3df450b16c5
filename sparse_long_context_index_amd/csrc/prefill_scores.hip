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
#include "dsa_common.hpp"
#include "indexer.hpp"
#include "kernels.hpp"

namespace dsa {

namespace {

constexpr int kGemmTok = 32;     // tokens per workgroup (8 per wave)
constexpr int kGemmKeys = 2048;  // keys per workgroup (128 blocks of 16)
constexpr int kGemmPF = 4;       // key blocks in flight per wave
constexpr int kGemmGroupT = 32;  // token tiles per L2 super-tile

constexpr int kRoundKeys = 16 * kGemmPF;            // keys per prefetch round
constexpr int kStageStride = kRoundKeys + 16;       // padded LDS row (one token)
static_assert(kRoundKeys == 16 * 4, "a round is 16 lanes x 4 keys of one stored row piece");

// one 16-key block against the wave's 8 tokens: 8 MFMAs, the ReLU-weighted
// head sums and the causal mask.  Lane group g gets the scores of tokens g
// (x) and g + 4 (y) for key kk + (lane % 16).  Blocks at or beyond Lk (the
// tail of the last tile) compute on clamped keys; their scores are not stored.
__device__ __forceinline__ float2 gemm_block(const i32x8 (&a)[8], const float* wv, const i32x8& b,
                                             int64_t kk, int t0, int64_t Lk, int T, int col, int grp) {
  const int64_t p0 = Lk - T + t0;                       // position of the wave's first token
  if (kk > p0 + 7) return make_float2(-INFINITY, -INFINITY);   // every key beyond every token
  f32x4 c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = mfma_f8_16x16x128(a[j], b, f32x4{0.f, 0.f, 0.f, 0.f});
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
  if (kk + 15 > p0) {                                   // the block crosses the causal edge
    const int64_t key = kk + col;
    if (key > p0 + grp) lo = -INFINITY;
    if (key > p0 + grp + 4) hi = -INFINITY;
  }
  return make_float2(lo, hi);
}

// A round's 8 x 64 scores, staged in the wave's LDS rows, leave as 16-byte
// stores: lane (c, g) writes keys 4c .. 4c+3 of tokens g and g + 4.  Rows
// that are not 16-byte aligned, the key tail and the token tail take 4-byte
// stores.
__device__ __forceinline__ void store_round(const float* st, int64_t rk, int t0, int64_t Lk, int T,
                                            float* __restrict__ scores, int64_t ld, int col, int grp) {
  const float4 v0 = *reinterpret_cast<const float4*>(st + grp * kStageStride + 4 * col);
  const float4 v1 = *reinterpret_cast<const float4*>(st + (grp + 4) * kStageStride + 4 * col);
  const int64_t key = rk + 4 * col;
  float* r0 = scores + (int64_t)(t0 + grp) * ld + key;
  float* r1 = scores + (int64_t)(t0 + grp + 4) * ld + key;
  const bool rows16 = (ld & 3) == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0;
  if (rows16 && rk + kRoundKeys <= Lk && t0 + 8 <= T) {   // wave-uniform
    // streaming stores: the score rows are read back only by a later kernel
    __builtin_nontemporal_store(f32x4{v0.x, v0.y, v0.z, v0.w}, reinterpret_cast<f32x4*>(r0));
    __builtin_nontemporal_store(f32x4{v1.x, v1.y, v1.z, v1.w}, reinterpret_cast<f32x4*>(r1));
    return;
  }
  const bool w0 = t0 + grp < T, w1 = t0 + grp + 4 < T;
  if (w0 && key < Lk) r0[0] = v0.x;
  if (w0 && key + 1 < Lk) r0[1] = v0.y;
  if (w0 && key + 2 < Lk) r0[2] = v0.z;
  if (w0 && key + 3 < Lk) r0[3] = v0.w;
  if (w1 && key < Lk) r1[0] = v1.x;
  if (w1 && key + 1 < Lk) r1[1] = v1.y;
  if (w1 && key + 2 < Lk) r1[2] = v1.z;
  if (w1 && key + 3 < Lk) r1[3] = v1.w;
}

__global__ __launch_bounds__(256) void idx_gemm_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint8_t* __restrict__ k_idx, int64_t Lk, int T, float* __restrict__ scores,
    int64_t ld, int64_t n_ttiles, int64_t n_ktiles, int64_t per_xcd) {
  // XCD-aware order: workgroup b runs on XCD b % 8; give each XCD a contiguous
  // range of logical tiles, ordered so consecutive tiles share a key tile
  // and a group of token tiles stays resident in that XCD's L2.
  const int64_t bid = blockIdx.x;
  const int64_t logical = (bid & 7) * per_xcd + (bid >> 3);
  const int64_t total = n_ttiles * n_ktiles;
  if (logical >= total) return;
  const int64_t gsz = kGemmGroupT * n_ktiles;
  const int64_t g = logical / gsz;
  const int64_t rem = logical - g * gsz;
  const int64_t g_tiles = (g + 1) * kGemmGroupT <= n_ttiles ? kGemmGroupT : n_ttiles - g * kGemmGroupT;
  const int64_t ktile = rem / g_tiles;
  const int64_t ttile = g * kGemmGroupT + rem % g_tiles;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int t0 = (int)(ttile * kGemmTok) + wave * 8;
  const int64_t s0 = ktile * kGemmKeys;
  if (t0 >= T) return;                                 // wave-uniform

  // the wave's 8 x 16 head weights sit in LDS (registers go to the operands)
  __shared__ __attribute__((aligned(16))) float wsm[4][8 * 16];
  {
    const int j = lane >> 3, h = 2 * (lane & 7);
    const int t = t0 + j < T ? t0 + j : T - 1;
    wsm[wave][j * 16 + h] = w[t * 16 + h];
    wsm[wave][j * 16 + h + 1] = w[t * 16 + h + 1];
  }
  const float* wv = wsm[wave];
  i32x8 a[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int t = t0 + j < T ? t0 + j : T - 1;
    a[j] = load_frag32_cached(q_idx + (size_t)(t * 16 + col) * 128 + 32 * grp);
  }
  // key blocks beyond the last visible key of the wave's last token need no
  // operand; their loads are clamped into the cache
  const int64_t last = Lk - 1;
  const bool tail = s0 + kGemmKeys > Lk;               // wave-uniform
  const uint8_t* kp = k_idx + (s0 + col) * 128 + 32 * grp;
  auto load_b = [&](int kb) {
    if (!tail) return load_frag32_cached(kp + kb * 16 * 128);
    const int64_t key = s0 + kb * 16 + col;
    return load_frag32_cached(k_idx + (key < last ? key : last) * 128 + 32 * grp);
  };
  constexpr int NB = kGemmKeys / 16;
  static_assert(NB % kGemmPF == 0, "whole prefetch rounds");
  i32x8 b[kGemmPF];
#pragma unroll
  for (int u = 0; u < kGemmPF; ++u) b[u] = load_b(u);
  const int64_t end = Lk - s0 < kGemmKeys ? Lk - s0 : kGemmKeys;   // keys of this tile
  __shared__ __attribute__((aligned(16))) float stage[4][8 * kStageStride];
  float* st = stage[wave];
#pragma unroll 1
  for (int kb = 0; kb < NB; kb += kGemmPF) {
    if ((int64_t)kb * 16 >= end) break;                // wave-uniform
#pragma unroll
    for (int u = 0; u < kGemmPF; ++u) {
      const i32x8 cur = b[u];
      const int nb = kb + kGemmPF + u;
      b[u] = load_b(nb < NB ? nb : NB - 1);           // unconditional: no branch around the load
      const float2 v = gemm_block(a, wv, cur, s0 + (kb + u) * 16, t0, Lk, T, col, grp);
      st[grp * kStageStride + 16 * u + col] = v.x;
      st[(grp + 4) * kStageStride + 16 * u + col] = v.y;
    }
    store_round(st, s0 + kb * 16, t0, Lk, T, scores, ld, col, grp);
  }
}

}  // namespace

hipError_t launch_idx_gemm(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t Lk, int T,
                           float* scores, int64_t ld, hipStream_t st) {
  const int64_t n_ttiles = cdiv(T, kGemmTok);
  const int64_t n_ktiles = cdiv(Lk, kGemmKeys);
  const int64_t per_xcd = cdiv(n_ttiles * n_ktiles, 8);
  const int64_t nblocks = per_xcd * 8;
  if (nblocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(idx_gemm_kernel, dim3((unsigned)nblocks), dim3(256), 0, st, q_idx, w, k_idx,
                     Lk, T, scores, ld, n_ttiles, n_ktiles, per_xcd);
  return hipGetLastError();
}

}  // namespace dsa
