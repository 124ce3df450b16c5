// indexer.hpp -- pieces shared by the two lightning-indexer kernels (the
// decode scan and the prefill contraction): operand loads and the
// ReLU-weighted head sum of a 16x16 head x key MFMA tile ("Naive-N0.5-Flash:
// no full-attention layers, and a runtime built by AI", section "Inside a DSA
// layer: the lightning indexer").
#pragma once

#include "dsa_common.hpp"

namespace dsa {

__device__ __forceinline__ i32x8 load_frag32_cached(const uint8_t* p) {
  const i32x4* q = reinterpret_cast<const i32x4*>(p);
  i32x4 lo = q[0];
  i32x4 hi = q[1];
  i32x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// 32 fp8 bytes -> four bf16x8 MFMA operands (k-step s takes bytes 8s..8s+7)
__device__ __forceinline__ void widen_fp8(const i32x8& r, bf16x8* out) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)r[2 * s], 1.0f, false);
    bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)r[2 * s], 1.0f, true);
    bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)r[2 * s + 1], 1.0f, false);
    bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)r[2 * s + 1], 1.0f, true);
    out[s] = bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  }
}

// Sum over the four 16-lane rows of the wave, in the order (r0 + r1) + (r2 +
// r3), on the VALU: permlane16_swap pairs rows 0-1 and 2-3, permlane32_swap
// the two halves; every lane ends with the same bits.
__device__ __forceinline__ float sum_rows4(float s) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  s = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// max(x, 0) on the integer unit: a float whose sign bit is set is a negative
// int32, every other float keeps its bits (-0.0 becomes +0.0)
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// ReLU-weighted head sum for the key of this lane's column.  c holds heads
// 4*grp + {0..3}; wv the matching weights; the row sum adds the partial sums
// of the four lane groups.
__device__ __forceinline__ float relu_weighted_part(const f32x4& c, const float* wv) {
  float s = wv[0] * relu_bits(c[0]);
  s = fmaf(wv[1], relu_bits(c[1]), s);
  s = fmaf(wv[2], relu_bits(c[2]), s);
  s = fmaf(wv[3], relu_bits(c[3]), s);
  return s;
}

__device__ __forceinline__ float relu_weighted_sum(const f32x4& c, const float* wv) {
  return sum_rows4(relu_weighted_part(c, wv));
}

// Row sums of four values at once: x[i] holds token i's partial sums in the
// four rows; the result holds in row r the full sum of token r, added in the
// order (r0 + r1) + (r2 + r3).  permlane16_swap(a, b) leaves rows (a0, b0, a2,
// b2) and (a1, b1, a3, b3), permlane32_swap(u, v) leaves (u0, u1, v0, v1) and
// (u2, u3, v2, v3).
__device__ __forceinline__ float sum_rows4x4(float x0, float x1, float x2, float x3) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x0), __float_as_uint(x1), false, false);
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x2), __float_as_uint(x3), false, false);
  const float u = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const float v = __uint_as_float(q[0]) + __uint_as_float(q[1]);
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(u), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace dsa

namespace dsa {

// ---------------------------------------------------------------- exact scores
// One query token's operands for the exact index arithmetic of the decode
// scan: the 16 heads' fp8 bytes widened to bf16 (lane: head col, k-group grp)
// and the weights of the 4 heads whose logits the lane's accumulator holds.
struct ExactQuery {
  bf16x8 a[4];
  float wv[4];
};

__device__ __forceinline__ void load_exact_query(const uint8_t* q_t, const float* w_t, ExactQuery& eq) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  widen_fp8(load_frag32_cached(q_t + (size_t)col * 128 + 32 * grp), eq.a);
#pragma unroll
  for (int i = 0; i < 4; ++i) eq.wv[i] = w_t[4 * grp + i];
}

// The score of the key whose 32 bytes of k-group (lane / 16) this lane holds
// in kr (one key per lane column): fp8 widened to bf16 (lossless), four bf16
// MFMAs over the 128 dims (exact products, fp32 sums), the ReLU-weighted head
// sum.  Same operands in the same order as the decode scan, so the same bits;
// every lane of the column receives the score.
__device__ __forceinline__ float exact_score(const ExactQuery& eq, const i32x8& kr) {
  bf16x8 b[4];
  widen_fp8(kr, b);
  f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4) c = mfma_bf16_16x16x32(eq.a[k4], b[k4], c);
  return relu_weighted_sum(c, eq.wv);
}

// Exact scores of query token q_t / w_t against keys 0 .. n - 1 into row,
// by the NT threads of a workgroup (each wave takes 16-key tiles, U tiles'
// loads in flight).  Plain stores: the caller synchronises before reading.
template <int NT, int U>
__device__ __forceinline__ void exact_scores_block(const uint8_t* q_t, const float* w_t, const uint8_t* k_idx,
                                                   int64_t n, float* row) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  ExactQuery eq;
  load_exact_query(q_t, w_t, eq);
  const int64_t ntiles = cdiv(n, 16);
  for (int64_t t0 = (int64_t)wave * U; t0 < ntiles; t0 += (int64_t)(NT / 64) * U) {
    i32x8 kr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t key = (t0 + u) * 16 + col;
      kr[u] = load_frag32_cached(k_idx + (key < n ? key : n - 1) * 128 + 32 * grp);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t key = (t0 + u) * 16 + col;
      const float s = exact_score(eq, kr[u]);
      if (grp == 0 && key < n) row[key] = s;
    }
  }
}

}  // namespace dsa
