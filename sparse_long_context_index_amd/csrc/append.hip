// append.hip -- the step before the index sweep for T new tokens: LayerNorm,
// partial RoPE and fp8 rounding of the lightning indexer's key and queries,
// partial RoPE of the attention queries and keys, and the cache appends
// ("Naive-N0.5-Flash: no full-attention layers, and a runtime built by AI",
// section "Inside a DSA layer" and Figure 1, panel B; RoPE on a third of each
// head with base 10,000,000 on the sparse layers, same section).
//
// Grid (T, 5): workgroup y = 0 handles the indexer (key and 16 query heads),
// y = 1 + g the attention's KV head g (its 16 query heads, key and value).
// Every global load and store moves a whole 16-byte piece (8 bf16 dims); a
// thread keeps the pieces it loaded in registers and stages them in LDS, from
// which a rotated dim reads its pair partner.  The index key's LayerNorm runs
// on one wave while others build the rotation table.
//
// Rotation angles a_i = p * base^(-2i/R): an absolute position near 2^20 times
// a float32 frequency would lose most of the angle's fraction, so the
// frequency and the product are float64, reduced modulo 2 pi in float64
// (two-part Cody-Waite: 2 pi = C1 + C2 to about 107 bits, each step a fused
// multiply-add), and cos / sin of the reduced angle are evaluated in float64
// and rounded once to float32.
#include <cmath>

#include "dsa_common.hpp"
#include "kernels.hpp"

namespace dsa {

namespace {

constexpr int kAppendNT = 256;
constexpr int kQPerKv = DSA_Q_HEADS / DSA_KV_HEADS;  // 16
constexpr int kRowPieces = DSA_QK_DIM / 8;         // 16-byte pieces of a 192-dim bf16 row
constexpr int kIdxPieces = DSA_IDX_DIM / 8;        // of a 128-dim bf16 row

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Per-dim rotation table of one token: y_d = x_d C[d] + x_{pair(d)} S[d] with
// pair(d) = d + R/2 below R/2 and d - R/2 from R/2 to R; S carries the sign.
// Entries from R up to the next multiple of 8 hold C = 1, S = 0.
constexpr int kTab = DSA_QK_DIM;

struct RotTable {
  float C[kTab], S[kTab];
};

__device__ __forceinline__ int pair_of(int d, int R) {
  const int h = R >> 1;
  return d < h ? d + h : (d < R ? d - h : d);
}

// threads d < ceil8(R) fill entry d: a_i = p f_i with i = d mod R/2, where
// f_i = base^(-2i/R) comes from the host, computed there in float64
__device__ __forceinline__ void rot_table(RotTable& rt, int64_t p, int R, const double* freq) {
  constexpr double kTwoPi1 = 6.283185307179586232;     // nearest double to 2 pi
  constexpr double kTwoPi2 = 2.4492935982947064e-16;   // 2 pi - kTwoPi1
  constexpr double kInvTwoPi = 0.15915494309189535;
  const int d = threadIdx.x, h = R >> 1;
  if (d < R) {
    const int i = d < h ? d : d - h;
    const double a = (double)p * freq[i];
    const double kq = rint(a * kInvTwoPi);
    const double r = fma(-kq, kTwoPi2, fma(-kq, kTwoPi1, a));
    double sn, cs;
    sincos(r, &sn, &cs);
    rt.C[d] = (float)cs;
    rt.S[d] = d < h ? -(float)sn : (float)sn;
  } else if (d < ((R + 7) & ~7)) {
    rt.C[d] = 1.f;
    rt.S[d] = 0.f;
  }
}

// 8 rotated values of dims d0 .. d0+7 (d0 < R, a multiple of 8) from own
// values x, their pair partners xp and the table in LDS; kWhole: all 8 dims
// lie below R (no dim passes through)
template <bool kWhole = false>
__device__ __forceinline__ void rot8(float (&y)[8], const float (&x)[8], const float (&xp)[8], int d0, int R,
                                     const RotTable& rt) {
  const float4 c0 = *reinterpret_cast<const float4*>(&rt.C[d0]);
  const float4 c1 = *reinterpret_cast<const float4*>(&rt.C[d0 + 4]);
  const float4 s0 = *reinterpret_cast<const float4*>(&rt.S[d0]);
  const float4 s1 = *reinterpret_cast<const float4*>(&rt.S[d0 + 4]);
  const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) y[j] = kWhole || d0 + j < R ? fmaf(x[j], c[j], xp[j] * sv[j]) : x[j];
}

// the same with the partners read one by one from the staged row
template <class Row>
__device__ __forceinline__ void rotate8(float (&y)[8], const float (&x)[8], const Row& row, int d0, int R,
                                        const RotTable& rt) {
  float xp[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) xp[j] = row(pair_of(d0 + j, R));
  rot8(y, x, xp, d0, R, rt);
}

__device__ __forceinline__ void unpack_bf16x8(float (&x)[8], const uint4& u) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = __uint_as_float(w[j] << 16);
    x[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
  }
}

// 8 floats -> 8 fp8 e4m3 codes, round to nearest even, saturating at +-448:
// the values are clamped to [-448, 448] and converted by the hardware
// (v_cvt_pk_fp8_f32, OCP e4m3), which then rounds to nearest even with
// subnormals in steps of 2^-9; an exhaustive comparison over every finite
// float with the rounding written out from the format (bias 7, 3 fraction
// bits) found no difference.
__device__ __forceinline__ uint2 pack_e4m3x8(const float (&y)[8]) {
  float c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_fmed3f(y[j], -448.f, 448.f);
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(c[4 * h], c[4 * h + 1], 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(c[4 * h + 2], c[4 * h + 3], v, true);
    w[h] = (uint32_t)v;
  }
  return make_uint2(w[0], w[1]);
}

struct AppendArgs {
  const uint16_t* idx_q;
  const uint16_t* idx_k;
  const float* ln_gamma;
  const float* ln_beta;
  float ln_eps;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t Lk;
  int T;
  int rot_idx, rot_main;
  double freq_idx[DSA_IDX_DIM / 2];   // base^(-2i/R) of the rotated index-head dims
  double freq_main[DSA_QK_DIM / 2];   // base^(-2i/R) of the rotated attention-head dims
  uint8_t* q_idx_out;
  uint8_t* k_idx_cache;
  uint16_t* q_out;
  uint16_t* k_cache;
  uint16_t* v_cache;
};

struct IdxShared {
  uint16_t xq[DSA_IDX_HEADS][DSA_IDX_DIM];
  float kn[DSA_IDX_DIM];
};

struct MainShared {
  uint16_t xs[kQPerKv + 1][DSA_QK_DIM];            // 16 query heads, then the key
};

union AppendShared {
  IdxShared ix;
  MainShared mn;
};

constexpr int kLnWave = kAppendNT / 64 - 1;          // the wave that normalises the index key

// wave kLnWave: LayerNorm of the index key, mean and variance in float64 (two
// passes), one fp32 rounding before the gain and bias
__device__ __forceinline__ void index_key_norm(const AppendArgs& ar, IdxShared& sh, int t) {
  const int l = threadIdx.x & 63;
  const uint16_t* kin = ar.idx_k + (size_t)t * DSA_IDX_DIM;
  const float x0 = bf16_to_f32(kin[l]), x1 = bf16_to_f32(kin[l + 64]);
  double s1 = (double)x0 + (double)x1;
  for (int o = 32; o > 0; o >>= 1) s1 += __shfl_xor(s1, o, 64);
  const double mean = s1 / DSA_IDX_DIM;
  const double d0 = (double)x0 - mean, d1 = (double)x1 - mean;
  double s2 = d0 * d0 + d1 * d1;
  for (int o = 32; o > 0; o >>= 1) s2 += __shfl_xor(s2, o, 64);
  const double inv = 1.0 / sqrt(s2 / DSA_IDX_DIM + (double)ar.ln_eps);
  const float g0 = ar.ln_gamma ? ar.ln_gamma[l] : 1.f, g1 = ar.ln_gamma ? ar.ln_gamma[l + 64] : 1.f;
  const float b0 = ar.ln_beta ? ar.ln_beta[l] : 0.f, b1 = ar.ln_beta ? ar.ln_beta[l + 64] : 0.f;
  sh.kn[l] = fmaf((float)(d0 * inv), g0, b0);
  sh.kn[l + 64] = fmaf((float)(d1 * inv), g1, b1);
}

__device__ __forceinline__ void append_indexer(const AppendArgs& ar, IdxShared& sh, RotTable& rt, int t,
                                               int64_t p) {
  const int tid = threadIdx.x;
  static_assert(DSA_IDX_HEADS * kIdxPieces == kAppendNT, "one 16-byte query piece per thread");
  const int r = tid / kIdxPieces, d0 = 8 * (tid % kIdxPieces);
  const uint4 own = *reinterpret_cast<const uint4*>(ar.idx_q + ((size_t)t * DSA_IDX_HEADS + r) * DSA_IDX_DIM + d0);
  rot_table(rt, p, ar.rot_idx, ar.freq_idx);
  if (tid >> 6 == kLnWave) index_key_norm(ar, sh, t);
  *reinterpret_cast<uint4*>(&sh.xq[r][d0]) = own;
  __syncthreads();
  const int R = ar.rot_idx;
  float x[8], y[8];
  unpack_bf16x8(x, own);
  if (d0 < R) rotate8(y, x, [&](int j) { return bf16_to_f32(sh.xq[r][j]); }, d0, R, rt);
  else
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = x[j];
  *reinterpret_cast<uint2*>(ar.q_idx_out + ((size_t)t * DSA_IDX_HEADS + r) * DSA_IDX_DIM + d0) = pack_e4m3x8(y);
  if (tid < kIdxPieces) {
    const int e0 = 8 * tid;
    const float4 a = *reinterpret_cast<const float4*>(&sh.kn[e0]);
    const float4 b = *reinterpret_cast<const float4*>(&sh.kn[e0 + 4]);
    const float xk[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float yk[8];
    if (e0 < R) rotate8(yk, xk, [&](int j) { return sh.kn[j]; }, e0, R, rt);
    else
#pragma unroll
      for (int j = 0; j < 8; ++j) yk[j] = xk[j];
    *reinterpret_cast<uint2*>(ar.k_idx_cache + (size_t)p * DSA_IDX_DIM + e0) = pack_e4m3x8(yk);
  }
}

__device__ __forceinline__ void append_kv_head(const AppendArgs& ar, MainShared& sh, RotTable& rt, int t,
                                               int64_t p, int g) {
  const int tid = threadIdx.x;
  constexpr int kPieces = (kQPerKv + 1) * kRowPieces;   // 408
  constexpr int kPer = (kPieces + kAppendNT - 1) / kAppendNT;
  uint4 own[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int c = tid + u * kAppendNT;
    if (c < kPieces) {
      const int r = c / kRowPieces, d0 = 8 * (c % kRowPieces);
      const uint16_t* src = r < kQPerKv ? ar.q + ((size_t)t * DSA_Q_HEADS + g * kQPerKv + r) * DSA_QK_DIM
                                        : ar.k + ((size_t)t * DSA_KV_HEADS + g) * DSA_QK_DIM;
      own[u] = *reinterpret_cast<const uint4*>(src + d0);
    }
  }
  if (tid < DSA_V_DIM / 8) {
    const size_t o = 8 * tid;
    *reinterpret_cast<uint4*>(ar.v_cache + ((size_t)p * DSA_KV_HEADS + g) * DSA_V_DIM + o) =
        *reinterpret_cast<const uint4*>(ar.v + ((size_t)t * DSA_KV_HEADS + g) * DSA_V_DIM + o);
  }
  rot_table(rt, p, ar.rot_main, ar.freq_main);
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int c = tid + u * kAppendNT;
    if (c < kPieces) *reinterpret_cast<uint4*>(&sh.xs[c / kRowPieces][8 * (c % kRowPieces)]) = own[u];
  }
  __syncthreads();
  const int R = ar.rot_main;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int c = tid + u * kAppendNT;
    if (c >= kPieces) continue;
    const int r = c / kRowPieces, d0 = 8 * (c % kRowPieces);
    uint4 o = own[u];                                   // unrotated dims pass through bit-exact
    if (d0 < R) {
      float x[8], y[8];
      unpack_bf16x8(x, own[u]);
      if ((R & 15) == 0) {
        // R / 2 is a multiple of 8: the piece is rotated whole and its 8
        // partners are the staged piece R / 2 away
        float xp[8];
        const int pd = d0 < (R >> 1) ? d0 + (R >> 1) : d0 - (R >> 1);
        unpack_bf16x8(xp, *reinterpret_cast<const uint4*>(&sh.xs[r][pd]));
        rot8<true>(y, x, xp, d0, R, rt);
      } else {
        rotate8(y, x, [&](int j) { return bf16_to_f32(sh.xs[r][j]); }, d0, R, rt);
      }
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = f32x2_to_bf16x2_rne(y[2 * j], y[2 * j + 1]);
      o = make_uint4(w[0], w[1], w[2], w[3]);
    }
    uint16_t* dst = r < kQPerKv ? ar.q_out + ((size_t)t * DSA_Q_HEADS + g * kQPerKv + r) * DSA_QK_DIM
                                : ar.k_cache + ((size_t)p * DSA_KV_HEADS + g) * DSA_QK_DIM;
    *reinterpret_cast<uint4*>(dst + d0) = o;
  }
}

__global__ __launch_bounds__(kAppendNT) void cache_append_kernel(AppendArgs ar) {
  __shared__ __attribute__((aligned(16))) AppendShared sh;
  __shared__ __attribute__((aligned(16))) RotTable rt;
  const int t = blockIdx.x, part = blockIdx.y;
  const int64_t p = ar.Lk - ar.T + t;
  if (part == 0)
    append_indexer(ar, sh.ix, rt, t, p);
  else
    append_kv_head(ar, sh.mn, rt, t, p, part - 1);
}

}  // namespace

hipError_t launch_cache_append(const uint16_t* idx_q, const uint16_t* idx_k, const float* ln_gamma,
                               const float* ln_beta, float ln_eps, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, int64_t Lk, int T, int rot_idx, int rot_main, double base,
                               uint8_t* q_idx_out, uint8_t* k_idx_cache, uint16_t* q_out, uint16_t* k_cache,
                               uint16_t* v_cache, hipStream_t st) {
  // the table threads (one per rotated dim) fit in the workgroup
  if (rot_idx > DSA_IDX_DIM || rot_main > DSA_QK_DIM || rot_idx < 2 || rot_main < 2 || (rot_idx | rot_main) & 1)
    return hipErrorInvalidValue;
  AppendArgs ar{idx_q, idx_k, ln_gamma, ln_beta, ln_eps, q, k, v, Lk, T, rot_idx, rot_main, {}, {},
                q_idx_out, k_idx_cache, q_out, k_cache, v_cache};
  const double lb = std::log2(base);
  for (int i = 0; i < rot_idx / 2; ++i) ar.freq_idx[i] = std::exp2(-2.0 * i / rot_idx * lb);
  for (int i = 0; i < rot_main / 2; ++i) ar.freq_main[i] = std::exp2(-2.0 * i / rot_main * lb);
  hipLaunchKernelGGL(cache_append_kernel, dim3(T, 1 + DSA_KV_HEADS), dim3(kAppendNT), 0, st, ar);
  return hipGetLastError();
}

}  // namespace dsa
