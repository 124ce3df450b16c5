// append.hip -- the step before the index sweep for T new tokens: LayerNorm,
// partial RoPE and fp8 rounding of the lightning indexer's key and queries,
// partial RoPE of the attention queries and keys, and the cache appends
// ("Naive-N0.5-Flash: no full-attention layers, and a runtime built by AI",
// section "Inside a DSA layer" and Figure 1, panel B; RoPE on a third of each
// head with base 10,000,000 on the sparse layers, same section).
//
// Grid (T, 5): workgroup y = 0 handles the indexer (key and 16 query heads),
// y = 1 + g the attention's KV head g (its 16 query heads, key and value).
// The rotation angles a_i = p * base^(-2i/R) are formed and reduced in float64
// once per workgroup (an absolute position near 2^20 times a float32
// frequency would lose most of the angle's fraction), then applied in float32.
#include "dsa_common.hpp"
#include "kernels.hpp"

namespace dsa {

namespace {

constexpr int kAppendNT = 256;
constexpr int kMaxRotHalf = 96;                    // R / 2 <= 96 (R <= 192)

// fp32 -> fp8 e4m3 code, round to nearest even, saturating at +-448: from the
// format (bias 7, 3 fraction bits, exponent field 0 subnormal in steps of 2^-9)
__device__ __forceinline__ uint8_t f32_to_e4m3_rne(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.f);
  if (a < 0.015625f) return (uint8_t)(sign | (uint32_t)rintf(a * 512.f));   // 8 is the smallest normal
  uint32_t b = __float_as_uint(a);
  b += 0x7FFFFu + ((b >> 20) & 1u);                 // keep 3 fraction bits, ties to even
  const uint32_t e = (b >> 23) - 120u;              // 127 - 7
  return (uint8_t)(sign | (e << 3) | ((b >> 20) & 7u));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

struct RotTable {
  float c[kMaxRotHalf], s[kMaxRotHalf];
};

// cos / sin of p * base^(-2i/R) for i < R/2, formed in float64
__device__ __forceinline__ void rot_table(RotTable& rt, int64_t p, int R, double base) {
  for (int i = threadIdx.x; i < R / 2; i += kAppendNT) {
    const double a = (double)p * pow(base, -2.0 * i / R);
    double sn, cs;
    sincos(a, &sn, &cs);
    rt.c[i] = (float)cs;
    rt.s[i] = (float)sn;
  }
}

// rotated value of dim d of a head whose element j is x(j)
template <class X>
__device__ __forceinline__ float rope_at(const X& x, int d, int R, const RotTable& rt) {
  const int h = R / 2;
  if (d >= R) return x(d);
  if (d < h) return x(d) * rt.c[d] - x(d + h) * rt.s[d];
  return x(d) * rt.c[d - h] + x(d - h) * rt.s[d - h];
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
  double base;
  uint8_t* q_idx_out;
  uint8_t* k_idx_cache;
  uint16_t* q_out;
  uint16_t* k_cache;
  uint16_t* v_cache;
};

__global__ __launch_bounds__(kAppendNT) void cache_append_kernel(AppendArgs ar) {
  __shared__ RotTable rt;
  __shared__ float kn[DSA_IDX_DIM];                // normalised index key
  __shared__ double red[2][kAppendNT / 64];
  const int t = blockIdx.x, part = blockIdx.y, tid = threadIdx.x;
  const int64_t p = ar.Lk - ar.T + t;

  if (part == 0) {
    // ---- the indexer: key (LayerNorm, RoPE, fp8, append) and 16 query heads
    rot_table(rt, p, ar.rot_idx, ar.base);
    const uint16_t* kin = ar.idx_k + (size_t)t * DSA_IDX_DIM;
    const float xv = tid < DSA_IDX_DIM ? bf16_to_f32(kin[tid]) : 0.f;
    // mean and variance in float64 (two passes over 128 values)
    double s1 = xv;
    for (int o = 32; o > 0; o >>= 1) s1 += __shfl_xor(s1, o, 64);
    if ((tid & 63) == 0) red[0][tid >> 6] = s1;
    __syncthreads();
    const double mean = (red[0][0] + red[0][1]) / DSA_IDX_DIM;
    const double dx = tid < DSA_IDX_DIM ? (double)xv - mean : 0.0;
    double s2 = dx * dx;
    for (int o = 32; o > 0; o >>= 1) s2 += __shfl_xor(s2, o, 64);
    if ((tid & 63) == 0) red[1][tid >> 6] = s2;
    __syncthreads();
    const double var = (red[1][0] + red[1][1]) / DSA_IDX_DIM;
    const double inv = 1.0 / sqrt(var + (double)ar.ln_eps);
    if (tid < DSA_IDX_DIM) {
      const float g = ar.ln_gamma ? ar.ln_gamma[tid] : 1.f;
      const float b = ar.ln_beta ? ar.ln_beta[tid] : 0.f;
      kn[tid] = (float)(dx * inv) * g + b;
    }
    __syncthreads();
    if (tid < DSA_IDX_DIM) {
      const float y = rope_at([&](int j) { return kn[j]; }, tid, ar.rot_idx, rt);
      ar.k_idx_cache[(size_t)p * DSA_IDX_DIM + tid] = f32_to_e4m3_rne(y);
    }
    for (int e = tid; e < DSA_IDX_HEADS * DSA_IDX_DIM; e += kAppendNT) {
      const int hd = e / DSA_IDX_DIM, d = e % DSA_IDX_DIM;
      const uint16_t* xin = ar.idx_q + ((size_t)t * DSA_IDX_HEADS + hd) * DSA_IDX_DIM;
      const float y = rope_at([&](int j) { return bf16_to_f32(xin[j]); }, d, ar.rot_idx, rt);
      ar.q_idx_out[((size_t)t * DSA_IDX_HEADS + hd) * DSA_IDX_DIM + d] = f32_to_e4m3_rne(y);
    }
    return;
  }

  // ---- attention KV head g: its 16 query heads, key and value
  const int g = part - 1;
  constexpr int GH = DSA_Q_HEADS / DSA_KV_HEADS;
  rot_table(rt, p, ar.rot_main, ar.base);
  __syncthreads();
  for (int e = tid; e < GH * DSA_QK_DIM; e += kAppendNT) {
    const int hd = g * GH + e / DSA_QK_DIM, d = e % DSA_QK_DIM;
    const uint16_t* xin = ar.q + ((size_t)t * DSA_Q_HEADS + hd) * DSA_QK_DIM;
    const float y = rope_at([&](int j) { return bf16_to_f32(xin[j]); }, d, ar.rot_main, rt);
    ar.q_out[((size_t)t * DSA_Q_HEADS + hd) * DSA_QK_DIM + d] = f32_to_bf16_rne(y);
  }
  if (tid < DSA_QK_DIM) {
    const uint16_t* xin = ar.k + ((size_t)t * DSA_KV_HEADS + g) * DSA_QK_DIM;
    const float y = rope_at([&](int j) { return bf16_to_f32(xin[j]); }, tid, ar.rot_main, rt);
    ar.k_cache[((size_t)p * DSA_KV_HEADS + g) * DSA_QK_DIM + tid] = f32_to_bf16_rne(y);
  }
  if (tid < DSA_V_DIM)
    ar.v_cache[((size_t)p * DSA_KV_HEADS + g) * DSA_V_DIM + tid] =
        ar.v[((size_t)t * DSA_KV_HEADS + g) * DSA_V_DIM + tid];
}

}  // namespace

hipError_t launch_cache_append(const uint16_t* idx_q, const uint16_t* idx_k, const float* ln_gamma,
                               const float* ln_beta, float ln_eps, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, int64_t Lk, int T, int rot_idx, int rot_main, double base,
                               uint8_t* q_idx_out, uint8_t* k_idx_cache, uint16_t* q_out, uint16_t* k_cache,
                               uint16_t* v_cache, hipStream_t st) {
  if (rot_idx > DSA_IDX_DIM || rot_main > DSA_QK_DIM || rot_main / 2 > kMaxRotHalf) return hipErrorInvalidValue;
  AppendArgs ar{idx_q, idx_k, ln_gamma, ln_beta, ln_eps, q, k, v, Lk, T, rot_idx, rot_main, base,
                q_idx_out, k_idx_cache, q_out, k_cache, v_cache};
  hipLaunchKernelGGL(cache_append_kernel, dim3(T, 1 + DSA_KV_HEADS), dim3(kAppendNT), 0, st, ar);
  return hipGetLastError();
}

}  // namespace dsa
