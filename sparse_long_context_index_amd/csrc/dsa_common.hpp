// dsa_common.hpp -- internal helpers shared by the HIP kernels of libdsa.so.
//
// gfx950 (CDNA4) only: wave64, MFMA matrix cores, 160 KiB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dsa.h"

namespace dsa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kHistBits1 = 12;            // level-1 radix digit: key bits [31:20]
constexpr int kHistBins = 1 << kHistBits1;
constexpr int kHist3Bins = 256;           // level-3 digit: key bits [7:0]

// Workspace layout: a fixed counter region at the front (zero between calls),
// then per-op scratch that every call overwrites before reading.
constexpr int kMaxCounterRows = 8;        // rows served by the multi-block top-k
constexpr int kHistReplicas = 16;         // level-1 histogram copies (spreads atomics)
constexpr size_t kCounterRegionBytes = size_t(4) << 20;

struct TopkCounters {
  uint32_t* h1;        // [kHistReplicas][rows][4096] level-1 histograms
  uint32_t* maxbin;    // [kHistReplicas][rows] highest level-1 bin seen, plus one
  uint32_t* h2;        // [rows][4096] level-2 histogram of the boundary bin
  uint32_t* overflow;  // [rows] a candidate slot overflowed
};

__host__ __device__ inline TopkCounters counters_at(void* ws) {
  uint32_t* b = reinterpret_cast<uint32_t*>(ws);
  TopkCounters c;
  c.h1 = b;
  c.maxbin = c.h1 + kHistReplicas * kMaxCounterRows * kHistBins;
  c.h2 = c.maxbin + kHistReplicas * kMaxCounterRows;
  c.overflow = c.h2 + kMaxCounterRows * kHistBins;
  return c;
}
static_assert((kHistReplicas + 1) * kMaxCounterRows * kHistBins * 4 + (kHistReplicas + 1) * kMaxCounterRows * 4 <=
                  (int)kCounterRegionBytes, "counter region");

// ---------------------------------------------------------------- MFMA
// 16x16x128 fp8(e4m3) x fp8(e4m3) -> f32, unit block scales (E8M0 127 = 2^0).
// Operand layout (A: 16 rows x 128 k, B: 128 k x 16 cols): lane l supplies
// row/col (l % 16) and 32 k-values of k-group (l / 16).  A and B use the same
// k-placement, so any consistent split of k over (lane group, byte) gives the
// plain dot product.  Result: lane l holds column (l % 16), rows
// 4*(l/16) + {0,1,2,3}.
__device__ __forceinline__ f32x4 mfma_f8_16x16x128(const i32x8& a, const i32x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// 16x16x32 bf16 -> f32: lane l supplies row/col (l % 16) and 8 k-values of
// k-group (l / 16).  Same output layout as above.
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- keys
// Order-preserving map float -> uint32 (larger float -> larger key).  -0.0 is
// folded onto +0.0 first so the two compare equal.
__device__ __forceinline__ uint32_t order_key(float f) {
  f = f + 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- misc
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }

// float -> bf16, round to nearest even, by the hardware conversion
// (v_cvt_pk_bf16_f32); an exhaustive comparison over every finite float with
// the rounding written out (add 0x7FFF plus the kept lsb, drop 16 bits) found
// no difference.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// two floats to bf16 (same rounding), a in the low half: one packed conversion
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

__device__ __forceinline__ uint32_t* h1_row(const TopkCounters& c, int rep, int t) {
  return c.h1 + ((size_t)rep * kMaxCounterRows + t) * kHistBins;
}

// Adds this block's level-1 histogram (in LDS) to replica `rep` of row t and
// raises the replica's max-bin mark.  All threads call it.
// Same, for a histogram kept as two 16-bit counters per word (bin b in word
// b/2, half b&1).
template <int NT>
__device__ void flush_level1_packed(const TopkCounters& ctr, int rep, int t, const uint32_t* lh,
                                    uint32_t* red_sm) {
  uint32_t* g = h1_row(ctr, rep, t);
  uint32_t top = 0;
  for (int i = threadIdx.x; i < kHistBins / 2; i += NT) {
    const uint32_t c = lh[i];
    const uint32_t c0 = c & 0xFFFFu, c1 = c >> 16;
    if (c0) {
      atomicAdd(&g[2 * i], c0);
      top = (uint32_t)(2 * i) + 1;
    }
    if (c1) {
      atomicAdd(&g[2 * i + 1], c1);
      top = (uint32_t)(2 * i) + 2;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t y = __shfl_xor(top, o, 64);
    top = y > top ? y : top;
  }
  if ((threadIdx.x & 63) == 0) red_sm[threadIdx.x >> 6] = top;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = 0;
    for (int i = 0; i < NT / 64; ++i) m = red_sm[i] > m ? red_sm[i] : m;
    if (m) atomicMax(&ctr.maxbin[rep * kMaxCounterRows + t], m);
  }
}

template <int NT>
__device__ void flush_level1(const TopkCounters& ctr, int rep, int t, const uint32_t* lh, uint32_t* red_sm) {
  uint32_t* g = h1_row(ctr, rep, t);
  uint32_t top = 0;                                      // highest non-empty bin + 1
  for (int i = threadIdx.x; i < kHistBins; i += NT) {
    const uint32_t c = lh[i];
    if (c) {
      atomicAdd(&g[i], c);
      top = (uint32_t)i + 1;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t y = __shfl_xor(top, o, 64);
    top = y > top ? y : top;
  }
  if ((threadIdx.x & 63) == 0) red_sm[threadIdx.x >> 6] = top;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = 0;
    for (int i = 0; i < NT / 64; ++i) m = red_sm[i] > m ? red_sm[i] : m;
    if (m) atomicMax(&ctr.maxbin[rep * kMaxCounterRows + t], m);
  }
}



}  // namespace dsa
