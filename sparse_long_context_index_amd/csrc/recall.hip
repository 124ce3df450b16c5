// recall.hip -- index-selection recall: the share of each head's dense
// softmax mass, over every visible key and without the sink, that the
// selected keys carry ("Naive-N0.5-Flash: no full-attention layers, and a
// runtime built by AI", section "How much of this did AI actually build?":
// the indexer's top-k was checked against a full-attention reference).
//
// recall[t,h] = exp(lse_sel[t,h] - lse_dense[t,h]): lse_sel comes from the
// gathered attention over the selected keys (no sink); lse_dense from
// dense_lse_kernel, a QK-only pass over every visible key:
//   grid (KV head g, key chunks of 2,048, token t), 4 waves x 512 keys --
//   the four heads of a chunk are neighbours in the dispatch order, so the
//   four slices of a key's K row (1,536 contiguous bytes) are read at about
//   the same time;
//   16x16x32 bf16 MFMA with the group's 16 query heads on M and 16 keys on N;
//   each lane reads 96 contiguous bytes of its key's row (the k-placement of
//   Q and K agree: lane group q takes dims 48q .. 48q+47), the next block's
//   loads in flight; per lane an online (max, sum) in base 2 for its 4
//   heads, reduced over the row's lanes, the waves, then the chunks.
#include "attn_core.hpp"
#include "dsa_common.hpp"
#include "kernels.hpp"

namespace dsa {

namespace {

constexpr int kLseChunk = 2048;
constexpr int kLseWaveKeys = kLseChunk / 4;

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  bf16x8 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

__global__ __launch_bounds__(256) void dense_lse_kernel(const uint16_t* __restrict__ q,
                                                        const uint16_t* __restrict__ k, int64_t Lk, int T,
                                                        float sm_scale, int n_chunks, float* __restrict__ part) {
  __shared__ float red[4][16][2];
  const int g = blockIdx.x, c = blockIdx.y, t = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int64_t p = Lk - T + t;                               // last visible key
  const float qs = sm_scale * kLog2e;
  // Q of head g*16 + col, dims 48*grp + 8s .. +7 (A operand, row = head)
  bf16x8 a[6];
  const uint16_t* qp = q + ((size_t)t * DSA_Q_HEADS + g * 16 + col) * DSA_QK_DIM + 48 * grp;
#pragma unroll
  for (int s = 0; s < 6; ++s) a[s] = ld8(qp + 8 * s);
  float m[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
  }
  const int64_t k0 = (int64_t)c * kLseChunk + (int64_t)wave * kLseWaveKeys;
  int64_t k1 = k0 + kLseWaveKeys;
  k1 = k1 < p + 1 ? k1 : p + 1;
  const int nb = k0 < k1 ? (int)((k1 - k0 + 15) / 16) : 0;     // wave-uniform
  auto load = [&](int b, bf16x8 (&r)[6]) {
    int64_t key = k0 + 16 * b + col;
    key = key < p ? key : p;                                  // stay on visible rows
    const uint16_t* kp = k + ((size_t)key * DSA_KV_HEADS + g) * DSA_QK_DIM + 48 * grp;
#pragma unroll
    for (int s = 0; s < 6; ++s) r[s] = ld8(kp + 8 * s);
  };
  bf16x8 cur[6], nxt[6];
  if (nb > 0) load(0, cur);
  for (int b = 0; b < nb; ++b) {
    if (b + 1 < nb) load(b + 1, nxt);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 6; ++s) acc = mfma_bf16_16x16x32(a[s], cur[s], acc);
    const int64_t key = k0 + 16 * b + col;
    const bool vis = key <= p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float z = vis ? acc[i] * qs : -INFINITY;
      const float mn = fmaxf(m[i], z);
      if (mn != -INFINITY) {
        l[i] = l[i] * exp2f(m[i] - mn) + exp2f(z - mn);
        m[i] = mn;
      }
    }
#pragma unroll
    for (int s = 0; s < 6; ++s) cur[s] = nxt[s];
  }
  // combine the 16 key columns of each head, then the waves
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const float mo = __shfl_xor(m[i], o, 64), lo = __shfl_xor(l[i], o, 64);
      const float mn = fmaxf(m[i], mo);
      if (mn != -INFINITY) {
        l[i] = l[i] * exp2f(m[i] - mn) + lo * exp2f(mo - mn);
        m[i] = mn;
      }
    }
  }
  if (col == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      red[wave][4 * grp + i][0] = m[i];
      red[wave][4 * grp + i][1] = l[i];
    }
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    const int h = threadIdx.x;
    float M = -INFINITY, L = 0.f;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red[w][h][0]);
    if (M != -INFINITY)
      for (int w = 0; w < 4; ++w)
        if (red[w][h][0] != -INFINITY) L += red[w][h][1] * exp2f(red[w][h][0] - M);
    float* o = part + (((size_t)t * DSA_KV_HEADS + g) * n_chunks + c) * 32;
    o[2 * h] = M;
    o[2 * h + 1] = L;
  }
}

// per (t, h), one wave: the lanes merge strided chunks, then the wave
// combines its lanes; lse_dense, then recall = exp(lse_sel - lse_dense)
__global__ __launch_bounds__(64) void recall_merge_kernel(const float* __restrict__ part, int n_chunks,
                                                          const float* __restrict__ lse_sel, float* __restrict__ recall,
                                                          float* __restrict__ lse_dense) {
  const int t = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int g = h / 16, hh = h % 16;
  const float* pp = part + ((size_t)t * DSA_KV_HEADS + g) * n_chunks * 32 + 2 * hh;
  float M = -INFINITY, L = 0.f;
  for (int c = lane; c < n_chunks; c += 64) {
    const float mc = pp[(size_t)c * 32], lc = pp[(size_t)c * 32 + 1];
    const float mn = fmaxf(M, mc);
    if (mn != -INFINITY) {
      L = L * exp2f(M - mn) + lc * exp2f(mc - mn);
      M = mn;
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float mo = __shfl_xor(M, o, 64), lo = __shfl_xor(L, o, 64);
    const float mn = fmaxf(M, mo);
    if (mn != -INFINITY) {
      L = L * exp2f(M - mn) + lo * exp2f(mo - mn);
      M = mn;
    }
  }
  if (lane != 0) return;
  const float ld = M == -INFINITY ? -INFINITY : (M + log2f(L)) * kLn2;
  const float ls = lse_sel[(size_t)t * DSA_Q_HEADS + h];
  recall[(size_t)t * DSA_Q_HEADS + h] = (ls == -INFINITY || ld == -INFINITY) ? 0.f : expf(ls - ld);
  if (lse_dense) lse_dense[(size_t)t * DSA_Q_HEADS + h] = ld;
}

}  // namespace

int recall_chunks(int64_t Lk) { return (int)cdiv(Lk, kLseChunk); }

hipError_t launch_index_recall(const uint16_t* q, const uint16_t* k, int64_t Lk, int T, float sm_scale,
                               const float* lse_sel, float* part, float* recall, float* lse_dense, hipStream_t st) {
  const int nc = recall_chunks(Lk);
  hipLaunchKernelGGL(dense_lse_kernel, dim3(DSA_KV_HEADS, nc, T), dim3(256), 0, st, q, k, Lk, T, sm_scale, nc, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(recall_merge_kernel, dim3(T, DSA_Q_HEADS), dim3(64), 0, st, (const float*)part, nc, lse_sel,
                     recall, lse_dense);
  return hipGetLastError();
}

}  // namespace dsa
