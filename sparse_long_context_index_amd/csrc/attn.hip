// attn.hip -- gathered GQA attention with a sink logit on gfx950.
//
// "Naive-N0.5-Flash: no full-attention layers, and a runtime built by AI",
// section "Inside a DSA layer: the lightning indexer": the main heads attend
// only to the selected keys (the rest are masked before the softmax), GQA
// with 4 KV heads on DSA layers and 8 on SWA layers, and a sink column; the
// section "What 'no full-attention layers' means" gives the SWA mask (offset
// from the query below the window).  Both are one kernel here: a DSA unit
// reads its key list from idx, an SWA unit uses the window of its sequence.
//
// Work unit: one query token (or sequence) t and one KV head g, i.e. the 16
// (DSA) or 8 (SWA) query heads sharing K/V rows.  A unit's key list may be
// split into chunks over several workgroups (decode); each chunk yields a
// partial (max, sum, unnormalised output) that a merge kernel combines with
// the sink.  Inside a workgroup each wave takes 32-key tiles:
//   QK : K rows are gathered straight into the A operand of two 16x16x32 bf16
//        MFMA chains (keys x head-columns), 6 k-steps over qk dim 192;
//   softmax: online, base-2, per head column, fp32;
//   PV : P (heads x 32 keys) is already in A-operand order; V rows are staged
//        through LDS and read as the B operand, 8 MFMAs over v dim 128.
// Empty slots (idx < 0, idx >= Lk, positions past the window) load no value
// row: their V lanes are written as zeros and their logits as -inf, so
// poisoned cache rows outside the set can never reach the output.
#include "dsa_common.hpp"
#include "kernels.hpp"

namespace dsa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kTileKeys = 32;
constexpr int kVStride = 136;               // bf16 per staged V row (272 B, 16-B aligned)
constexpr int kPartFloats = 16 + 16 + 16 * 128;

template <int NW>
struct AttnSmem {
  static constexpr int stage = NW * kTileKeys * kVStride * 2;       // V tiles
  static constexpr int merge = NW * 16 * 128 * 4 + NW * 32 * 4;     // wave partials
  static constexpr int bytes = stage > merge ? stage : merge;
};

// list position -> cache row, or -1 for an empty slot
struct IdxList {
  const int32_t* row_idx;   // idx[t] row
  int len;
  int64_t n_rows;
  __device__ int64_t row(int p) const {
    if (p >= len) return -1;
    const int32_t j = row_idx[p];
    return (j >= 0 && (int64_t)j < n_rows) ? (int64_t)j : -1;
  }
};

struct Window {
  int64_t first;            // cache row of list position 0
  int len;
  int64_t n_rows;
  __device__ int64_t row(int p) const {
    if (p >= len) return -1;
    const int64_t r = first + p;
    return (r >= 0 && r < n_rows) ? r : -1;
  }
};

template <int HKV, int NW, class Src>
__device__ void attend_chunk(const AttnArgs& a, const Src& src, int t, int g, int c, int n_chunks,
                             int p0, int p1, float* part, char* smem) {
  constexpr int GH = 64 / HKV;              // query heads per KV head
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int kg = lane >> 4;
  const float qscale = a.sm_scale * kLog2e;

  // Q as the B operand: column = head, k-group kg covers dims 48*kg .. 48*kg+47
  bf16x8 qf[6];
  {
    const bool hv = col < GH;
    const int h = g * GH + (hv ? col : 0);
    const uint16_t* qp = a.q + ((size_t)t * 64 + h) * 192 + 48 * kg;
#pragma unroll
    for (int s = 0; s < 6; ++s) {
      u16x8 raw = *reinterpret_cast<const u16x8*>(qp + 8 * s);
      if (!hv) raw = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      qf[s] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  f32x4 o[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) o[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;       // running max of this lane's head column (base 2)
  float lsum = 0.f;          // this lane's share of the running denominator

  uint16_t* vs = reinterpret_cast<uint16_t*>(smem) + wave * kTileKeys * kVStride;
  const int ntiles = (p1 - p0 + kTileKeys - 1) / kTileKeys;
  const int rounds = (ntiles + NW - 1) / NW;

  for (int rd = 0; rd < rounds; ++rd) {
    const int tile = rd * NW + wave;
    const bool active = tile < ntiles;       // wave-uniform
    const int tb = p0 + tile * kTileKeys;
    bf16x8 pf;
    if (active) {
      // ---- all index and row loads first: one dependent round trip per tile
      const int kv = lane >> 1;                          // V staging: key lane/2, half lane&1
      const int64_t rv = tb + kv < p1 ? src.row(tb + kv) : -1;
      int64_t rk[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int p = tb + b * 16 + col;
        rk[b] = p < p1 ? src.row(p) : -1;
      }
      u16x8 kraw[2][6];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const uint16_t* kp = a.k + ((size_t)(rk[b] >= 0 ? rk[b] : 0) * HKV + g) * 192 + 48 * kg;
#pragma unroll
        for (int s = 0; s < 6; ++s) kraw[b][s] = *reinterpret_cast<const u16x8*>(kp + 8 * s);
      }
      u16x8 vraw[8];
      {
        const u16x8* sp = reinterpret_cast<const u16x8*>(a.v + ((size_t)(rv >= 0 ? rv : 0) * HKV + g) * 128 +
                                                         (lane & 1) * 64);
#pragma unroll
        for (int i = 0; i < 8; ++i) vraw[i] = sp[i];
      }
      // ---- stage V rows (an empty slot stages zeros, never the row it loaded)
      {
        u16x8* dst = reinterpret_cast<u16x8*>(vs + kv * kVStride + (lane & 1) * 64);
        const u16x8 zero = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 8; ++i) dst[i] = rv >= 0 ? vraw[i] : zero;
      }
      // ---- QK for the two 16-key blocks
      f32x4 acc[2];
      uint64_t valid[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        valid[b] = __ballot(rk[b] >= 0);
        acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 6; ++s)
          acc[b] = mfma_bf16_16x16x32(__builtin_bit_cast(bf16x8, kraw[b][s]), qf[s], acc[b]);
      }
      // ---- online softmax, lane holds head `col`, keys 16*b + 4*kg + i
      float z[2][4];
      float mx = -INFINITY;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = (valid[b] >> (4 * kg + i)) & 1ull;
          z[b][i] = ok ? acc[b][i] * qscale : -INFINITY;
          mx = fmaxf(mx, z[b][i]);
        }
      mx = fmaxf(mx, shfl_xor_f(mx, 16));
      mx = fmaxf(mx, shfl_xor_f(mx, 32));
      const float mn = fmaxf(m, mx);
      const bool dead = mn == -INFINITY;
      const float alpha = dead ? 1.0f : exp2f(m - mn);
      float ps = 0.f;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = dead ? 0.0f : exp2f(z[b][i] - mn);
          ps += pv;
          pf[b * 4 + i] = (__bf16)pv;
        }
      lsum = lsum * alpha + ps;
      m = mn;
      // rescale O rows (heads 4*kg + i) by their column's alpha
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float al = __shfl(alpha, 4 * kg + i, 64);
#pragma unroll
        for (int b = 0; b < 8; ++b) o[b][i] *= al;
      }
    }
    __syncthreads();
    if (active) {
      // ---- PV: B operand = V[key(kg,e)][16*blk + col], key(kg,e) = e<4 ? 4kg+e : 12+4kg+e
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) {
        u16x8 vb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int kk = e < 4 ? 4 * kg + e : 12 + 4 * kg + e;
          vb[e] = vs[kk * kVStride + blk * 16 + col];
        }
        o[blk] = mfma_bf16_16x16x32(pf, __builtin_bit_cast(bf16x8, vb), o[blk]);
      }
    }
    __syncthreads();
  }

  // ---- combine the waves of this workgroup
  lsum += shfl_xor_f(lsum, 16);
  lsum += shfl_xor_f(lsum, 32);
  float* mw = reinterpret_cast<float*>(smem);              // [NW][16]
  float* lw = mw + NW * 16;                                 // [NW][16]
  float* ow = lw + NW * 16;                                 // [NW][16][128]
  __syncthreads();                                          // V staging is dead
  if (lane < 16) {
    mw[wave * 16 + lane] = m;
    lw[wave * 16 + lane] = lsum;
  }
#pragma unroll
  for (int blk = 0; blk < 8; ++blk)
#pragma unroll
    for (int i = 0; i < 4; ++i) ow[(wave * 16 + 4 * kg + i) * 128 + blk * 16 + col] = o[blk][i];
  __syncthreads();

  const int unit = t * HKV + g;
  for (int e = threadIdx.x; e < GH * 128; e += NW * 64) {
    const int hc = e >> 7;          // head column
    const int dv = e & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, mw[w * 16 + hc]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = exp2f(mw[w * 16 + hc] - M);
        L += f * lw[w * 16 + hc];
        O += f * ow[(w * 16 + hc) * 128 + dv];
      }
    }
    const int h = g * GH + hc;
    if (n_chunks == 1) {
      float Mf = M;
      float sl = 0.f;
      if (a.sink) {
        const float s2 = a.sink[h] * kLog2e;
        Mf = fmaxf(M, s2);
        sl = exp2f(s2 - Mf);
      }
      float outv = 0.f, lse = -INFINITY;
      if (Mf != -INFINITY) {
        const float sc = M == -INFINITY ? 0.f : exp2f(M - Mf);
        const float Lf = L * sc + sl;
        outv = Lf > 0.f ? (O * sc) / Lf : 0.f;
        lse = (Mf + log2f(Lf)) * kLn2;
      }
      a.out[((size_t)t * 64 + h) * 128 + dv] = f32_to_bf16_rne(outv);
      if (a.lse && dv == 0) a.lse[(size_t)t * 64 + h] = lse;
    } else {
      float* pp = part + ((size_t)unit * n_chunks + c) * kPartFloats;
      if (dv == 0) {
        pp[hc] = M;
        pp[16 + hc] = L;
      }
      pp[32 + hc * 128 + dv] = O;
    }
  }
}

template <int HKV, int NW>
__global__ __launch_bounds__(NW * 64) void sparse_attn_kernel(AttnArgs a, int n_chunks, int chunk_keys,
                                                             float* part) {
  __shared__ __attribute__((aligned(16))) char smem[AttnSmem<NW>::bytes];
  const int c = blockIdx.x, g = blockIdx.y, t = blockIdx.z;
  const int p0 = c * chunk_keys;
  const int p1 = p0 + chunk_keys < a.k_len ? p0 + chunk_keys : a.k_len;
  IdxList src{a.idx + (size_t)t * a.k_len, a.k_len, a.n_rows};
  attend_chunk<HKV, NW>(a, src, t, g, c, n_chunks, p0, p1, part, smem);
}

template <int HKV, int NW>
__global__ __launch_bounds__(NW * 64) void swa_attn_kernel(AttnArgs a, int n_chunks, int chunk_keys,
                                                          float* part) {
  __shared__ __attribute__((aligned(16))) char smem[AttnSmem<NW>::bytes];
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int64_t n = a.seq_len[b];
  const int len = n <= 0 ? 0 : (int)(n < a.window ? n : a.window);
  Window src{a.seq_start[b] + n - len, len, a.n_rows};
  const int p0 = c * chunk_keys;
  const int p1 = p0 + chunk_keys < len ? p0 + chunk_keys : len;
  attend_chunk<HKV, NW>(a, src, b, g, c, n_chunks, p0 < p1 ? p0 : p1, p1, part, smem);
}

// merge the chunk partials of every (t, head) and add the sink; every load is
// issued before any is used
constexpr int kMaxChunks = 32;

template <int HKV>
__global__ __launch_bounds__(128) void attn_merge_kernel(AttnArgs a, int n_chunks, const float* part) {
  constexpr int GH = 64 / HKV;
  const int h = blockIdx.x, t = blockIdx.y;
  const int g = h / GH, hc = h % GH;
  const int dv = threadIdx.x;
  const float* pp = part + ((size_t)(t * HKV + g) * n_chunks) * kPartFloats;
  float mc[kMaxChunks], lc[kMaxChunks], oc[kMaxChunks];
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const bool ok = c < n_chunks;
    const float* q = pp + (size_t)(ok ? c : 0) * kPartFloats;
    mc[c] = ok ? q[hc] : -INFINITY;
    lc[c] = ok ? q[16 + hc] : 0.f;
    oc[c] = ok ? q[32 + hc * 128 + dv] : 0.f;
  }
  const float s2 = a.sink ? a.sink[h] * kLog2e : -INFINITY;
  float M = s2;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) M = fmaxf(M, mc[c]);
  float L = 0.f, O = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      const float f = mc[c] == -INFINITY ? 0.f : exp2f(mc[c] - M);
      L += f * lc[c];
      O += f * oc[c];
    }
    if (a.sink) L += exp2f(s2 - M);
  }
  const float outv = (M != -INFINITY && L > 0.f) ? O / L : 0.f;
  a.out[((size_t)t * 64 + h) * 128 + dv] = f32_to_bf16_rne(outv);
  if (a.lse && dv == 0) a.lse[(size_t)t * 64 + h] = M == -INFINITY ? -INFINITY : (M + log2f(L)) * kLn2;
}

constexpr int kNW = 4;                          // waves per workgroup, unsplit units
constexpr int kSplitNW = 2;                     // waves per workgroup when a unit is split
constexpr int kSplitChunk = kSplitNW * kTileKeys;

int sparse_chunks(int T, int k_len) {
  // split a unit's key list over several workgroups only when the grid is small
  if (T * DSA_KV_HEADS >= 256) return 1;
  const int c = (k_len + kSplitChunk - 1) / kSplitChunk;
  return c < kMaxChunks ? c : kMaxChunks;
}

}  // namespace

size_t attn_scratch_bytes(int T, int k_len, int hkv) {
  const int c = hkv == DSA_KV_HEADS ? sparse_chunks(T, k_len) : 1;
  if (c <= 1) return 256;
  return (size_t)T * hkv * c * kPartFloats * sizeof(float) + 256;
}

hipError_t launch_sparse_attn(const AttnArgs& a, void* scratch, hipStream_t st) {
  const int n_chunks = sparse_chunks(a.T, a.k_len);
  float* part = reinterpret_cast<float*>(scratch);
  if (n_chunks == 1) {
    hipLaunchKernelGGL((sparse_attn_kernel<DSA_KV_HEADS, kNW>), dim3(1, DSA_KV_HEADS, a.T), dim3(kNW * 64), 0,
                       st, a, 1, a.k_len, part);
    return hipGetLastError();
  }
  const int chunk = (int)cdiv(cdiv(a.k_len, n_chunks), kTileKeys) * kTileKeys;
  const int n_used = (int)cdiv(a.k_len, chunk);
  hipLaunchKernelGGL((sparse_attn_kernel<DSA_KV_HEADS, kSplitNW>), dim3(n_used, DSA_KV_HEADS, a.T),
                     dim3(kSplitNW * 64), 0, st, a, n_used, chunk, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_merge_kernel<DSA_KV_HEADS>), dim3(64, a.T), dim3(128), 0, st, a, n_used,
                     (const float*)part);
  return hipGetLastError();
}

hipError_t launch_swa_attn(const AttnArgs& a, void* scratch, hipStream_t st) {
  (void)scratch;
  const int chunk = (int)cdiv(a.window, kTileKeys) * kTileKeys;
  hipLaunchKernelGGL((swa_attn_kernel<SWA_KV_HEADS, kNW>), dim3(1, SWA_KV_HEADS, a.T), dim3(kNW * 64), 0, st, a,
                     1, chunk, (float*)nullptr);
  return hipGetLastError();
}

}  // namespace dsa
