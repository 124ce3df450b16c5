// attn_core.hpp -- the gathered-attention tile loop shared by the attention
// kernels (internal to libdsa.so).  See attn.hip for the method.
#pragma once

#include "dsa_common.hpp"
#include "kernels.hpp"

namespace dsa {

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

// NTB: threads of the workgroup (at least NW waves); waves beyond NW only take
// part in the barriers.
template <int HKV, int NW, class Src, int NTB = NW * 64>
__device__ __forceinline__ void attend_chunk(const AttnArgs& a, const Src& src, int t, int g, int c, int n_chunks,
                             int p0, int p1, float* part, char* smem) {
  constexpr int GH = 64 / HKV;              // query heads per KV head
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const bool wave_on = wave < NW;
  static_assert(NTB >= NW * 64 && NTB % 64 == 0, "workgroup shape");
  const int col = lane & 15;
  const int kg = lane >> 4;
  const float qscale = a.sm_scale * kLog2e;

  // Q as the B operand: column = head; k-step s, k-group kg covers dims
  // 32 s + 8 kg .. + 7 (K uses the same order, so the 4 k-groups of a key row
  // read 64 contiguous bytes per load)
  bf16x8 qf[6];
  {
    const bool hv = col < GH;
    const int h = g * GH + (hv ? col : 0);
    const uint16_t* qp = a.q + ((size_t)t * 64 + h) * 192 + 8 * kg;
#pragma unroll
    for (int s = 0; s < 6; ++s) {
      u16x8 raw = *reinterpret_cast<const u16x8*>(qp + 32 * s);
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
    const bool active = wave_on && tile < ntiles;   // wave-uniform
    const int tb = p0 + tile * kTileKeys;
    bf16x8 pf;
    if (active) {
      // ---- all index and row loads first: one dependent round trip per tile.
      // Every load instruction reads whole runs of a few rows: K, 64 bytes of
      // each of 16 rows; V, load i covers keys 4 i .. 4 i + 3, 16 lanes per
      // 256-byte row.
      int64_t rk[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int p = tb + b * 16 + col;
        rk[b] = p < p1 ? src.row(p) : -1;
      }
      int64_t rv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int p = tb + 4 * i + (lane >> 4);
        rv[i] = p < p1 ? src.row(p) : -1;
      }
      u16x8 kraw[2][6];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const uint16_t* kp = a.k + ((size_t)(rk[b] >= 0 ? rk[b] : 0) * HKV + g) * 192 + 8 * kg;
#pragma unroll
        for (int s = 0; s < 6; ++s) kraw[b][s] = *reinterpret_cast<const u16x8*>(kp + 32 * s);
      }
      u16x8 vraw[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        vraw[i] = *reinterpret_cast<const u16x8*>(a.v + ((size_t)(rv[i] >= 0 ? rv[i] : 0) * HKV + g) * 128 +
                                                  8 * (lane & 15));
      // ---- stage V rows (an empty slot stages zeros, never the row it loaded)
      {
        const u16x8 zero = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 8; ++i)
          *reinterpret_cast<u16x8*>(vs + (4 * i + (lane >> 4)) * kVStride + 8 * (lane & 15)) =
              rv[i] >= 0 ? vraw[i] : zero;
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
  if (wave_on) {
    if (lane < 16) {
      mw[wave * 16 + lane] = m;
      lw[wave * 16 + lane] = lsum;
    }
#pragma unroll
    for (int blk = 0; blk < 8; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) ow[(wave * 16 + 4 * kg + i) * 128 + blk * 16 + col] = o[blk][i];
  }
  __syncthreads();
  if (threadIdx.x >= NW * 64) return;

  // every thread combines outputs (head hc, dim dv) for hc = h0 + R*q; all
  // LDS reads are issued before any result is written
  const int unit = t * HKV + g;
  constexpr int R = NW * 64 / 128;             // heads covered per pass
  constexpr int Q = GH / R;                    // passes
  static_assert(NW * 64 % 128 == 0 && GH % R == 0, "combine layout");
  const int dv = threadIdx.x & 127;
  const int h0 = threadIdx.x >> 7;
  float Mq[Q], Lq[Q], Oq[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int hc = h0 + R * q;
    float mwv[NW], lwv[NW], owv[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mwv[w] = mw[w * 16 + hc];
      lwv[w] = lw[w * 16 + hc];
      owv[w] = ow[(w * 16 + hc) * 128 + dv];
    }
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, mwv[w]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = M == -INFINITY ? 0.f : exp2f(mwv[w] - M);
      L += f * lwv[w];
      O += f * owv[w];
    }
    Mq[q] = M;
    Lq[q] = L;
    Oq[q] = O;
  }
  if (n_chunks == 1) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int h = g * GH + h0 + R * q;
      const float M = Mq[q], L = Lq[q], O = Oq[q];
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
    }
  } else {
    float* pp = part + ((size_t)unit * n_chunks + c) * kPartFloats;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int hc = h0 + R * q;
      if (dv == 0) {
        pp[hc] = Mq[q];
        pp[16 + hc] = Lq[q];
      }
      pp[32 + hc * 128 + dv] = Oq[q];
    }
  }
}


}  // namespace dsa
