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

// List position p -> cache row, or -1 for an empty slot (p >= p1 included).
// The position is clamped into the list and its entry always read, then
// masked: a read under a branch would be waited for inside the branch, so
// the reads of a tile would run one after another instead of together.
struct IdxList {
  const int32_t* row_idx;   // idx[t] row
  int len;                  // >= 1
  int64_t n_rows;
  __device__ int64_t row(int p, int p1) const {
    const int32_t j = row_idx[p < len ? p : len - 1];
    const bool ok = (p < p1) & (p < len) & (j >= 0) & ((int64_t)j < n_rows);   // no short-circuit branch
    return ok ? (int64_t)j : -1;
  }
};

struct Window {
  int64_t first;            // cache row of list position 0
  int len;
  int64_t n_rows;
  __device__ int64_t row(int p, int p1) const {
    const int64_t r = first + p;
    const bool ok = (p < p1) & (p < len) & (r >= 0) & (r < n_rows);
    return ok ? r : -1;
  }
};

// 2^x on the exp unit (v_exp_f32): 1 for 0, 0 for -inf, results below the
// smallest normal float flushed to zero -- a softmax term that small is below
// 2^-126 of its row's largest term (which is 1) and cannot change a sum of
// them by a float ulp
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// ds_read_b64_tr_b16 (gfx950): a transposing 8-byte LDS read, see the P.V
// operand below for its lane layout (measured on the hardware with distinct
// values in every LDS element); p must be an 8-byte aligned LDS address
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<uint16_t*>(p)));
}

// Orders a wave's LDS accesses before and after this point (compiler and
// hardware: a wave's LDS operations complete in order).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// NTB: threads of the workgroup (at least NW waves); waves beyond NW only take
// part in the combine's barriers.
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
  // read 64 contiguous bytes per load).  With fewer than 16 query heads per KV
  // head (GH = 8) columns GH .. 15 repeat real heads: their logits, weights
  // and output rows are never combined or written, and no value is masked, so
  // nothing waits for these loads before the K/V loads are issued.
  bf16x8 qf[6];
  {
    const int h = g * GH + (col % GH);
    const uint16_t* qp = a.q + ((size_t)t * 64 + h) * 192 + 8 * kg;
#pragma unroll
    for (int s = 0; s < 6; ++s) qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(qp + 32 * s));
  }
  // The combine's thread layout (see below) and, for a unit in one chunk, the
  // sink logits of the heads this thread writes, loaded now with the queries
  // (read after the combine they would add a round trip at the very end).
  // Without a sink the loads read the query instead and are discarded.
  // Pass p of thread i combines head (p NC + i) / 32, dims 4 ((p NC + i) % 32)
  // .. + 3, NC = NW * 64 threads.
  constexpr int NC = NW * 64;
  constexpr int P = GH * 32 / NC;              // passes
  static_assert(GH * 32 % NC == 0, "combine layout");
  const int ci = (int)(threadIdx.x & (NC - 1));
  float sinkv[P];
  {
    const float* sp = a.sink ? a.sink + g * GH : reinterpret_cast<const float*>(a.q);
#pragma unroll
    for (int p = 0; p < P; ++p) sinkv[p] = sp[(p * NC + ci) >> 5];
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
    bf16x8 pf, pl;           // P as bf16 high and low parts: pf + pl carries ~16 bits of each probability
    if (active) {
      // ---- all index and row loads first: one dependent round trip per tile.
      // Every load instruction reads whole runs of a few rows: K, 64 bytes of
      // each of 16 rows; V, load i covers keys 4 i .. 4 i + 3, 16 lanes per
      // 256-byte row.
      int64_t rk[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        rk[b] = src.row(tb + b * 16 + col, p1);
      }
      int64_t rv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        rv[i] = src.row(tb + 4 * i + (lane >> 4), p1);
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
      __builtin_amdgcn_sched_barrier(0);   // every load leaves before the QK (the scheduler would delay V's)
      // ---- QK for the two 16-key blocks (waits for the K rows only)
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
      // before a wave's first tile its running sums are zero: nothing to rescale
      const bool rescale = rd > 0;                  // wave-uniform
      const float alpha = (dead || !rescale) ? 1.0f : exp2_hw(m - mn);
      float ps = 0.f;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = dead ? 0.0f : exp2_hw(z[b][i] - mn);
          ps += pv;
          const __bf16 hi = (__bf16)pv;
          pf[b * 4 + i] = hi;
          pl[b * 4 + i] = (__bf16)(pv - (float)hi);
        }
      lsum = lsum * alpha + ps;
      m = mn;
      // rescale O rows (heads 4*kg + i) by their column's alpha
      if (rescale) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float al = __shfl(alpha, 4 * kg + i, 64);
#pragma unroll
          for (int b = 0; b < 8; ++b) o[b][i] *= al;
        }
      }
      // ---- stage V rows, after QK and the softmax so that those need not
      // wait for them (the V loads are issued last).  An empty slot stages
      // zeros, never the row it loaded: the row is ANDed with a mask that an
      // empty asm hides from the compiler, since a select between the loaded
      // row and zeros let it move that load into a branch followed by a wait
      // for every outstanding load, ahead of the QK.
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int msk = rv[i] >= 0 ? -1 : 0;
        asm volatile("" : "+v"(msk));
        *reinterpret_cast<i32x4*>(vs + (4 * i + (lane >> 4)) * kVStride + 8 * (lane & 15)) =
            __builtin_bit_cast(i32x4, vraw[i]) & msk;
      }
    }
    // the V staging area is the wave's own: its stores precede its reads
    // (LDS operations of a wave complete in order), so no workgroup barrier
    // holds this wave for the slowest wave's loads
    wave_lds_sync();
    if (active) {
      // ---- PV: B operand = V[key(kg,e)][16*blk + col], key(kg,e) = e<4 ? 4kg+e : 12+4kg+e.
      // Two LDS transpose reads per 16-dim block: in each 16-lane group,
      // ds_read_b64_tr_b16 gives lane i, element s, element i % 4 of the 8
      // bytes that lane i / 4 + 4 s of the group addresses; lane q of group kg
      // addresses dims 4 (q % 4) .. + 3 of key row 4 kg + q / 4 (keys 0-15)
      // and the same 16 rows down (keys 16-31), so lane (kg, col) receives
      // V[4 kg + s][16 blk + col] and V[16 + 4 kg + s][16 blk + col].
      const int tq = lane & 15;
      const uint16_t* vr = vs + (4 * kg + (tq >> 2)) * kVStride + 4 * (tq & 3);
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) {
        const s16x4 lo = lds_read_tr16(vr + blk * 16);
        const s16x4 hi = lds_read_tr16(vr + 16 * kVStride + blk * 16);
        const u16x8 vb = u16x8{(uint16_t)lo[0], (uint16_t)lo[1], (uint16_t)lo[2], (uint16_t)lo[3],
                               (uint16_t)hi[0], (uint16_t)hi[1], (uint16_t)hi[2], (uint16_t)hi[3]};
        o[blk] = mfma_bf16_16x16x32(pf, __builtin_bit_cast(bf16x8, vb), o[blk]);
        o[blk] = mfma_bf16_16x16x32(pl, __builtin_bit_cast(bf16x8, vb), o[blk]);
      }
    }
    wave_lds_sync();                                        // this round's reads before the next round's stores
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

  // every thread combines, per pass, four dims of one head from the NW wave
  // partials: all LDS reads (16-byte pieces for the outputs) are issued
  // before any result is written
  const int unit = t * HKV + g;
  float Mp[P], Lp[P];
  float4 Op[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int idx = p * NC + ci;
    const int hc = idx >> 5, dq = (idx & 31) * 4;
    float mwv[NW], lwv[NW];
    float4 owv[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mwv[w] = mw[w * 16 + hc];
      lwv[w] = lw[w * 16 + hc];
      owv[w] = *reinterpret_cast<const float4*>(ow + (w * 16 + hc) * 128 + dq);
    }
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, mwv[w]);
    float L = 0.f;
    float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = M == -INFINITY ? 0.f : exp2_hw(mwv[w] - M);
      L += f * lwv[w];
      O.x += f * owv[w].x;
      O.y += f * owv[w].y;
      O.z += f * owv[w].z;
      O.w += f * owv[w].w;
    }
    Mp[p] = M;
    Lp[p] = L;
    Op[p] = O;
  }
  if (n_chunks == 1) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int idx = p * NC + ci;
      const int hc = idx >> 5, dq = (idx & 31) * 4;
      const int h = g * GH + hc;
      const float M = Mp[p], L = Lp[p];
      float Mf = M;
      float sl = 0.f;
      if (a.sink) {
        const float s2 = sinkv[p] * kLog2e;
        Mf = fmaxf(M, s2);
        sl = exp2_hw(s2 - Mf);
      }
      float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
      float Lf = 0.f;
      if (Mf != -INFINITY) {
        const float sc = M == -INFINITY ? 0.f : exp2_hw(M - Mf);
        Lf = L * sc + sl;
        if (Lf > 0.f) {
          const float inv = sc / Lf;                        // one division for the four dims
          r = make_float4(Op[p].x * inv, Op[p].y * inv, Op[p].z * inv, Op[p].w * inv);
        }
      }
      *reinterpret_cast<uint2*>(a.out + ((size_t)t * 64 + h) * 128 + dq) =
          make_uint2(f32x2_to_bf16x2_rne(r.x, r.y), f32x2_to_bf16x2_rne(r.z, r.w));
      if (a.lse && (idx & 31) == 0)
        a.lse[(size_t)t * 64 + h] = Mf == -INFINITY ? -INFINITY : (Mf + log2f(Lf)) * kLn2;
    }
  } else {
    float* pp = part + ((size_t)unit * n_chunks + c) * kPartFloats;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int idx = p * NC + ci;
      const int hc = idx >> 5, dq = (idx & 31) * 4;
      if ((idx & 31) == 0) {
        pp[hc] = Mp[p];
        pp[16 + hc] = Lp[p];
      }
      *reinterpret_cast<float4*>(pp + 32 + hc * 128 + dq) = Op[p];
    }
  }
}


}  // namespace dsa
