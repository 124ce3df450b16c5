// select.hpp -- block-level exact radix selection on order-preserving 32-bit
// keys (internal to libdsa.so).
//
// The selection rule is the top-k one: keep the `need` largest keys, ties at
// the threshold broken towards the earlier element.  Keys are found with a
// three-digit radix descent (bits 31..20, 19..8, 7..0) over an array that a
// functor exposes; the result is the threshold key tau and r, the number of
// elements equal to tau that are kept (r >= 1).
#pragma once

#include "dsa_common.hpp"

namespace dsa {

// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele within each
// row of 16 lanes by DPP row shifts, then the row totals are carried across
// rows by the row broadcasts of lane 15 and lane 31.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);   // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);   // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);   // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);   // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);   // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);   // row_bcast:31
  return x;
}

// Inclusive max / min over the lanes of a wave by the same DPP steps; lane 63
// holds the wave's result.
template <bool kMax>
__device__ __forceinline__ uint32_t wave_incl_minmax(uint32_t x) {
  const int id = kMax ? 0 : -1;
  auto op = [](uint32_t a, uint32_t b) { return kMax ? (a > b ? a : b) : (a < b ? a : b); };
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x111, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x112, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x114, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x118, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x142, 0xA, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x143, 0xC, 0xF, false));
  return x;
}

// Block-wide max of a, min of b, min of c and sum of n, returned to every
// thread; sm holds 4 * (NT / 64) words.
template <int NT>
__device__ __forceinline__ void block_reduce_mmms(uint32_t& a, uint32_t& b, uint32_t& c, uint32_t& n,
                                                  uint32_t* sm) {
  constexpr int W = NT / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint32_t ra = wave_incl_minmax<true>(a), rb = wave_incl_minmax<false>(b);
  const uint32_t rc = wave_incl_minmax<false>(c), rn = wave_incl_scan(n);
  if (lane == 63) {
    sm[wv] = ra;
    sm[W + wv] = rb;
    sm[2 * W + wv] = rc;
    sm[3 * W + wv] = rn;
  }
  __syncthreads();
  a = 0u;
  b = c = 0xFFFFFFFFu;
  n = 0u;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    a = a > sm[i] ? a : sm[i];
    b = b < sm[W + i] ? b : sm[W + i];
    c = c < sm[2 * W + i] ? c : sm[2 * W + i];
    n += sm[3 * W + i];
  }
  __syncthreads();
}

// Exclusive prefix sum over the block; *total receives the block sum.  All
// threads must call it; sm holds NT / 64 words.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sm, uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) sm[wv] = x;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    uint32_t s = sm[i];
    base += (i < wv) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// Largest bin b with suffix(b) = sum_{b' >= b} hist[b'] >= need (need >= 1 and
// the histogram total >= need).  Writes the bin and suffix(b + 1) to *bin and
// *above (shared).  All threads must call it.  hist must be 16-byte aligned
// when NB / NT is a multiple of 4.
template <int NT, int NB>
__device__ __forceinline__ void find_threshold_bin(const uint32_t* hist, uint32_t need, uint32_t* scan_sm,
                                   uint32_t* bin, uint32_t* above) {
  constexpr int PER = NB >= NT ? NB / NT : 1;
  static_assert(NB < NT || PER * NT == NB, "bins per thread");
  const int j = threadIdx.x;
  const int base = NB - (j + 1) * PER;          // thread 0 owns the top bins
  const bool owns = base >= 0;                  // threads beyond the bins own none
  uint32_t h[PER];
  uint32_t sum = 0;
  if constexpr (PER % 4 == 0) {
#pragma unroll
    for (int i = 0; i < PER; i += 4) {
      const uint4 q = owns ? *reinterpret_cast<const uint4*>(hist + base + i) : make_uint4(0u, 0u, 0u, 0u);
      h[i] = q.x;
      h[i + 1] = q.y;
      h[i + 2] = q.z;
      h[i + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) h[i] = owns ? hist[base + i] : 0u;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) sum += h[i];
  uint32_t tot;
  const uint32_t excl = block_excl_scan<NT>(sum, scan_sm, &tot);
  if (owns && excl < need && excl + sum >= need) {
    uint32_t acc = excl;
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) {
      if (acc + h[i] >= need) {
        *bin = (uint32_t)(base + i);
        *above = acc;
        break;
      }
      acc += h[i];
    }
  }
  __syncthreads();
}

// block_excl_scan with one barrier: sm (NT / 64 words) is written once and
// must not be written again by the block without a barrier in between.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan_once(uint32_t v, uint32_t* sm, uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) sm[wv] = x;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const uint32_t s = sm[i];
    base += (i < wv) ? s : 0u;
    tot += s;
  }
  *total = tot;
  return base + x - v;
}

// find_threshold_bin with two barriers, returning to every thread the bin,
// the entries in the bins above it and the entries in it.  sm (NT / 64 words)
// and out (3 words) are written once, as in block_excl_scan_once.
template <int NT, int NB>
__device__ __forceinline__ void find_threshold_bin_once(const uint32_t* hist, uint32_t need, uint32_t* sm,
                                                        uint32_t* out, uint32_t* bin, uint32_t* above,
                                                        uint32_t* count) {
  constexpr int PER = NB / NT;
  static_assert(PER * NT == NB && PER % 4 == 0, "bins per thread");
  const int base = NB - ((int)threadIdx.x + 1) * PER;      // thread 0 owns the top bins
  uint32_t h[PER];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < PER; i += 4) {
    const uint4 q = *reinterpret_cast<const uint4*>(hist + base + i);
    h[i] = q.x;
    h[i + 1] = q.y;
    h[i + 2] = q.z;
    h[i + 3] = q.w;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) sum += h[i];
  uint32_t tot;
  const uint32_t excl = block_excl_scan_once<NT>(sum, sm, &tot);
  if (excl < need && excl + sum >= need) {
    uint32_t acc = excl;
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) {
      if (acc + h[i] >= need) {
        out[0] = (uint32_t)(base + i);
        out[1] = acc;
        out[2] = h[i];
        break;
      }
      acc += h[i];
    }
  }
  __syncthreads();
  *bin = out[0];
  *above = out[1];
  *count = out[2];
}

struct alignas(16) RadixShared {
  uint32_t hist[kHistBins];
  uint32_t scan[16];
  uint32_t bin, above;
};

// Threshold of the `need` largest of n keys key_at(i) (i < n).  Inactive
// elements must report key 0 and there must be at least `need` keys > 0.
// Returns tau in *tau_out and the count of tau-equal keys to keep in *r_out;
// *eq_out receives the number of keys equal to tau.
template <int NT, class KeyAt>
__device__ __forceinline__ void radix_threshold(const KeyAt& key_at, int n, uint32_t need, RadixShared& rs, uint32_t* tau_out,
                                uint32_t* r_out, uint32_t* eq_out) {
  // level 1: bits 31..20
  for (int i = threadIdx.x; i < kHistBins; i += NT) rs.hist[i] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += NT) {
    const uint32_t key = key_at(i);
    if (key) atomicAdd(&rs.hist[key >> 20], 1u);
  }
  __syncthreads();
  find_threshold_bin<NT, kHistBins>(rs.hist, need, rs.scan, &rs.bin, &rs.above);
  const uint32_t b1 = rs.bin;
  const uint32_t k1 = need - rs.above;
  // level 2: bits 19..8 of the keys in bin b1
  for (int i = threadIdx.x; i < kHistBins; i += NT) rs.hist[i] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += NT) {
    const uint32_t key = key_at(i);
    if (key && (key >> 20) == b1) atomicAdd(&rs.hist[(key >> 8) & 0xFFF], 1u);
  }
  __syncthreads();
  find_threshold_bin<NT, kHistBins>(rs.hist, k1, rs.scan, &rs.bin, &rs.above);
  const uint32_t pre = (b1 << 12) | rs.bin;
  const uint32_t k2 = k1 - rs.above;
  // level 3: bits 7..0
  for (int i = threadIdx.x; i < kHist3Bins; i += NT) rs.hist[i] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += NT) {
    const uint32_t key = key_at(i);
    if (key && (key >> 8) == pre) atomicAdd(&rs.hist[key & 0xFF], 1u);
  }
  __syncthreads();
  find_threshold_bin<NT, kHist3Bins>(rs.hist, k2, rs.scan, &rs.bin, &rs.above);
  const uint32_t b3 = rs.bin;
  *tau_out = (pre << 8) | b3;
  *r_out = k2 - rs.above;
  *eq_out = rs.hist[b3];
  __syncthreads();
}

// Ordered compaction of the kept elements: element i is kept when
// key_at(i) > tau, or key_at(i) == tau and fewer than r tau-equal elements
// precede it (in i order).  emit(pos, i) is called for every kept element with
// its output position.  Each thread walks a contiguous run of i.  Returns the
// number kept (block-uniform).
template <int NT, class KeyAt, class Emit>
__device__ __forceinline__ uint32_t ordered_keep(const KeyAt& key_at, int n, uint32_t tau, uint32_t r, uint32_t* scan_sm,
                                 const Emit& emit) {
  const int per = (n + NT - 1) / NT;
  const int i0 = threadIdx.x * per;
  const int i1 = i0 + per < n ? i0 + per : n;
  uint32_t n_gt = 0, n_eq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = key_at(i);
    n_gt += key > tau;
    n_eq += key == tau;
  }
  uint32_t tot_gt, tot_eq;
  const uint32_t gt_base = block_excl_scan<NT>(n_gt, scan_sm, &tot_gt);
  const uint32_t eq_base = block_excl_scan<NT>(n_eq, scan_sm, &tot_eq);
  uint32_t pos = gt_base + (eq_base < r ? eq_base : r);
  uint32_t eq_seen = eq_base;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = key_at(i);
    bool take = key > tau;
    if (key == tau) {
      take = eq_seen < r;
      ++eq_seen;
    }
    if (take) emit(pos++, i);
  }
  return tot_gt + (tot_eq < r ? tot_eq : r);
}

}  // namespace dsa

namespace dsa {

// Sorts the `need` indices in sel[0 .. need) (sel holds DSA_TOPK_MAX words)
// ascending and writes them to out[0 .. k), padded with -1.  All NT threads
// call it after the indices are in place; it ends with a barrier.
template <int NT>
__device__ __forceinline__ void sort_emit(uint32_t* sel, uint32_t need, int k, int32_t* out) {
  constexpr int kSortN = DSA_TOPK_MAX;
  for (uint32_t i = need + threadIdx.x; i < (uint32_t)kSortN; i += NT) sel[i] = 0xFFFFFFFFu;
  // bitonic sort of the kSortN slots, ascending
  for (int size = 2; size <= kSortN; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int i = threadIdx.x; i < kSortN / 2; i += NT) {
        const int a = 2 * i - (i & (stride - 1));
        const int b = a + stride;
        const uint32_t x = sel[a], y = sel[b];
        const bool up = (a & size) == 0;
        if ((x > y) == up) {
          sel[a] = y;
          sel[b] = x;
        }
      }
    }
  }
  __syncthreads();
  for (int j = threadIdx.x; j < k; j += NT) out[j] = j < (int)need ? (int32_t)sel[j] : -1;
  __syncthreads();
}

// Writes the indices of the set bits of bm[0 .. nw) in ascending order to
// out[0 .. k), padded with -1: every thread counts the bits of a run of
// words, one prefix sum places the runs.  All NT threads call it after the
// bits are set; it ends with a barrier.
template <int NT>
__device__ __forceinline__ void bitmap_emit(const uint32_t* bm, int nw, uint32_t* scan_sm, int k, int32_t* out) {
  const int per = (nw + NT - 1) / NT;
  const int w0 = (int)threadIdx.x * per;
  const int w1 = w0 + per < nw ? w0 + per : nw;
  uint32_t c = 0;
  for (int w = w0; w < w1; ++w) c += (uint32_t)__popc(bm[w]);
  uint32_t tot;
  uint32_t pos = block_excl_scan<NT>(c, scan_sm, &tot);
  for (int w = w0; w < w1; ++w) {
    uint32_t x = bm[w];
    while (x) {
      const int b = __builtin_ctz(x);
      x &= x - 1u;
      if (pos < (uint32_t)k) out[pos] = w * 32 + b;
      ++pos;
    }
  }
  for (uint32_t j = tot + threadIdx.x; j < (uint32_t)k; j += NT) out[j] = -1;
  __syncthreads();
}

// The exact top `need` (need <= DSA_TOPK_MAX) of n candidates (order keys
// ckey[i] > 0, key indices cidx[i]) by (key desc, index asc), written to
// out[0 .. k) in ascending index order and padded with -1.  The threshold
// key and, among keys equal to it, the largest kept index come from radix
// descents; the kept indices are collected in sel (DSA_TOPK_MAX words) and
// sorted there.  All NT threads call it; it ends with a barrier.
template <int NT>
__device__ __forceinline__ void select_sorted(const uint32_t* ckey, const uint32_t* cidx, int n, uint32_t need,
                                              int k, RadixShared& rs, uint32_t* sel, uint32_t* nsel,
                                              int32_t* out) {
  if (threadIdx.x == 0) *nsel = 0;
  uint32_t tau, r, eq;
  radix_threshold<NT>([&](int i) { return ckey[i]; }, n, need, rs, &tau, &r, &eq);
  // among tau-equal entries the r lowest indices win: threshold on ~index
  uint32_t imax = 0xFFFFFFFFu;
  if (eq > r) {
    uint32_t tau2, r2, eq2;
    radix_threshold<NT>([&](int i) { return ckey[i] == tau ? ~cidx[i] : 0u; }, n, r, rs, &tau2, &r2, &eq2);
    imax = ~tau2;
  }
  for (int i = threadIdx.x; i < n; i += NT) {
    const uint32_t key = ckey[i], id = cidx[i];
    if (key > tau || (key == tau && id <= imax)) sel[atomicAdd(nsel, 1u)] = id;
  }
  __syncthreads();
  sort_emit<NT>(sel, need, k, out);
}

}  // namespace dsa
