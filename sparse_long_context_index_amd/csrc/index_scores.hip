// index_scores.hip -- lightning-indexer scores on gfx950.
//
// S[t,s] = sum_h w[t,h] * max(q_idx[t,h,:] . k_idx[s,:], 0) for s <= p_t, -inf
// beyond ("Naive-N0.5-Flash: no full-attention layers, and a runtime built by
// AI", section "Inside a DSA layer: the lightning indexer": 16 fp8 query heads
// against one shared fp8 key head, ReLU of the dot, per-head weights combine
// them into one score per key).
//
// Both kernels put the 16 index heads on the M dimension of a 16x16 MFMA and
// 16 keys on N, so one accumulator holds all head logits of 16 keys for one
// query token: 4 heads of one key per lane.  The ReLU-weighted head sum is 4
// FMAs in the lane plus two cross-lane-group butterflies.
//
//  * idx_scan_kernel<T> (T <= 8, decode / speculative verify): a coalesced
//    stream over the 128-byte fp8 key rows (2 KiB per 16-key tile, several
//    tiles in flight per wave).  The stream is HBM-bound, so the dot engine
//    can afford exactness: fp8 bytes are widened to bf16 in registers
//    (lossless) and multiplied on the bf16 MFMA, whose products are exact and
//    whose sums are fp32-accurate.  Optionally the kernel also builds the
//    level-1 radix histogram of its scores for the top-k that follows.
//  * T > 8 (prefill) goes to idx_gemm_kernel (prefill_scores.hip).
#include "dsa_common.hpp"
#include "indexer.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace dsa {

namespace {

constexpr int kScanUnroll = 4;   // 16-key tiles per wave in flight
constexpr int kScanBlocks = 512; // persistent workgroups of the list scan (2 per CU): one list each
constexpr int kPlainScanBlocks = 768;   // persistent workgroups of the scan without lists (3 per CU)

__device__ __forceinline__ i32x8 load_frag32(const uint8_t* p) {
  // 32 bytes as two 16-byte loads (only 16-byte alignment is guaranteed)
  const i32x4* q = reinterpret_cast<const i32x4*>(p);
  i32x4 lo = __builtin_nontemporal_load(q);
  i32x4 hi = __builtin_nontemporal_load(q + 1);
  i32x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// Decode scan.  Without lists, persistent workgroups (3 per CU) take groups
// of 16 consecutive 16-key tiles in grid-stride order.  With lists, 16-key
// tiles are dealt round-robin to the workgroups (tile j belongs to workgroup
// j % G), so any run of consecutive keys is spread over many workgroups and
// their lists.  Either way the chip streams one contiguous stretch of the key
// cache at any moment.  Each wave takes kScanUnroll tiles per step, loads each
// with fully coalesced 16-byte loads (1 KiB per instruction), stages it in a
// wave-private LDS area with a padded row stride, and reads it back in MFMA
// operand order (key = lane % 16, 32 bytes of k-group lane / 16).  The next
// step's loads are in flight while the current one is scored.
//
// with_hist: also build the level-1 radix histogram of the scores (top-k's
// first digit) with two 16-bit counters per LDS word; the workgroup adds its
// counts to replica blockIdx.x % kHistReplicas.
//
// lists (optional, exclusive with with_hist): every wave also keeps, per
// query row, the running top kListM of the keys it has scored: keys above the
// wave's threshold are appended to a wave-private LDS buffer, and a buffer
// that passes kBufTrigger entries is cut back to its exact top kListM, whose
// smallest key becomes the new threshold (a later key equal to it has a larger
// index and cannot enter).  At the end the four wave sets are merged by rank
// into the workgroup's exact top kListM, written as a list sorted by (score
// desc, index asc) of order keys and key indices, with a count word (bit 31:
// more than kListM of its keys were visible).  The fused decode step selects
// the global top-k from these lists.  The scores themselves are stored only
// when asked for (store_scores): the selection needs them only in its rare
// re-selection, which can recompute them.
constexpr int kStageRow = 144;                     // padded LDS bytes per 128-byte key row
constexpr int kBufCap = 256;                       // wave buffer entries per row
constexpr int kBufTrigger = kBufCap - 4 * 16;      // room for one more step of appends

template <int T>
struct ListShared {
  alignas(16) uint32_t bk[4][T][kBufCap];          // wave buffers: order keys
  alignas(16) uint32_t bi[4][T][kBufCap];          // and key indices
  uint32_t rank[T][4 * kListM];                    // merge: partial ranks of the wave sets' entries
};
static_assert(sizeof(ListShared<1>) == 8 * 4 * kBufCap + 4 * 4 * kListM, "list LDS size");
static_assert(sizeof(ListShared<4>) == 4 * (8 * 4 * kBufCap + 4 * 4 * kListM), "list LDS size");

// Cuts a wave's buffer (n entries, n <= kBufCap) back to its top kListM by
// (key desc, index asc), in place and in no particular order; returns the
// new count and sets *theta, when the buffer was cut, to a key at or below the
// smallest one kept and at or above every key dropped.
// The kListM-th key and, for ties, the kept indices are found bit by bit with
// ballots over the E entries each lane holds (n <= 64 E).
// The top kListM by (key desc, index asc) of the valid entries (v) that the
// wave's lanes hold, E each, when more than kListM are valid: sets keep[] and
// *theta (see wave_cut_top_e).
template <int E>
__device__ __forceinline__ void wave_top_keep(const uint32_t* kk, const uint32_t* ii, const bool* v, bool* keep,
                                              uint32_t* theta) {
  // Every count is a ballot of one comparison masked by a wave-uniform mask
  // (a ballot of a compound condition went through a per-lane 0/1 value and
  // a second comparison: two more VALU instructions per count)
  uint64_t vm[E];
#pragma unroll
  for (int q = 0; q < E; ++q) vm[q] = __ballot(v[q]);
  auto count_ge = [&](uint32_t x) {
    uint32_t c = 0;
#pragma unroll
    for (int q = 0; q < E; ++q) c += (uint32_t)__popcll(__ballot(kk[q] >= x) & vm[q]);
    return c;
  };
  // The candidates lie in [lo, hi], so the bits above the highest one in
  // which lo and hi differ are common to all and need no test.  The descent
  // finds the largest tau with at least kListM keys >= tau, and stops early at
  // a tau with exactly kListM (those keys are then the top kListM, and tau a
  // valid threshold: no key below it can enter).
  uint32_t hl = 0u, ll = 0xFFFFFFFFu;
#pragma unroll
  for (int q = 0; q < E; ++q)
    if (v[q]) {
      hl = hl > kk[q] ? hl : kk[q];
      ll = ll < kk[q] ? ll : kk[q];
    }
  const uint32_t hi = __builtin_amdgcn_readlane(wave_incl_minmax<true>(hl), 63);
  const uint32_t lo = __builtin_amdgcn_readlane(wave_incl_minmax<false>(ll), 63);
  const uint32_t diff = hi ^ lo;
  uint32_t tau = diff ? hi & ~(0xFFFFFFFFu >> __builtin_clz(diff)) : hi;
  for (int bit = diff ? 31 - __builtin_clz(diff) : -1; bit >= 0; --bit) {
    const uint32_t tr = tau | (1u << bit);
    const uint32_t c = count_ge(tr);
    if (c >= (uint32_t)kListM) {
      tau = tr;
      if (c == (uint32_t)kListM) break;
    }
  }
  const uint32_t above = tau == 0xFFFFFFFFu ? 0u : count_ge(tau + 1u);
  const uint32_t r = (uint32_t)kListM - above;             // tau-equal entries to keep
  uint32_t eq = 0;
  uint64_t em[E];                                          // valid entries equal to tau
#pragma unroll
  for (int q = 0; q < E; ++q) {
    em[q] = __ballot(kk[q] == tau) & vm[q];
    eq += (uint32_t)__popcll(em[q]);
  }
  uint32_t imax = 0xFFFFFFFFu;                             // keep tau-equal entries with index <= imax
  if (eq > r) {
    uint32_t y = 0;                                        // the r-th largest ~index among them
#pragma unroll
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t tr = y | (1u << bit);
      uint32_t cnt = 0;
#pragma unroll
      for (int q = 0; q < E; ++q) cnt += (uint32_t)__popcll(__ballot(~ii[q] >= tr) & em[q]);
      if (cnt >= r) y = tr;
    }
    imax = ~y;
  }
#pragma unroll
  for (int q = 0; q < E; ++q) keep[q] = v[q] && (kk[q] > tau || (kk[q] == tau && ii[q] <= imax));
  *theta = tau;
}

template <int E>
__device__ __forceinline__ uint32_t wave_cut_top_e(uint32_t* bk, uint32_t* bi, uint32_t n, uint32_t* theta) {
  const int lane = threadIdx.x & 63;
  bool v[E], keep[E];
  uint32_t kk[E], ii[E];
#pragma unroll
  for (int q = 0; q < E; ++q) {
    v[q] = (uint32_t)(lane + 64 * q) < n;
    kk[q] = bk[lane + 64 * q];
    ii[q] = bi[lane + 64 * q];
    if (!v[q]) kk[q] = 0u;
  }
  wave_top_keep<E>(kk, ii, v, keep, theta);
  const uint64_t below = (1ull << lane) - 1ull;
  uint32_t pos[E];
  uint32_t base = 0;
#pragma unroll
  for (int q = 0; q < E; ++q) {
    const uint64_t m = __ballot(keep[q]);
    pos[q] = base + (uint32_t)__popcll(m & below);
    base += (uint32_t)__popcll(m);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");   // all reads above precede the writes below
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int q = 0; q < E; ++q)
    if (keep[q]) {
      bk[pos[q]] = kk[q];
      bi[pos[q]] = ii[q];
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  return (uint32_t)kListM;
}

// wave_cut_top_e with as few entries per lane as n allows (n is wave-uniform)
__device__ __forceinline__ uint32_t wave_cut_top(uint32_t* bk, uint32_t* bi, uint32_t n, uint32_t* theta) {
  const uint32_t nu = __builtin_amdgcn_readfirstlane(n);
  if (nu <= (uint32_t)kListM) return nu;
  if (nu <= 64u) return wave_cut_top_e<1>(bk, bi, nu, theta);
  if (nu <= 128u) return wave_cut_top_e<2>(bk, bi, nu, theta);
  return wave_cut_top_e<kBufCap / 64>(bk, bi, nu, theta);
}

// (kj, ij) precedes (key, id) in (key desc, index asc) order
__device__ __forceinline__ uint32_t precedes(uint32_t kj, uint32_t ij, uint32_t key, uint32_t id) {
  return (uint32_t)(kj > key) | ((uint32_t)(kj == key) & (uint32_t)(ij < id));
}

// count of the N entries (16-byte aligned) preceding (key, id); all reads are
// issued before the comparisons
template <int N>
__device__ __forceinline__ uint32_t count_preceding(const uint32_t* ks, const uint32_t* is, uint32_t key,
                                                    uint32_t id) {
  uint4 k4[N / 4], i4[N / 4];
#pragma unroll
  for (int q = 0; q < N / 4; ++q) {
    k4[q] = *reinterpret_cast<const uint4*>(ks + 4 * q);
    i4[q] = *reinterpret_cast<const uint4*>(is + 4 * q);
  }
  uint32_t c = 0;
#pragma unroll
  for (int q = 0; q < N / 4; ++q)
    c += precedes(k4[q].x, i4[q].x, key, id) + precedes(k4[q].y, i4[q].y, key, id) +
         precedes(k4[q].z, i4[q].z, key, id) + precedes(k4[q].w, i4[q].w, key, id);
  return c;
}

// NV: list groups per workgroup (lists only).  Each group of four waves is
// one list's workgroup of the deal (group v of workgroup x is list NV x + v);
// with NV = 2 the two lists of a CU run in one workgroup, dispatched together.
template <int T, bool kLists, int NV = 1>
__global__ __launch_bounds__(256 * NV) void idx_scan_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint8_t* __restrict__ k_idx, int64_t Lk, float* __restrict__ scores,
    int64_t ld, int64_t ngroups, TopkCounters ctr, int with_hist, ScanLists lists, SeqBatch sb) {
  static_assert(NV == 1 || kLists, "list groups only with lists");
  const int vg = (int)(threadIdx.x >> 8);                       // this wave's list group
  int64_t wg = (int64_t)blockIdx.x * NV + vg, G = (int64_t)gridDim.x * NV;   // its list among the row's, and their number
  if (!kLists && sb.len) {
    // batch: the sequence b, its keys, queries and score rows
    int b = blockIdx.y;
    if (sb.spread) {
      // Workgroups dealt by length: every workgroup derives the same deal from
      // the lengths -- sequence i (ng_i key groups of N in all) gets 1 +
      // floor((768 - B) ng_i / N) workgroups, at most ng_i, in sequence order
      // -- and takes its place in it.  The deal uses at most 768 workgroups,
      // the number that runs at once (3 per CU), so none waits for a slot;
      // the grid has 768 + B, and the spares exit.  Grid dimension y is 1.
      __shared__ uint32_t deal_sm[4];
      __shared__ int64_t deal_out[3];
      int64_t f0;
      int64_t n_i = (int)threadIdx.x < sb.spread ? seq_keys(sb, threadIdx.x, &f0) - sb.tail : 0;
      n_i = n_i > 0 ? n_i : 0;
      const uint32_t ng = (uint32_t)cdiv(cdiv(n_i, 16), 4 * kScanUnroll);
      uint32_t N, used;
      (void)block_excl_scan<256>(ng, deal_sm, &N);
      uint32_t per = 0;
      if (ng) {
        per = 1u + (uint32_t)((uint64_t)(kPlainScanBlocks - sb.spread) * ng / N);
        per = per < ng ? per : ng;
      }
      const uint32_t ex = block_excl_scan<256>(per, deal_sm, &used);
      if (blockIdx.x >= used) return;                           // block-uniform: a spare workgroup
      if (blockIdx.x >= ex && blockIdx.x < ex + per) {
        deal_out[0] = threadIdx.x;
        deal_out[1] = blockIdx.x - ex;
        deal_out[2] = per;
      }
      __syncthreads();
      b = (int)deal_out[0];
      wg = deal_out[1];
      G = deal_out[2];
    }
    int64_t first;
    Lk = seq_keys(sb, b, &first) - sb.tail;
    Lk = Lk > 0 ? Lk : 0;
    const int ts = sb.tstride ? sb.tstride : T;
    q_idx += (size_t)b * ts * 16 * 128;
    w += (size_t)b * ts * 16;
    k_idx += first * 128;
    scores += (size_t)b * ts * ld;
    ngroups = cdiv(cdiv(Lk, 16), 4 * kScanUnroll);
    if (Lk == 0) return;
  }
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* stage = smem;                                        // [4 NV waves][U*16 rows][kStageRow]
  uint32_t* lhist = reinterpret_cast<uint32_t*>(smem + 4 * kScanUnroll * 16 * kStageRow);  // [T][2048]
  ListShared<T>& ls = reinterpret_cast<ListShared<T>*>(smem + 4 * NV * kScanUnroll * 16 * kStageRow)[vg];
  uint32_t bcnt[T], theta[T];                                   // wave buffer fill and threshold per row
#pragma unroll
  for (int t = 0; t < T; ++t) bcnt[t] = theta[t] = 0u;
  __shared__ uint32_t red_sm[4];
  const int lane = threadIdx.x & 63;
  const int wave = (threadIdx.x >> 6) & 3;                      // within its list group
  const int col = lane & 15;
  const int grp = lane >> 4;

  if (with_hist) {
    for (int i = threadIdx.x; i < T * kHistBins / 2; i += 256) lhist[i] = 0;
    __syncthreads();
  }

  bf16x8 a[T][4];
  float wv[T][4];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    widen_fp8(load_frag32_cached(q_idx + (size_t)(t * 16 + col) * 128 + 32 * grp), a[t]);
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[t][i] = w[t * 16 + 4 * grp + i];
  }

  const int64_t last = Lk - 1;
  const int64_t ntiles = cdiv(Lk, 16);
  uint8_t* st = stage + (threadIdx.x >> 6) * kScanUnroll * 16 * kStageRow;
  i32x4 buf[2 * kScanUnroll];
  // With lists, local tile lt of list wg is global tile wg + G * lt and step
  // `it` gives wave w of its group the local tiles 16 it + kScanUnroll w + u;
  // without, step `it` covers the group of 16 consecutive tiles blockIdx.x +
  // G * it, kScanUnroll of them per wave.  Load i covers 8 keys of tile i / 2.
  auto tile_of = [&](int it, int u) -> int64_t {
    if (kLists) return wg + G * ((int64_t)it * 4 * kScanUnroll + wave * kScanUnroll + u);
    return (wg + G * (int64_t)it) * 4 * kScanUnroll + wave * kScanUnroll + u;
  };
  auto load_step = [&](int it) {
#pragma unroll
    for (int i = 0; i < 2 * kScanUnroll; ++i) {
      int64_t key = tile_of(it, i >> 1) * 16 + 8 * (i & 1) + (lane >> 3);
      key = key < last ? key : last;                            // ragged tail: stay in bounds
      buf[i] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(k_idx + key * 128 + 16 * (lane & 7)));
    }
  };

  const int n_steps = kLists ? (int)cdiv(cdiv(ntiles - wg, G), 4 * kScanUnroll)
                             : (int)cdiv(ngroups - wg, G);
  int iter = 0;
  if (n_steps > 0) load_step(0);
  for (; iter < n_steps; ++iter) {
#pragma unroll
    for (int i = 0; i < 2 * kScanUnroll; ++i)
      *reinterpret_cast<i32x4*>(st + (8 * i + (lane >> 3)) * kStageRow + 16 * (lane & 7)) = buf[i];
    __builtin_amdgcn_wave_barrier();
    if (iter + 1 < n_steps) load_step(iter + 1);
#pragma unroll
    for (int u = 0; u < kScanUnroll; ++u) {
      const int64_t tile = tile_of(iter, u);
      if (tile >= ntiles) continue;                             // wave-uniform
      const int64_t key = tile * 16 + col;
      const uint8_t* rp = st + (u * 16 + col) * kStageRow + 32 * grp;
      const i32x4 lo = *reinterpret_cast<const i32x4*>(rp);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(rp + 16);
      i32x8 kr;
      kr[0] = lo[0]; kr[1] = lo[1]; kr[2] = lo[2]; kr[3] = lo[3];
      kr[4] = hi[0]; kr[5] = hi[1]; kr[6] = hi[2]; kr[7] = hi[3];
      bf16x8 b[4];
      widen_fp8(kr, b);
      float s[T];
#pragma unroll
      for (int t = 0; t < T; ++t) {
        f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) c = mfma_bf16_16x16x32(a[t][k4], b[k4], c);
        s[t] = relu_weighted_sum(c, wv[t]);
        if (key > Lk - T + t) s[t] = -INFINITY;       // causal: beyond p_t
      }
      if (kLists) {                                             // append the keys above the threshold
        const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const uint32_t kk = ((t & 3) == grp && key <= Lk - T + t) ? order_key(s[t]) : 0u;
          const bool pass = kk > theta[t];
          const uint64_t m = __ballot(pass);
          const uint32_t pos = bcnt[t] + (uint32_t)__popcll(m & below);
          if (pass) {
            ls.bk[wave][t][pos] = kk;
            ls.bi[wave][t][pos] = (uint32_t)key;
          }
          bcnt[t] += (uint32_t)__popcll(m);
        }
      }
      if (key < Lk && (!kLists || lists.store_scores)) {
#pragma unroll
        for (int t = 0; t < T; ++t)
          if ((t & 3) == grp) {
            scores[(int64_t)t * ld + key] = s[t];
            if (with_hist && key <= Lk - T + t) {
              const uint32_t bin = order_key(s[t]) >> 20;
              atomicAdd(&lhist[t * (kHistBins / 2) + (bin >> 1)], 1u << (16 * (bin & 1)));
            }
          }
      }
    }
    if (kLists) {
#pragma unroll
      for (int t = 0; t < T; ++t)
        if (__builtin_amdgcn_readfirstlane(bcnt[t]) > (uint32_t)kBufTrigger)
          bcnt[t] = wave_cut_top(ls.bk[wave][t], ls.bi[wave][t], bcnt[t], &theta[t]);
    }
    __builtin_amdgcn_wave_barrier();
  }
  if (with_hist) {
    __syncthreads();
    for (int t = 0; t < T; ++t) {
      flush_level1_packed<256>(ctr, blockIdx.x % kHistReplicas, t, lhist + t * (kHistBins / 2), red_sm);
      __syncthreads();
    }
  }
  if (kLists) {
    // each wave's exact top kListM per row, padded with key 0 (ranks below every key)
#pragma unroll
    for (int t = 0; t < T; ++t) {
      uint32_t* bk = ls.bk[wave][t];
      uint32_t* bi = ls.bi[wave][t];
      const uint32_t nw = wave_cut_top(bk, bi, bcnt[t], &theta[t]);
      if ((uint32_t)lane >= nw && lane < kListM) {
        bk[lane] = 0u;
        bi[lane] = 0xFFFFFFFFu;
      }
    }
    __syncthreads();
    // Wave w merges rows w, w + 4, ...: the row's top kListM of the four wave
    // sets (128 entries, two per lane, key 0 = empty), compacted into the
    // row's merge area, then each kept entry's rank among them (its place in
    // the list, sorted by key desc, index asc).
    const uint32_t bx = (uint32_t)wg, G32 = (uint32_t)G;
    const uint64_t below = (1ull << lane) - 1ull;
    for (int t = wave; t < T; t += 4) {                          // wave-uniform
      uint32_t kk[2], ii[2];
      bool v[2], keep[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        kk[q] = ls.bk[2 * q + (lane >> 5)][t][lane & 31];
        ii[q] = ls.bi[2 * q + (lane >> 5)][t][lane & 31];
        v[q] = kk[q] != 0u;
        keep[q] = v[q];
      }
      const uint32_t nv = (uint32_t)__popcll(__ballot(v[0])) + (uint32_t)__popcll(__ballot(v[1]));
      if (nv > (uint32_t)kListM) {
        uint32_t th;
        wave_top_keep<2>(kk, ii, v, keep, &th);
      }
      uint32_t* mk = ls.rank[t];                                 // kListM keys, then kListM indices
      uint32_t* mi = ls.rank[t] + kListM;
      const uint64_t m0 = __ballot(keep[0]), m1 = __ballot(keep[1]);
      const uint32_t nk = (uint32_t)__popcll(m0) + (uint32_t)__popcll(m1);
      const uint32_t pos0 = (uint32_t)__popcll(m0 & below), pos1 = (uint32_t)__popcll(m0) + (uint32_t)__popcll(m1 & below);
      if (keep[0]) {
        mk[pos0] = kk[0];
        mi[pos0] = ii[0];
      }
      if (keep[1]) {
        mk[pos1] = kk[1];
        mi[pos1] = ii[1];
      }
      if ((uint32_t)lane >= nk && lane < kListM) {             // padding ranks below every key
        mk[lane] = 0u;
        mi[lane] = 0xFFFFFFFFu;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const uint32_t P = (uint32_t)(Lk - T + t + 1);            // keys visible to row t
      // visible keys of this workgroup: whole tiles below P / 16, plus the partial one
      const uint32_t F = P >> 4, rem = P & 15u;
      uint32_t n_vis = F > bx ? (F - bx + G32 - 1) / G32 * 16u : 0u;
      if (rem && F >= bx && (F - bx) % G32 == 0) n_vis += rem;
      const bool full = n_vis > (uint32_t)kListM;
      const uint32_t kept = full ? (uint32_t)kListM : n_vis;
      if ((uint32_t)lane < nk) {
        const uint32_t key = mk[lane], id = mi[lane];
        const uint32_t rank = count_preceding<kListM>(mk, mi, key, id);
        const size_t off = ((size_t)t * kListM + rank) * G32 + bx;
        lists.keys[off] = key;
        lists.idx[off] = id;
      }
      if ((uint32_t)lane >= kept && lane < kListM) {             // unused entries
        const size_t off = ((size_t)t * kListM + lane) * G32 + bx;
        lists.keys[off] = 0u;
        lists.idx[off] = 0xFFFFFFFFu;
      }
      if (lane == 0) lists.count[(size_t)t * G32 + bx] = kept | (full ? 0x80000000u : 0u);
    }
  }
}

}  // namespace

int scan_grid(int64_t Lk) {
  // one list per workgroup and up to one workgroup per 16-key tile: a short
  // row still spreads over many lists (an 8K-key row over 512)
  const int64_t ntiles = cdiv(Lk, 16);
  return (int)(ntiles < kScanBlocks ? ntiles : kScanBlocks);
}

// the scan without lists streams groups of 16 consecutive tiles with 3
// workgroups per CU
static int plain_scan_grid(int64_t Lk) {
  const int64_t ngroups = cdiv(cdiv(Lk, 16), 4 * kScanUnroll);
  return (int)(ngroups < kPlainScanBlocks ? ngroups : kPlainScanBlocks);
}

int scan_list_cap(int64_t Lk) {
  const int64_t ngroups = cdiv(cdiv(Lk, 16), 4 * kScanUnroll);
  return (int)(cdiv(ngroups, plain_scan_grid(Lk)) * 4 * kScanUnroll * 16);   // workgroup 0 has the most
}

size_t scan_lds_bytes(int64_t Lk, int T, bool lists) {
  (void)Lk;
  return (size_t)4 * kScanUnroll * 16 * kStageRow +
         (lists ? (size_t)T * (8 * 4 * kBufCap + sizeof(uint32_t) * 4 * kListM) : 0);
}

hipError_t launch_index_scores(const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                               int64_t Lk, int T, float* scores, int64_t ld, hipStream_t st,
                               void* topk_counters, ScanLists lists) {
  const int with_hist = topk_counters != nullptr;
  if (with_hist && lists.keys) return hipErrorInvalidValue;
  const TopkCounters ctr = topk_counters ? counters_at(topk_counters) : TopkCounters{};
  if (T <= kDecodeTMax) {
    if (with_hist && T > kScanHistTMax) return hipErrorInvalidValue;
    const int64_t ntiles = cdiv(Lk, 16);
    const int64_t ngroups = cdiv(ntiles, 4 * kScanUnroll);
    // 16-bit histogram counters: a workgroup must see fewer than 65536 keys
    const int64_t grid = lists.keys ? scan_grid(Lk) : plain_scan_grid(Lk);
    if (with_hist && scan_list_cap(Lk) >= 65536) return hipErrorInvalidValue;
    const size_t lds = scan_lds_bytes(Lk, T, lists.keys != nullptr) +
                       (with_hist ? (size_t)T * (kHistBins / 2) * sizeof(uint32_t) : 0);
    const bool with_lists = lists.keys != nullptr;
    // with several rows an even list grid runs two lists per workgroup (one
    // workgroup per CU: the two lists of a CU are dispatched together; with
    // one row the separate workgroups measured faster)
    const bool pairs = with_lists && T > 1 && grid % 2 == 0;
    if ((pairs ? 2 * lds : lds) > 160 * 1024) return hipErrorInvalidValue;
    if (with_lists && T > kScanListTMax) return hipErrorInvalidValue;
    switch (T) {
#define DSA_SCAN_PLAIN(n)                                                                                   \
  hipLaunchKernelGGL((idx_scan_kernel<n, false>), dim3((unsigned)grid), dim3(256), lds, st, q_idx, w, k_idx, Lk, \
                     scores, ld, ngroups, ctr, with_hist, lists, SeqBatch{})
#define DSA_SCAN_CASE(n)                                                                                    \
  case n:                                                                                                   \
    if (with_lists && n > 1 && grid % 2 == 0)                                                               \
      hipLaunchKernelGGL((idx_scan_kernel<n, true, 2>), dim3((unsigned)(grid / 2)), dim3(512), 2 * lds, st,  \
                         q_idx, w, k_idx, Lk, scores, ld, ngroups, ctr, with_hist, lists, SeqBatch{});      \
    else if (with_lists)                                                                                    \
      hipLaunchKernelGGL((idx_scan_kernel<n, true>), dim3((unsigned)grid), dim3(256), lds, st, q_idx, w,    \
                         k_idx, Lk, scores, ld, ngroups, ctr, with_hist, lists, SeqBatch{});                \
    else                                                                                                    \
      DSA_SCAN_PLAIN(n);                                                                                    \
    break;
      DSA_SCAN_CASE(1) DSA_SCAN_CASE(2) DSA_SCAN_CASE(3) DSA_SCAN_CASE(4)
      case 5: DSA_SCAN_PLAIN(5); break;
      case 6: DSA_SCAN_PLAIN(6); break;
      case 7: DSA_SCAN_PLAIN(7); break;
      case 8: DSA_SCAN_PLAIN(8); break;
#undef DSA_SCAN_CASE
#undef DSA_SCAN_PLAIN
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (with_hist) return hipErrorInvalidValue;
  return launch_idx_gemm(q_idx, w, k_idx, Lk, T, scores, ld, st);
}

hipError_t launch_index_scores_batch(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, const SeqBatch& sb,
                                     int B, int T, float* scores, int64_t ld, hipStream_t st) {
  if (B < 1 || T < 1 || ld < sb.max_len || B > 65535) return hipErrorInvalidValue;
  if (sb.tstride == 0 && T > kDecodeTMax) {
    // more tokens than one scan holds: the scan over groups of up to
    // kDecodeTMax tokens (the same exact arithmetic; the keys are read once
    // per group)
    for (int t0 = 0; t0 < T; t0 += kDecodeTMax) {
      const int tg = T - t0 < kDecodeTMax ? T - t0 : kDecodeTMax;
      SeqBatch g = sb;
      g.tstride = T;
      g.tail = T - t0 - tg;
      const hipError_t e = launch_index_scores_batch(q_idx + (size_t)t0 * 16 * 128, w + (size_t)t0 * 16, k_idx, g, B,
                                                     tg, scores + (size_t)t0 * ld, ld, st);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (T > kDecodeTMax) return hipErrorInvalidValue;
  const size_t lds = scan_lds_bytes(sb.max_len, T, false);
  const TopkCounters ctr{};
  const int64_t max_groups = cdiv(cdiv(sb.max_len, 16), 4 * kScanUnroll);
  if (B <= 256) {
    // workgroups dealt by length inside the kernel (768 + B, the spares exit)
    SeqBatch sp = sb;
    sp.spread = B;
    switch (T) {
#define DSA_SCAN_SPREAD(n)                                                                                  \
  case n:                                                                                                   \
    hipLaunchKernelGGL((idx_scan_kernel<n, false>), dim3((unsigned)(kPlainScanBlocks + B)), dim3(256), lds, st, \
                       q_idx, w, k_idx, sb.max_len, scores, ld, max_groups, ctr, 0, ScanLists{}, sp);       \
    break;
      DSA_SCAN_SPREAD(1) DSA_SCAN_SPREAD(2) DSA_SCAN_SPREAD(3) DSA_SCAN_SPREAD(4)
      DSA_SCAN_SPREAD(5) DSA_SCAN_SPREAD(6) DSA_SCAN_SPREAD(7) DSA_SCAN_SPREAD(8)
#undef DSA_SCAN_SPREAD
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  // more sequences: per sequence a share of the plain scan's workgroups, at most its key groups
  int64_t per = cdiv(kPlainScanBlocks, B);
  per = per < max_groups ? per : max_groups;
  per = per < 1 ? 1 : per;
  switch (T) {
#define DSA_SCAN_BATCH(n)                                                                                   \
  case n:                                                                                                   \
    hipLaunchKernelGGL((idx_scan_kernel<n, false>), dim3((unsigned)per, (unsigned)B), dim3(256), lds, st, q_idx, \
                       w, k_idx, sb.max_len, scores, ld, max_groups, ctr, 0, ScanLists{}, sb);              \
    break;
    DSA_SCAN_BATCH(1) DSA_SCAN_BATCH(2) DSA_SCAN_BATCH(3) DSA_SCAN_BATCH(4)
    DSA_SCAN_BATCH(5) DSA_SCAN_BATCH(6) DSA_SCAN_BATCH(7) DSA_SCAN_BATCH(8)
#undef DSA_SCAN_BATCH
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dsa
