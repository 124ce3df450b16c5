// topk.hip -- exact per-row top-k with stable ties on gfx950.
//
// Semantics ("Naive-N0.5-Flash: no full-attention layers, and a runtime built
// by AI", section "What 'no full-attention layers' means": the DSA path keeps
// the first index_top_k entries of a descending argsort of the index scores;
// section "How much of this did AI actually build?": the argsort is stable):
// keep the min(k, n) visible keys ordered by (score desc, index asc) and emit
// them in ascending index order, padded with -1.
//
// Method: radix select on the order-preserving 32-bit key of each score in
// three digits (bits 31..20, 19..8, 7..0).  The threshold key tau is exact;
// keys above tau are kept, and of the keys equal to tau the r lowest indices
// are kept (r = k - #above).  Candidates are gathered in index order, so the
// emission is an ordered compaction -- no sort is needed and the result does
// not depend on scheduling.
//
//  * Few long rows (decode, T <= 16): many workgroups per row.
//      topk_hist_kernel     level-1 histogram (LDS, then global atomics)
//      topk_collect_kernel  each block finds the level-1 threshold digit,
//                           compacts its candidates (digit >= threshold) in
//                           order into its own slot, adds level-2 digits of
//                           the boundary bin to a global histogram; the last
//                           block of the row resolves tau and emits the row.
//  * Many rows (prefill), and rows too short for the multi-block path:
//    topk_row_kernel, one 1024-thread workgroup per row, candidates in LDS
//    (a row of up to 16,384 keys is held in LDS whole, one of up to 65,536
//    keys in registers).
// A candidate slot that overflows switches the row's final pass to reading
// the scores row itself (same result, slower).
#include "dsa_common.hpp"
#include "indexer.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace dsa {

namespace {

constexpr int kCollectThreads = 256;
constexpr int kCollectPer = 16;                                 // per thread
constexpr int kCollectRange = kCollectThreads * kCollectPer;    // per block
constexpr int kSlotCap = 512;                                   // candidates per block
constexpr int kMaxSegs = 1024;                                  // blocks per row (multi-block path)
constexpr int kCandCap = 16384;                                 // LDS candidates of the final block
constexpr int kHistRange = 2048;                                // per hist block
constexpr int kRowThreads = 1024;
constexpr int kRowCap = 6144;                                   // LDS candidates per row
constexpr int kRowReps = 8;                                     // level-1 histogram copies (lane l uses l % 8)

// Sources of candidates for the final pass, walked in ascending index order
// as nseg() consecutive segments.  get() returns (key, index); key 0 marks an
// element that is not a candidate.
struct SlotSource {      // per-block ordered slots (multi-block path)
  const uint2* slots;    // [G][kSlotCap] of this row
  const uint32_t* cnt;   // [G]
  int G;
  __device__ int nseg() const { return G; }
  __device__ int seg_len(int w) const { return (int)cnt[w]; }
  __device__ uint2 get(int w, int i) const { return slots[(size_t)w * kSlotCap + i]; }
};

struct RowSource {       // the scores row itself (overflow fallback)
  const float* row;
  int64_t n;
  int64_t seg;           // elements per segment
  int G;
  uint32_t b1;           // level-1 digit filter (0 keeps everything)
  __device__ int nseg() const { return G; }
  __device__ int seg_len(int w) const {
    int64_t lo = (int64_t)w * seg;
    int64_t hi = lo + seg < n ? lo + seg : n;
    return hi > lo ? (int)(hi - lo) : 0;
  }
  __device__ uint2 get(int w, int i) const {
    int64_t s = (int64_t)w * seg + i;
    uint32_t key = order_key(row[s]);
    if ((key >> 20) < b1) key = 0;
    return make_uint2(key, (uint32_t)s);
  }
};

struct FlatSource {      // an ordered candidate array (LDS, row kernel)
  const uint2* a;
  int n;
  int G;                 // segments = threads
  __device__ int nseg() const { return G; }
  __device__ int seg_len(int w) const {
    int per = (n + G - 1) / G;
    int lo = w * per;
    int hi = lo + per < n ? lo + per : n;
    return hi > lo ? hi - lo : 0;
  }
  __device__ uint2 get(int w, int i) const { return a[w * ((n + G - 1) / G) + i]; }
};

// Row t of a launch: its visible keys and, for a batch (row t is token t % T
// of sequence t / T), the first cache row of its sequence.
__device__ __forceinline__ int64_t row_keys(const SeqBatch& sb, int64_t Lk, int T, int t, int64_t* first) {
  int64_t n;
  if (sb.len) {
    n = seq_keys(sb, t / T, first) - T + t % T + 1;
  } else {
    *first = 0;
    n = Lk - T + t + 1;
  }
  return n > 0 ? n : 0;
}

struct FinalShared {
  uint32_t scan[1024 / 64];
  uint32_t h3[kHist3Bins];
  uint32_t bin, above;
};

// Resolve tau from the level-2 histogram (h2, global or shared) and a level-3
// pass over the candidates, then emit the row.  One workgroup, NT threads.
//   all_mode: n <= k, every visible key is kept.
//   k1: keys still to take from the level-1 boundary bin b1.
template <int NT, class Src>
__device__ void final_select(const Src& src, int k, bool all_mode, uint32_t b1, uint32_t k1,
                             const uint32_t* h2, FinalShared& fs, int32_t* out_row) {
  uint32_t tau = 0, r = 0;
  if (!all_mode) {
    find_threshold_bin<NT, kHistBins>(h2, k1, fs.scan, &fs.bin, &fs.above);
    const uint32_t b2 = fs.bin;
    const uint32_t k2 = k1 - fs.above;
    for (int i = threadIdx.x; i < kHist3Bins; i += NT) fs.h3[i] = 0;
    __syncthreads();
    const uint32_t pre = (b1 << 12) | b2;          // key bits 31..8 of the boundary
    const int nseg = src.nseg();
    for (int w = threadIdx.x; w < nseg; w += NT) {
      const int len = src.seg_len(w);
      for (int i = 0; i < len; ++i) {
        const uint32_t key = src.get(w, i).x;
        if ((key >> 8) == pre) atomicAdd(&fs.h3[key & 0xFF], 1u);
      }
    }
    __syncthreads();
    find_threshold_bin<NT, kHist3Bins>(fs.h3, k2, fs.scan, &fs.bin, &fs.above);
    tau = (pre << 8) | fs.bin;
    r = k2 - fs.above;
  }
  // ordered emission: a thread owns a contiguous run of segments
  const int nseg = src.nseg();
  const int spt = (nseg + NT - 1) / NT;
  const int w0 = threadIdx.x * spt;
  const int w1 = w0 + spt < nseg ? w0 + spt : nseg;
  uint32_t n_gt = 0, n_eq = 0;
  for (int w = w0; w < w1; ++w) {
    const int len = src.seg_len(w);
    for (int i = 0; i < len; ++i) {
      const uint32_t key = src.get(w, i).x;
      n_gt += key > tau;
      n_eq += key == tau;
    }
  }
  uint32_t tot_gt, tot_eq;
  const uint32_t gt_base = block_excl_scan<NT>(n_gt, fs.scan, &tot_gt);
  const uint32_t eq_base = block_excl_scan<NT>(n_eq, fs.scan, &tot_eq);
  if (all_mode) r = 0;                       // tau = 0: every candidate is "above"
  uint32_t pos = gt_base + (eq_base < r ? eq_base : r);
  uint32_t eq_seen = eq_base;
  for (int w = w0; w < w1; ++w) {
    const int len = src.seg_len(w);
    for (int i = 0; i < len; ++i) {
      const uint2 e = src.get(w, i);
      bool take = e.x > tau;
      if (e.x == tau) {
        take = eq_seen < r;
        ++eq_seen;
      }
      if (take && pos < (uint32_t)k) out_row[pos++] = (int32_t)e.y;
    }
  }
  const uint32_t total = tot_gt + (tot_eq < r ? tot_eq : r);
  for (uint32_t i = total + threadIdx.x; i < (uint32_t)k; i += NT) out_row[i] = -1;
}

// ------------------------------------------------------------ multi-block path

__global__ __launch_bounds__(256) void topk_hist_kernel(const float* __restrict__ scores, int64_t ld,
                                                        int64_t Lk, int T, TopkCounters ctr) {
  __shared__ uint32_t h[kHistBins];
  __shared__ uint32_t red[4];
  const int t = blockIdx.y;
  const int64_t n = Lk - T + t + 1;
  const int64_t lo = (int64_t)blockIdx.x * kHistRange;
  if (lo >= n) return;                                   // block-uniform
  const int64_t hi = lo + kHistRange < n ? lo + kHistRange : n;
  for (int i = threadIdx.x; i < kHistBins; i += 256) h[i] = 0;
  __syncthreads();
  const float* row = scores + (int64_t)t * ld;
  for (int64_t s = lo + threadIdx.x; s < hi; s += 256) atomicAdd(&h[order_key(row[s]) >> 20], 1u);
  __syncthreads();
  flush_level1<256>(ctr, blockIdx.x % kHistReplicas, t, h, red);
}

// Level-1 threshold digit: the largest bin whose suffix count reaches `need`,
// searched downward from the highest non-empty bin in chunks of NT bins (one
// chunk almost always suffices).
template <int NT>
__device__ void find_b1(const TopkCounters& ctr, int t, uint32_t need, uint32_t* scan_sm, uint32_t* s_bin,
                        uint32_t* s_above) {
  uint32_t mb = 0;
#pragma unroll
  for (int r = 0; r < kHistReplicas; ++r) {
    const uint32_t v = ctr.maxbin[r * kMaxCounterRows + t];
    mb = v > mb ? v : mb;
  }
  uint32_t acc = 0;
  for (int c0 = (int)mb - 1; c0 >= 0; c0 -= NT) {
    const int bin = c0 - (int)threadIdx.x;
    uint32_t hv[kHistReplicas];
#pragma unroll
    for (int r = 0; r < kHistReplicas; ++r) hv[r] = bin >= 0 ? h1_row(ctr, r, t)[bin] : 0u;
    uint32_t h = 0;
#pragma unroll
    for (int r = 0; r < kHistReplicas; ++r) h += hv[r];
    uint32_t tot;
    const uint32_t excl = block_excl_scan<NT>(h, scan_sm, &tot);
    if (acc + excl < need && acc + excl + h >= need) {
      *s_bin = (uint32_t)bin;
      *s_above = acc + excl;
    }
    acc += tot;
    if (acc >= need) break;                                            // uniform
  }
  __syncthreads();
}

// Each block compacts, in index order, the keys of its range whose level-1
// digit reaches the threshold digit into its own slot, and adds the level-2
// digits of the boundary bin to the row's level-2 histogram.  Element e of
// thread j is key lo + 256 e + j (coalesced loads); the index order is (e, j),
// so the compaction offsets come from per-wave ballots and one 64-entry scan.
__global__ __launch_bounds__(256) void topk_collect_kernel(
    const float* __restrict__ scores, int64_t ld, int64_t Lk, int T, int k, TopkCounters ctr,
    uint2* __restrict__ slots, uint32_t* __restrict__ slot_cnt, uint32_t* __restrict__ rowinfo, int G,
    SeqBatch sb) {
  __shared__ uint32_t h2[kHistBins];
  __shared__ uint32_t scan_sm[4];
  __shared__ uint32_t wcnt[kCollectPer * 4];
  __shared__ uint32_t s_b1, s_above1;
  const int t = blockIdx.y;
  const int wg = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int64_t first;
  const int64_t n = row_keys(sb, Lk, T, t, &first);
  const bool all_mode = n <= (int64_t)k;
  if (all_mode) return;                                  // the final kernel keeps every visible key
  const float* row = scores + (int64_t)t * ld;
  const int64_t lo = (int64_t)wg * kCollectRange + threadIdx.x;

  float v[kCollectPer];
#pragma unroll
  for (int e = 0; e < kCollectPer; ++e) v[e] = (lo + 256 * e < n) ? row[lo + 256 * e] : 0.0f;
  for (int i = threadIdx.x; i < kHistBins; i += 256) h2[i] = 0;

  uint32_t b1 = 0;
  if (!all_mode) {
    find_b1<256>(ctr, t, (uint32_t)k, scan_sm, &s_b1, &s_above1);
    b1 = s_b1;
    if (wg == 0 && threadIdx.x == 0) {
      rowinfo[2 * t] = s_b1;
      rowinfo[2 * t + 1] = s_above1;
    }
  } else {
    __syncthreads();
  }

  uint32_t key[kCollectPer];
  uint64_t mask[kCollectPer];
#pragma unroll
  for (int e = 0; e < kCollectPer; ++e) {
    key[e] = order_key(v[e]);
    const bool f = (lo + 256 * e < n) && (key[e] >> 20) >= b1;
    mask[e] = __ballot(f);
    if (f && !all_mode && (key[e] >> 20) == b1) atomicAdd(&h2[(key[e] >> 8) & 0xFFF], 1u);
    if (lane == 0) wcnt[e * 4 + wave] = (uint32_t)__popcll(mask[e]);
  }
  __syncthreads();
  // exclusive prefix of the 64 (e, wave) counts, in index order
  __shared__ uint32_t wpre[kCollectPer * 4 + 1];
  if (wave == 0) {
    const uint32_t c = wcnt[lane];
    uint32_t x = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    wpre[lane] = x - c;
    if (lane == 63) wpre[64] = x;
  }
  __syncthreads();
  const uint32_t total = wpre[64];
  uint2* my_slots = slots + ((size_t)t * G + wg) * kSlotCap;
#pragma unroll
  for (int e = 0; e < kCollectPer; ++e) {
    if ((mask[e] >> lane) & 1ull) {
      const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask[e] >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)mask[e], 0u));
      const uint32_t pos = wpre[e * 4 + wave] + below;
      if (pos < kSlotCap) my_slots[pos] = make_uint2(key[e], (uint32_t)(lo + 256 * e));
    }
  }
  if (threadIdx.x == 0) {
    slot_cnt[(size_t)t * G + wg] = total < kSlotCap ? total : kSlotCap;
    if (total > kSlotCap) atomicOr(&ctr.overflow[t], 1u);
  }
  if (!all_mode) {
    uint32_t* g2 = ctr.h2 + (size_t)t * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += 256) {
      const uint32_t c = h2[i];
      if (c) atomicAdd(&g2[i], c);
    }
  }
}

constexpr int kFinalThreads = 1024;
static_assert(kMaxSegs <= kFinalThreads, "one slot per thread");

struct FinalKernelShared {
  uint2 cand[kCandCap];
  FinalShared fs;
};

// Grid (T, 1 + kHistReplicas).  Block (t, 0) gathers the ordered candidates of
// all slots of row t into LDS, resolves the exact threshold and emits the row;
// blocks (t, 1 + r) clear level-1 replica r of the row for the next call.
__global__ __launch_bounds__(kFinalThreads) void topk_final_kernel(
    const float* __restrict__ scores, int64_t ld, int64_t Lk, int T, int k, TopkCounters ctr,
    const uint2* __restrict__ slots, const uint32_t* __restrict__ slot_cnt, const uint32_t* __restrict__ rowinfo,
    int G, int32_t* __restrict__ idx, SeqBatch sb, int32_t* __restrict__ idx_rows) {
  __shared__ FinalKernelShared sh;
  const int t = blockIdx.x;
  if (blockIdx.y > 0) {
    const int r = blockIdx.y - 1;
    uint4* z = reinterpret_cast<uint4*>(h1_row(ctr, r, t));
    for (int i = threadIdx.x; i < kHistBins / 4; i += kFinalThreads) z[i] = make_uint4(0, 0, 0, 0);
    if (threadIdx.x == 0) ctr.maxbin[r * kMaxCounterRows + t] = 0;
    return;
  }
  int64_t first;
  const int64_t n = row_keys(sb, Lk, T, t, &first);
  const bool all_mode = n <= (int64_t)k;
  const float* row = scores + (int64_t)t * ld;
  int32_t* out_row = idx + (size_t)t * k;
  if (all_mode) {
    // every visible key is kept (the collect kernel skipped the row)
    for (int j = threadIdx.x; j < k; j += kFinalThreads) {
      out_row[j] = j < n ? j : -1;
      if (idx_rows) idx_rows[(size_t)t * k + j] = j < n ? (int32_t)(first + j) : -1;
    }
    uint4* z2 = reinterpret_cast<uint4*>(ctr.h2 + (size_t)t * kHistBins);
    for (int i = threadIdx.x; i < kHistBins / 4; i += kFinalThreads) z2[i] = make_uint4(0, 0, 0, 0);
    if (threadIdx.x == 0) ctr.overflow[t] = 0;
    return;
  }
  // every independent load first
  const uint32_t ovf = ctr.overflow[t];
  const uint32_t b1 = all_mode ? 0u : rowinfo[2 * t];
  const uint32_t above1 = all_mode ? 0u : rowinfo[2 * t + 1];
  const int j = threadIdx.x;
  const uint32_t c_own = j < G ? slot_cnt[(size_t)t * G + j] : 0u;
  const uint32_t* g2 = ctr.h2 + (size_t)t * kHistBins;

  uint32_t M;
  const uint32_t base = block_excl_scan<kFinalThreads>(c_own, sh.fs.scan, &M);
  if (!ovf && M <= (uint32_t)kCandCap) {
    // thread j copies slot j, eight independent loads at a time
    const uint2* sp = slots + ((size_t)t * G + (j < G ? j : 0)) * kSlotCap;
    for (uint32_t i0 = 0; i0 < c_own; i0 += 8) {
      uint2 buf[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) buf[i] = i0 + i < c_own ? sp[i0 + i] : make_uint2(0u, 0u);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i0 + i < c_own) sh.cand[base + i0 + i] = buf[i];
    }
    __syncthreads();
    FlatSource src{sh.cand, (int)M, kFinalThreads};
    final_select<kFinalThreads>(src, k, all_mode, b1, (uint32_t)k - above1, g2, sh.fs, out_row);
  } else {
    RowSource src{row, n, kCollectRange, G, b1};
    final_select<kFinalThreads>(src, k, all_mode, b1, (uint32_t)k - above1, g2, sh.fs, out_row);
  }
  __syncthreads();
  uint4* z2 = reinterpret_cast<uint4*>(ctr.h2 + (size_t)t * kHistBins);
  for (int i = threadIdx.x; i < kHistBins / 4; i += kFinalThreads) z2[i] = make_uint4(0, 0, 0, 0);
  if (threadIdx.x == 0) ctr.overflow[t] = 0;
  if (idx_rows) {
    // the same set as cache rows of the sequence
    for (int j = threadIdx.x; j < k; j += kFinalThreads) {
      const int32_t v = out_row[j];
      idx_rows[(size_t)t * k + j] = v >= 0 ? (int32_t)(first + v) : -1;
    }
  }
}

// ------------------------------------------------------------ row path

// Per row: the level-1 histogram of the order keys (in kRowReps copies:
// scores of one row fall into few level-1 bins, and LDS atomics on one
// address serialise; lane l counts into copy l % kRowReps, the copies' rows
// padded so that copies of one bin sit in different banks), its threshold
// bin b1, then every key at or above the bin is a candidate: each wave
// appends its candidates to a region of its own (positions from its ballots,
// no atomics), unused slots hold key 0.  The
// exact top k of the candidates is resolved and emitted in index order by
// select_sorted.  A row whose candidates overflow the LDS slots takes the
// ordered full-row path of final_select instead (same result, slower).
constexpr int kRepStride = kHistBins + 4;
constexpr int kRowWaves = kRowThreads / 64;
constexpr int kWaveCap = kRowCap / kRowWaves;                   // candidate slots per wave

// The smallest float whose order key is at least K: the candidate tests of
// the row kernel compare the scores themselves.  Keys at or below that of
// -inf map to -inf, keys above that of +inf to +inf.
__device__ __forceinline__ float key_floor(uint32_t K) {
  if (K <= 0x007FFFFFu) return -INFINITY;
  if (K >= 0xFF800000u) return INFINITY;
  return __uint_as_float((K & 0x80000000u) ? (K & 0x7FFFFFFFu) : ~K);
}

struct RowCand {
  uint32_t key[kRowCap];
  uint32_t idx[kRowCap];
};

constexpr int kSmallRow = 16384;                   // rows up to this many keys stay in LDS
static_assert(kSmallRow % kRowThreads == 0 && kSmallRow / 32 <= DSA_TOPK_MAX, "short-row layout");

// The top-k of a short row (k < n <= kSmallRow): its order keys are read once
// into K (LDS) and the three-digit radix descent runs there (ties: a descent
// over the complemented indices); the kept set leaves in index order through
// the bitmap bm (n / 32 words).  All NT threads call it; scan_sm holds NT / 64
// words.
template <int NT>
__device__ void short_row_select(const float* __restrict__ row, int n, int k, uint32_t* K, RadixShared& rs,
                                 uint32_t* bm, uint32_t* scan_sm, int32_t* out_row) {
  constexpr int kS = kSmallRow / NT;
  float v[kS];
#pragma unroll
  for (int e = 0; e < kS; ++e) {
    if (e % 8 == 0 && e * NT >= n) break;
    const int s = e * NT + (int)threadIdx.x;
    v[e] = row[s < n ? s : n - 1];
  }
#pragma unroll
  for (int e = 0; e < kS; ++e) {
    if (e % 8 == 0 && e * NT >= n) break;
    const int s = e * NT + (int)threadIdx.x;
    if (s < n) K[s] = order_key(v[e]);
  }
  __syncthreads();
  uint32_t tau, r, eq;
  radix_threshold<NT>([&](int i) { return K[i]; }, n, (uint32_t)k, rs, &tau, &r, &eq);
  uint32_t imax = 0xFFFFFFFFu;
  if (eq > r) {                                        // block-uniform
    uint32_t tau2, r2, eq2;
    radix_threshold<NT>([&](int i) { return K[i] == tau ? ~(uint32_t)i : 0u; }, n, r, rs, &tau2, &r2, &eq2);
    imax = ~tau2;
  }
  const int nw = (n + 31) / 32;
  for (int i = threadIdx.x; i < nw; i += NT) bm[i] = 0u;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += NT) {
    const uint32_t key = K[i];
    if (key > tau || (key == tau && (uint32_t)i <= imax)) atomicOr(&bm[i >> 5], 1u << (i & 31));
  }
  __syncthreads();
  bitmap_emit<NT>(bm, nw, scan_sm, k, out_row);
}

// Rows of kSmallRow < n <= kRegRow keys: each thread keeps its kRegPer keys
// (elements e * NT + thread) in registers, so the row is read once and every
// pass after it runs on registers and LDS.
//   1. a lower bound L0 of the threshold: with c = ceil(k / NT), every thread
//      holds c keys at or above its own c-th largest, so the smallest of those
//      c-th largest keys has at least c * NT >= k keys at or above it;
//   2. a histogram of the keys >= L0 over [L0, max] in 4,096 bins (the range
//      adapts to the row, so the keys spread over the bins instead of piling
//      into the few that a fixed digit gives them), and the bin b1 that holds
//      the k-th key;
//   3. when b1 holds few keys, they are collected and ranked directly by (key
//      desc, index asc): the k-th key (tk, ti) of the row is the one of rank
//      k - (keys above the bin) - 1;
//   4. the kept keys (key > tk, or key == tk and index <= ti) are marked in a
//      bitmap by wave ballots and emitted in index order.
// A crowded threshold bin (ties, narrow rows) returns false without output;
// the caller then takes the general path.
constexpr int kRegPer = 64;
constexpr int kRegRow = kRegPer * kRowThreads;
constexpr int kBinCap = 256;                       // threshold-bin keys ranked directly
static_assert(kSmallRow >= 2 * kRowThreads && DSA_TOPK_MAX <= 2 * kRowThreads, "threshold bound of step 1");

struct RegRowShared {
  uint32_t hist[kHistBins];
  uint64_t bm[kRegRow / 64];                       // kept-key bitmap, bit s % 64 of word s / 64
  alignas(16) uint32_t ck[kBinCap];                // keys of the threshold bin
  alignas(16) uint32_t ci[kBinCap];                // and their indices
  uint32_t red[4 * kRowWaves];
  uint32_t bscan[kRowWaves], bout[3];
  uint32_t escan[kRowWaves];
  uint32_t n1, tk, ti;
};

template <int NT>
__device__ bool reg_row_select(const float* __restrict__ row, int n, int k, RegRowShared& g,
                               int32_t* __restrict__ out_row) {
  constexpr int E = kRegPer;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // ---- the keys: every load in flight at once (positions past the row read
  // its last score and are masked to key 0, which no score maps to)
  uint32_t key[E];
  {
    float v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int s = e * NT + tid;
      v[e] = row[s < n ? s : n - 1];
    }
#pragma unroll
    for (int e = 0; e < E; ++e) key[e] = e * NT + tid < n ? order_key(v[e]) : 0u;
  }
  // ---- 1. the largest key, and each thread's c-th largest (c <= 2)
  const int c = (k + NT - 1) / NT;
  uint32_t m1 = 0u, m2 = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t lo = m1 < key[e] ? m1 : key[e];
    m1 = m1 > key[e] ? m1 : key[e];
    m2 = m2 > lo ? m2 : lo;
  }
  const int cnt = tid < n ? (n - 1 - tid) / NT + 1 : 0;      // this thread's keys
  uint32_t kmax = m1, L0 = cnt >= c ? (c == 1 ? m1 : m2) : 0xFFFFFFFFu, unused = 0xFFFFFFFFu;
  uint32_t nc = cnt >= c ? 1u : 0u;
  for (int i = tid; i < kHistBins; i += NT) g.hist[i] = 0u;
  if (tid == 0) g.n1 = 0u;
  block_reduce_mmms<NT>(kmax, L0, unused, nc, g.red);
  if ((uint64_t)nc * (uint32_t)c < (uint64_t)k) L0 = 1u;     // not reached for n > kSmallRow; every key counts
  // ---- 2. histogram of the keys >= L0 over [L0, kmax]
  const uint32_t span = kmax - L0;
  const int bits = span ? 32 - __builtin_clz(span) : 0;
  const int s1 = bits > 12 ? bits - 12 : 0;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (key[e] >= L0) atomicAdd(&g.hist[(key[e] - L0) >> s1], 1u);
  __syncthreads();
  uint32_t b1, above1, cnt1;
  find_threshold_bin_once<NT, kHistBins>(g.hist, (uint32_t)k, g.bscan, g.bout, &b1, &above1, &cnt1);
  if (cnt1 > (uint32_t)kBinCap) {                  // block-uniform
    __syncthreads();                               // the caller reuses this memory
    return false;
  }
  const uint32_t need = (uint32_t)k - above1;     // 1 <= need <= cnt1
  const uint32_t lo = L0 + (b1 << s1);
  const uint32_t wid = (1u << s1) - 1u;
  const uint32_t hi = lo > 0xFFFFFFFFu - wid ? 0xFFFFFFFFu : lo + wid;
  // ---- 3. collect the bin's keys (padded to 16 with key 0, which ranks last) and rank them
#pragma unroll
  for (int e = 0; e < E; ++e)
    if ((key[e] >= lo) & (key[e] <= hi)) {
      const uint32_t p = atomicAdd(&g.n1, 1u);
      g.ck[p] = key[e];
      g.ci[p] = (uint32_t)(e * NT + tid);
    }
  const uint32_t ncp = (cnt1 + 15u) & ~15u;
  if ((uint32_t)tid >= cnt1 && (uint32_t)tid < ncp) {
    g.ck[tid] = 0u;
    g.ci[tid] = 0xFFFFFFFFu;
  }
  __syncthreads();
  if ((uint32_t)tid < cnt1) {
    const uint32_t kt = g.ck[tid], it = g.ci[tid];
    auto before = [&](uint32_t kj, uint32_t ij) {
      return (uint32_t)(kj > kt) | ((uint32_t)(kj == kt) & (uint32_t)(ij < it));
    };
    uint32_t rank = 0;
    for (uint32_t j0 = 0; j0 < ncp; j0 += 16) {
      uint4 k4[4], i4[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        k4[q] = *reinterpret_cast<const uint4*>(&g.ck[j0 + 4 * q]);
        i4[q] = *reinterpret_cast<const uint4*>(&g.ci[j0 + 4 * q]);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        rank += before(k4[q].x, i4[q].x) + before(k4[q].y, i4[q].y) + before(k4[q].z, i4[q].z) +
                before(k4[q].w, i4[q].w);
    }
    if (rank == need - 1u) {
      g.tk = kt;
      g.ti = it;
    }
  }
  __syncthreads();
  const uint32_t tk = g.tk, ti = g.ti;
  // ---- 4. bitmap of the kept keys: the ballot of element e covers keys
  // e * NT + 64 * wave .. + 63, one 64-bit word; lane e keeps it and every
  // lane stores one word
  uint64_t mine = 0ull;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t s = (uint32_t)(e * NT + tid);
    const uint64_t m = __ballot((key[e] > tk) | ((key[e] == tk) & (s <= ti)));
    mine = lane == e ? m : mine;
  }
  g.bm[lane * (NT / 64) + wv] = mine;
  __syncthreads();
  bitmap_emit<NT>(reinterpret_cast<const uint32_t*>(g.bm), (n + 31) / 32, g.escan, k, out_row);
  return true;
}

union RowShared {
  uint32_t rep[kRowReps * kRepStride];
  static_assert(kRowReps * kRepStride >= kSmallRow, "a short row's keys fit the level-1 copies' space");
  RowCand c;
  RegRowShared g;
};

struct RowSel {
  RadixShared rs;
  uint32_t sel[DSA_TOPK_MAX];
  uint32_t nsel, count;
  uint32_t wcount[kRowWaves];
};

// The top-k of one scores row of n visible keys into out_row[0 .. k), by the
// kRowThreads threads of a workgroup (the shared structures are the caller's).
// kRegRows: rows of up to kRegRow keys take the register-resident selection
// (a kernel whose other work needs the registers leaves it out).
template <bool kRegRows>
__device__ __forceinline__ void row_topk(const float* __restrict__ row, int64_t n, int k, int32_t* __restrict__ out_row,
                         RowShared& rsh, RowSel& sh, FinalShared& fs) {
  const int lane = threadIdx.x & 63;

  if (n <= (int64_t)k) {
    // every visible key is kept
    for (int j = threadIdx.x; j < k; j += kRowThreads) out_row[j] = j < n ? j : -1;
  } else if (n <= (int64_t)kSmallRow) {
    short_row_select<kRowThreads>(row, (int)n, k, rsh.rep, sh.rs, sh.sel, fs.scan, out_row);
  } else if (kRegRows && n <= (int64_t)kRegRow && reg_row_select<kRowThreads>(row, (int)n, k, rsh.g, out_row)) {
    // done
  } else {
    // ---- level-1 histogram
    static_assert((kRowReps * kRepStride) % 4 == 0, "16-byte clears");
    for (int i = threadIdx.x; i < kRowReps * kRepStride / 4; i += kRowThreads)
      reinterpret_cast<uint4*>(rsh.rep)[i] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    uint32_t* hrep = rsh.rep + (lane % kRowReps) * kRepStride;
    // Rounds of kH scores per thread (score base + e * kRowThreads + thread),
    // all loads issued first; groups of 8 that start past the row are skipped
    // (the test is uniform over the workgroup).
    constexpr int kH = 32;
    for (int64_t base = 0; base < n; base += (int64_t)kH * kRowThreads) {
      float v[kH];
#pragma unroll
      for (int e = 0; e < kH; ++e) {
        if (e % 8 == 0 && base + (int64_t)e * kRowThreads >= n) break;
        const int64_t s = base + (int64_t)e * kRowThreads + threadIdx.x;
        v[e] = row[s < n ? s : n - 1];
      }
#pragma unroll
      for (int e = 0; e < kH; ++e) {
        if (e % 8 == 0 && base + (int64_t)e * kRowThreads >= n) break;
        if (base + (int64_t)e * kRowThreads + threadIdx.x < n) atomicAdd(&hrep[order_key(v[e]) >> 20], 1u);
      }
    }
    __syncthreads();
    for (int i = 4 * threadIdx.x; i < kHistBins; i += 4 * kRowThreads) {
      uint4 sum = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int r = 0; r < kRowReps; ++r) {
        const uint4 q = *reinterpret_cast<const uint4*>(&rsh.rep[r * kRepStride + i]);
        sum.x += q.x;
        sum.y += q.y;
        sum.z += q.z;
        sum.w += q.w;
      }
      *reinterpret_cast<uint4*>(&sh.rs.hist[i]) = sum;
    }
    __syncthreads();
    find_threshold_bin<kRowThreads, kHistBins>(sh.rs.hist, (uint32_t)k, fs.scan, &sh.rs.bin, &sh.rs.above);
    const uint32_t b1 = sh.rs.bin, above1 = sh.rs.above;
    // ---- candidates: keys whose level-1 digit is >= b1 (the copies are
    // dead); the level-2 digits of the boundary bin's keys go to h2, which
    // lies past the candidate slots
    uint32_t* h2 = rsh.rep + 2 * kRowCap;
    for (int i = threadIdx.x; i < kHistBins; i += kRowThreads) h2[i] = 0;
    __syncthreads();
    const uint64_t below = (1ull << lane) - 1ull;
    const int wv = threadIdx.x >> 6;
    uint32_t* wkey = rsh.c.key + wv * kWaveCap;
    uint32_t* widx = rsh.c.idx + wv * kWaveCap;
    uint32_t wcnt = 0;                                 // wave-uniform
    const float flo = key_floor(b1 << 20);             // level-1 digit >= b1 <=> score >= flo
    const float fhi = b1 == 0xFFFu ? INFINITY : key_floor((b1 + 1u) << 20);   // +inf: test the digit
    for (int64_t base = 0; base < n; base += (int64_t)kH * kRowThreads) {
      float v[kH];
#pragma unroll
      for (int e = 0; e < kH; ++e) {
        if (e % 8 == 0 && base + (int64_t)e * kRowThreads >= n) break;
        const int64_t s = base + (int64_t)e * kRowThreads + threadIdx.x;
        v[e] = row[s < n ? s : n - 1];
      }
#pragma unroll
      for (int e = 0; e < kH; ++e) {
        if (e % 8 == 0 && base + (int64_t)e * kRowThreads >= n) break;
        const int64_t s = base + (int64_t)e * kRowThreads + threadIdx.x;
        const bool f = s < n && v[e] >= flo;
        const uint64_t m = __ballot(f);
        if (f) {
          const uint32_t key = order_key(v[e]);
          if (fhi == INFINITY ? (key >> 20) == b1 : v[e] < fhi) atomicAdd(&h2[(key >> 8) & 0xFFF], 1u);
          const uint32_t pos = wcnt + (uint32_t)__popcll(m & below);
          if (pos < (uint32_t)kWaveCap) {
            wkey[pos] = key;
            widx[pos] = (uint32_t)s;
          }
        }
        wcnt += (uint32_t)__popcll(m);
      }
    }
    for (uint32_t i = wcnt + lane; i < (uint32_t)kWaveCap; i += 64) wkey[i] = 0u;   // unused slots
    if (lane == 0) sh.wcount[wv] = wcnt;
    __syncthreads();
    bool fits = true;
#pragma unroll
    for (int w = 0; w < kRowWaves; ++w) fits &= sh.wcount[w] <= (uint32_t)kWaveCap;
    const uint32_t count = kRowCap;                    // slots, the unused ones with key 0
    if (fits) {
      // threshold key tau: level 2 from h2, level 3 over the candidates
      const uint32_t* ck = rsh.c.key;
      const uint32_t* ci = rsh.c.idx;
      find_threshold_bin<kRowThreads, kHistBins>(h2, (uint32_t)k - above1, fs.scan, &fs.bin, &fs.above);
      const uint32_t b2 = fs.bin;
      const uint32_t k2 = (uint32_t)k - above1 - fs.above;
      for (int i = threadIdx.x; i < kHist3Bins; i += kRowThreads) fs.h3[i] = 0;
      __syncthreads();
      const uint32_t pre = (b1 << 12) | b2;           // key bits 31..8 of the boundary
      for (uint32_t i = threadIdx.x; i < count; i += kRowThreads)
        if (ck[i] && (ck[i] >> 8) == pre) atomicAdd(&fs.h3[ck[i] & 0xFF], 1u);
      __syncthreads();
      find_threshold_bin<kRowThreads, kHist3Bins>(fs.h3, k2, fs.scan, &fs.bin, &fs.above);
      const uint32_t tau = (pre << 8) | fs.bin;
      const uint32_t r = k2 - fs.above;                // tau-equal keys to keep: the r lowest indices
      const uint32_t eq = fs.h3[fs.bin];
      uint32_t imax = 0xFFFFFFFFu;
      if (eq > r) {                                    // block-uniform
        uint32_t tau2, r2, eq2;
        radix_threshold<kRowThreads>([&](int i) { return ck[i] == tau ? ~ci[i] : 0u; }, (int)count, r, sh.rs,
                                     &tau2, &r2, &eq2);
        imax = ~tau2;
      }
      // the kept set in index order: a bitmap over the row when it fits in
      // sel, else the sort
      const int nw = (int)((n + 31) / 32);
      if (nw <= DSA_TOPK_MAX) {
        for (int i = threadIdx.x; i < nw; i += kRowThreads) sh.sel[i] = 0u;
        __syncthreads();
        for (uint32_t i = threadIdx.x; i < count; i += kRowThreads) {
          const uint32_t key = ck[i], id = ci[i];
          if (key > tau || (key == tau && id <= imax)) atomicOr(&sh.sel[id >> 5], 1u << (id & 31));
        }
        __syncthreads();
        bitmap_emit<kRowThreads>(sh.sel, nw, fs.scan, k, out_row);
      } else {
        if (threadIdx.x == 0) sh.nsel = 0;
        __syncthreads();
        for (uint32_t i = threadIdx.x; i < count; i += kRowThreads) {
          const uint32_t key = ck[i], id = ci[i];
          if (key > tau || (key == tau && id <= imax)) sh.sel[atomicAdd(&sh.nsel, 1u)] = id;
        }
        __syncthreads();
        sort_emit<kRowThreads>(sh.sel, (uint32_t)k, k, out_row);
      }
    } else {
      // overflow: the ordered pass over the row
      const int64_t seg = (n + kRowThreads - 1) / kRowThreads;
      RowSource src{row, n, seg, kRowThreads, b1};
      final_select<kRowThreads>(src, k, false, b1, (uint32_t)k - above1, h2, fs, out_row);
    }
  }
}

__global__ __launch_bounds__(kRowThreads) void topk_row_kernel(const float* __restrict__ scores, int64_t ld,
                                                               int64_t Lk, int T, int k,
                                                               int32_t* __restrict__ idx, SeqBatch sb,
                                                               int32_t* __restrict__ idx_rows) {
  __shared__ __attribute__((aligned(16))) RowShared rsh;
  __shared__ __attribute__((aligned(16))) RowSel sh;
  __shared__ FinalShared fs;
  const int t = blockIdx.x;
  int64_t first = 0;
  if (sb.len) Lk = seq_keys(sb, t / T, &first);        // batch: row t is token t % T of sequence t / T
  const int tt = sb.len ? t % T : t;
  int64_t n = Lk - T + tt + 1;
  n = n > 0 ? n : 0;
  int32_t* out_row = idx + (size_t)t * k;
  row_topk<true>(scores + (int64_t)t * ld, n, k, out_row, rsh, sh, fs);
  if (idx_rows) {
    // the same set as cache rows of the sequence
    __syncthreads();
    for (int j = threadIdx.x; j < k; j += kRowThreads) {
      const int32_t v = out_row[j];
      idx_rows[(size_t)t * k + j] = v >= 0 ? (int32_t)(first + v) : -1;
    }
  }
}

// The exact fallback of the fused prefill top-k: each workgroup takes the
// listed rows blockIdx.x, blockIdx.x + gridDim.x, ... below *nfail, scores the
// row's visible keys with the exact index arithmetic into its own buffer row
// (buf + blockIdx.x * ld) and selects the row's top-k from it.  A launch with
// no listed row ends at once.
__global__ __launch_bounds__(kRowThreads) void prefill_fallback_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ w, const uint8_t* __restrict__ k_idx, int64_t Lk,
    int T, int k, const uint32_t* __restrict__ nfail, const uint32_t* __restrict__ failed, float* __restrict__ buf,
    int64_t ld, int32_t* __restrict__ idx) {
  __shared__ __attribute__((aligned(16))) RowShared rsh;
  __shared__ __attribute__((aligned(16))) RowSel sh;
  __shared__ FinalShared fs;
  uint32_t nf = *nfail;
  nf = nf < (uint32_t)T ? nf : (uint32_t)T;
  float* row = buf + (int64_t)blockIdx.x * ld;
  for (uint32_t i = blockIdx.x; i < nf; i += gridDim.x) {
    const uint32_t t = failed[i];
    if (t >= (uint32_t)T) continue;                    // block-uniform; never written so by the refine kernel
    const int64_t n = Lk - T + (int64_t)t + 1;
    exact_scores_block<kRowThreads, 4>(q_idx + (size_t)t * 16 * 128, w + (size_t)t * 16, k_idx, n, row);
    __syncthreads();
    row_topk<false>(row, n, k, idx + (size_t)t * k, rsh, sh, fs);
    __syncthreads();
  }
}

// Few long rows take the multi-block path: enough blocks that a row's
// candidates (about k plus the boundary bin) spread well within the blocks'
// slots; shorter rows are served by one workgroup each.
bool multi_block(int64_t Lk, int T, int k) {
  const int64_t G = cdiv(Lk, kCollectRange);
  return T <= kTopkMultiRowsMax && G <= kMaxSegs && G * kSlotCap >= (int64_t)4 * k;
}

}  // namespace


size_t topk_scratch_bytes(int64_t Lk, int T, int k) {
  if (!multi_block(Lk, T, k)) return 256;
  const int64_t G = cdiv(Lk, kCollectRange);
  return (size_t)T * G * kSlotCap * sizeof(uint2) + (size_t)T * G * sizeof(uint32_t) + (size_t)T * 8 + 256;
}

hipError_t launch_topk(const float* scores, int64_t ld, int64_t Lk, int T, int k, int32_t* idx,
                       void* ws_counters, void* scratch, hipStream_t st, bool hist_ready) {
  if (!multi_block(Lk, T, k)) {
    hipLaunchKernelGGL(topk_row_kernel, dim3(T), dim3(kRowThreads), 0, st, scores, ld, Lk, T, k, idx, SeqBatch{},
                       (int32_t*)nullptr);
    return hipGetLastError();
  }
  TopkCounters ctr = counters_at(ws_counters);
  const int64_t G = cdiv(Lk, kCollectRange);
  uint2* slots = reinterpret_cast<uint2*>(scratch);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(slots + (size_t)T * G * kSlotCap);
  uint32_t* rowinfo = cnt + (size_t)T * G;
  hipError_t e;
  if (!hist_ready) {
    const int64_t Gh = cdiv(Lk, kHistRange);
    hipLaunchKernelGGL(topk_hist_kernel, dim3((unsigned)Gh, T), dim3(256), 0, st, scores, ld, Lk, T, ctr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(topk_collect_kernel, dim3((unsigned)G, T), dim3(256), 0, st, scores, ld, Lk, T, k, ctr,
                     slots, cnt, rowinfo, (int)G, SeqBatch{});
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_final_kernel, dim3(T, 1 + kHistReplicas), dim3(kFinalThreads), 0, st, scores, ld, Lk, T,
                     k, ctr, (const uint2*)slots, (const uint32_t*)cnt, (const uint32_t*)rowinfo, (int)G, idx,
                     SeqBatch{}, (int32_t*)nullptr);
  return hipGetLastError();
}

bool topk_multi_block(int64_t Lk, int T, int k) { return multi_block(Lk, T, k); }

hipError_t launch_prefill_fallback(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t Lk, int T,
                                   int k, const uint32_t* nfail, const uint32_t* failed, float* buf, int64_t ld,
                                   int blocks, int32_t* idx, hipStream_t st) {
  if (blocks < 1 || ld < Lk || k < 1 || k > DSA_TOPK_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prefill_fallback_kernel, dim3((unsigned)blocks), dim3(kRowThreads), 0, st, q_idx, w, k_idx, Lk,
                     T, k, nfail, failed, buf, ld, idx);
  return hipGetLastError();
}

hipError_t launch_topk_batch(const float* scores, int64_t ld, const SeqBatch& sb, int B, int T, int k, int32_t* idx,
                             int32_t* idx_rows, hipStream_t st) {
  const int64_t rows = (int64_t)B * T;
  if (rows < 1 || rows > 0x7FFFFFFF || !sb.len) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_row_kernel, dim3((unsigned)rows), dim3(kRowThreads), 0, st, scores, ld, sb.max_len, T, k,
                     idx, sb, idx_rows);
  return hipGetLastError();
}

}  // namespace dsa
