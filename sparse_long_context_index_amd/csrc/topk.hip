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
//  * Many rows (prefill): topk_row_kernel, one 1024-thread workgroup per row,
//    candidates in LDS.
// A candidate slot that overflows switches the row's final pass to reading
// the scores row itself (same result, slower).
#include "dsa_common.hpp"
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
    uint2* __restrict__ slots, uint32_t* __restrict__ slot_cnt, uint32_t* __restrict__ rowinfo, int G) {
  __shared__ uint32_t h2[kHistBins];
  __shared__ uint32_t scan_sm[4];
  __shared__ uint32_t wcnt[kCollectPer * 4];
  __shared__ uint32_t s_b1, s_above1;
  const int t = blockIdx.y;
  const int wg = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t n = Lk - T + t + 1;
  const bool all_mode = n <= (int64_t)k;
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
    int G, int32_t* __restrict__ idx) {
  __shared__ FinalKernelShared sh;
  const int t = blockIdx.x;
  if (blockIdx.y > 0) {
    const int r = blockIdx.y - 1;
    uint4* z = reinterpret_cast<uint4*>(h1_row(ctr, r, t));
    for (int i = threadIdx.x; i < kHistBins / 4; i += kFinalThreads) z[i] = make_uint4(0, 0, 0, 0);
    if (threadIdx.x == 0) ctr.maxbin[r * kMaxCounterRows + t] = 0;
    return;
  }
  const int64_t n = Lk - T + t + 1;
  const bool all_mode = n <= (int64_t)k;
  const float* row = scores + (int64_t)t * ld;
  int32_t* out_row = idx + (size_t)t * k;
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
}

// ------------------------------------------------------------ row path

__global__ __launch_bounds__(kRowThreads) void topk_row_kernel(const float* __restrict__ scores, int64_t ld,
                                                               int64_t Lk, int T, int k,
                                                               int32_t* __restrict__ idx, SeqBatch sb,
                                                               int32_t* __restrict__ idx_rows) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[kHistBins];
  __shared__ uint2 cand[kRowCap];
  __shared__ FinalShared fs;
  __shared__ uint32_t s_b1, s_above1;
  const int t = blockIdx.x;
  int64_t first = 0;
  if (sb.len) Lk = seq_keys(sb, t / T, &first);        // batch: row t is token t % T of sequence t / T
  const int tt = sb.len ? t % T : t;
  int64_t n = Lk - T + tt + 1;
  n = n > 0 ? n : 0;
  const bool all_mode = n <= (int64_t)k;
  const float* row = scores + (int64_t)t * ld;
  int32_t* out_row = idx + (size_t)t * k;

  uint32_t b1 = 0, k1 = 0;
  if (!all_mode) {
    for (int i = threadIdx.x; i < kHistBins; i += kRowThreads) hist[i] = 0;
    __syncthreads();
    // 32 independent loads in flight per thread
    constexpr int kH = 32;
    for (int64_t s0 = threadIdx.x; s0 < n; s0 += kH * kRowThreads) {
      float v[kH];
#pragma unroll
      for (int e = 0; e < kH; ++e) {
        const int64_t s = s0 + (int64_t)e * kRowThreads;
        v[e] = row[s < n ? s : n - 1];
      }
#pragma unroll
      for (int e = 0; e < kH; ++e)
        if (s0 + (int64_t)e * kRowThreads < n) atomicAdd(&hist[order_key(v[e]) >> 20], 1u);
    }
    __syncthreads();
    find_threshold_bin<kRowThreads, kHistBins>(hist, (uint32_t)k, fs.scan, &s_b1, &s_above1);
    b1 = s_b1;
    k1 = (uint32_t)k - s_above1;
    for (int i = threadIdx.x; i < kHistBins; i += kRowThreads) hist[i] = 0;   // becomes h2
    __syncthreads();
  }
  // ordered compaction of candidates (level-1 digit >= b1) into LDS.  A
  // round covers kPer * kRowThreads elements, element base + e * kRowThreads
  // + tid in thread tid (coalesced loads, all issued first); positions follow
  // the index order (e, wave, lane): per-(e, wave) counts from the ballots,
  // one scan over them, then each lane's rank in its ballot.
  constexpr int kPer = 24;
  constexpr int kW = kRowThreads / 64;
  __shared__ uint32_t woff[kPer * kW];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint64_t below = (1ull << lane) - 1ull;
  uint32_t count = 0;
  for (int64_t base = 0; base < n; base += (int64_t)kPer * kRowThreads) {
    uint32_t key[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int64_t s = base + (int64_t)e * kRowThreads + threadIdx.x;
      key[e] = __float_as_uint(row[s < n ? s : n - 1]);
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int64_t s = base + (int64_t)e * kRowThreads + threadIdx.x;
      key[e] = s < n ? order_key(__uint_as_float(key[e])) : 0u;
      const bool f = s < n && (key[e] >> 20) >= b1;
      if (f && !all_mode && (key[e] >> 20) == b1) atomicAdd(&hist[(key[e] >> 8) & 0xFFF], 1u);
      const uint64_t m = __ballot(f);
      if (lane == e) woff[e * kW + wv] = (uint32_t)__builtin_popcountll(m);
    }
    __syncthreads();
    uint32_t tot;
    const uint32_t x = threadIdx.x < kPer * kW ? woff[threadIdx.x] : 0u;
    const uint32_t off = block_excl_scan<kRowThreads>(x, fs.scan, &tot);
    if (threadIdx.x < kPer * kW) woff[threadIdx.x] = off;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int64_t s = base + (int64_t)e * kRowThreads + threadIdx.x;
      const bool f = s < n && (key[e] >> 20) >= b1;
      const uint64_t m = __ballot(f);
      if (f) {
        const uint32_t p = count + woff[e * kW + wv] + (uint32_t)__builtin_popcountll(m & below);
        if (p < kRowCap) cand[p] = make_uint2(key[e], (uint32_t)s);
      }
    }
    count += tot;
    __syncthreads();                                   // woff is rewritten by the next round
  }
  __syncthreads();
  if (count <= kRowCap) {
    FlatSource src{cand, (int)count, kRowThreads};
    final_select<kRowThreads>(src, k, all_mode, b1, k1, hist, fs, out_row);
  } else {
    const int64_t seg = (n + kRowThreads - 1) / kRowThreads;
    RowSource src{row, n, seg, kRowThreads, all_mode ? 0u : b1};
    final_select<kRowThreads>(src, k, all_mode, b1, k1, hist, fs, out_row);
  }
  if (idx_rows) {
    // the same set as cache rows of the sequence
    __syncthreads();
    for (int j = threadIdx.x; j < k; j += kRowThreads) {
      const int32_t v = out_row[j];
      idx_rows[(size_t)t * k + j] = v >= 0 ? (int32_t)(first + v) : -1;
    }
  }
}

bool multi_block(int64_t Lk, int T) {
  return T <= kTopkMultiRowsMax && cdiv(Lk, kCollectRange) <= kMaxSegs;
}

}  // namespace


size_t topk_scratch_bytes(int64_t Lk, int T, int k) {
  (void)k;
  if (!multi_block(Lk, T)) return 256;
  const int64_t G = cdiv(Lk, kCollectRange);
  return (size_t)T * G * kSlotCap * sizeof(uint2) + (size_t)T * G * sizeof(uint32_t) + (size_t)T * 8 + 256;
}

hipError_t launch_topk(const float* scores, int64_t ld, int64_t Lk, int T, int k, int32_t* idx,
                       void* ws_counters, void* scratch, hipStream_t st, bool hist_ready) {
  if (!multi_block(Lk, T)) {
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
                     slots, cnt, rowinfo, (int)G);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_final_kernel, dim3(T, 1 + kHistReplicas), dim3(kFinalThreads), 0, st, scores, ld, Lk, T,
                     k, ctr, (const uint2*)slots, (const uint32_t*)cnt, (const uint32_t*)rowinfo, (int)G, idx);
  return hipGetLastError();
}

bool topk_multi_block(int64_t Lk, int T) { return multi_block(Lk, T); }

hipError_t launch_topk_batch(const float* scores, int64_t ld, const SeqBatch& sb, int B, int T, int k, int32_t* idx,
                             int32_t* idx_rows, hipStream_t st) {
  const int64_t rows = (int64_t)B * T;
  if (rows < 1 || rows > 0x7FFFFFFF || !sb.len) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_row_kernel, dim3((unsigned)rows), dim3(kRowThreads), 0, st, scores, ld, sb.max_len, T, k,
                     idx, sb, idx_rows);
  return hipGetLastError();
}

}  // namespace dsa
