// decode.hip -- the tail of the fused DSA decode step: top-k selection and
// sparse GQA-4 attention with sink in one kernel ("Naive-N0.5-Flash: no
// full-attention layers, and a runtime built by AI", Figure 1: the main heads
// attend to the top-2,048 positions the indexer picked).
//
// The decode scan leaves, for every query row, one list per scan workgroup
// holding that workgroup's exact local top-32 keys sorted by (score desc,
// index asc), with a flag when more than 32 of its keys were visible.  Every
// workgroup of this kernel (512 threads, one list each) then, redundantly and
// without communicating:
//   1. loads its threads' lists (keys and indices) into registers;
//   2. finds the k-th entry of the union in (score desc, index asc) order: a
//      histogram of the keys over the range between a lower bound of the
//      threshold and the largest key picks the bin that holds it, and the
//      entries of that bin are ranked directly when few (otherwise a radix
//      descent over the bin's keys, and then over tied indices, finishes);
//   3. keeps from every list the prefix that precedes that entry, and checks
//      that the union held the true top-k: when a capped list keeps its last
//      entry, keys it dropped may belong to the top-k, and only then the
//      workgroup re-selects from the whole scores row (same result, slower;
//      when the caller asked for no scores the scan stored none, and the
//      workgroup first recomputes the row);
//   4. attends over its chunk of 128 kept keys for one KV head (the same tile
//      loop as sparse_gqa_attn) and writes a partial (max, sum, output), or
//      the output itself when one chunk covers the k keys.
// The partials are merged with the sink by the attention merge kernel.  Every
// workgroup derives the same kept list in the same order, so the result is
// deterministic; the list is sorted only for the optional idx output.  The
// scan deals 16-key tiles round-robin to its workgroups, so a run of up to
// 2,048 consecutive winners puts at most 16 in any one list.
#include "attn_core.hpp"
#include "dsa_common.hpp"
#include "indexer.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace dsa {

namespace {

constexpr int kDecNT = 512;                        // threads: one scan list each
constexpr int kDecNW = 4;                          // attention waves
constexpr int kDecChunk = kDecNW * kTileKeys;      // kept keys per workgroup
constexpr int kMaxLists = 512;
constexpr int kLPT = kMaxLists / kDecNT;           // scan lists per thread
constexpr int kDecMaxChunks = DSA_TOPK_MAX / kDecChunk;
constexpr int kC1Cap = 64;                         // threshold-bin entries ranked directly

// The scores of row t for keys 0 .. n_vis - 1, recomputed by this workgroup
// into row with the scan's arithmetic (the same MFMA operands and order, so
// the same bits) when the scan stored none.  Every workgroup of the row
// writes the same values; the accesses are relaxed atomics, so the concurrent
// writes of equal bits are well defined and a workgroup reads back its own.
__device__ void rescore_row(const DecodeArgs& d, int t, int64_t n_vis, float* row) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  bf16x8 a[4];
  float wv[4];
  widen_fp8(load_frag32_cached(d.q_idx + (size_t)(t * 16 + col) * 128 + 32 * grp), a);
#pragma unroll
  for (int i = 0; i < 4; ++i) wv[i] = d.w[t * 16 + 4 * grp + i];
  constexpr int U = 8;                                          // 16-key tiles per wave in flight
  const int64_t ntiles = cdiv(n_vis, 16);
  for (int64_t t0 = (int64_t)wave * U; t0 < ntiles; t0 += (int64_t)(kDecNT / 64) * U) {
    i32x8 kr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t key = (t0 + u) * 16 + col;
      kr[u] = load_frag32_cached(d.k_idx + (key < n_vis ? key : n_vis - 1) * 128 + 32 * grp);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t key = (t0 + u) * 16 + col;
      bf16x8 b[4];
      widen_fp8(kr[u], b);
      f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) c = mfma_bf16_16x16x32(a[k4], b[k4], c);
      const float s = relu_weighted_sum(c, wv);
      if (grp == 0 && key < n_vis)
        __hip_atomic_store(reinterpret_cast<uint32_t*>(row) + key, __float_as_uint(s), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
}

struct DecodeShared {
  union {
    struct {
      RadixShared rs;
      alignas(16) uint32_t ck[kC1Cap];             // entries of the threshold bin
      alignas(16) uint32_t ci[kC1Cap];
      uint32_t rk[kC1Cap];                         // their ranks within the bin
      uint32_t tk, ti;                             // the k-th entry (key, index)
    } s;
    int32_t sorted[DSA_TOPK_MAX];
    char attn[AttnSmem<kDecNW>::bytes];
  };
  int32_t sel[DSA_TOPK_MAX];
  uint32_t scan[32];
  // written once per launch (no barrier needed before their reuse)
  uint32_t red[kDecNT / 64][5];                    // step 1's reduction
  uint32_t bscan[kDecNT / 64], bout[3];            // the first digit's threshold bin
  uint32_t pscan[kDecNT / 64];                     // the direct path's packed prefix sum
  alignas(16) uint32_t cf[kC1Cap];                 // threshold-bin entry is a capped list's last
};

// Block-wide reduction of step 1 with one barrier: sum of n, or of f, max of
// a, min of b, sum of c.
__device__ __forceinline__ void reduce_lists(uint32_t& n, uint32_t& f, uint32_t& a, uint32_t& b, uint32_t& c,
                                             uint32_t (*red)[5]) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint32_t rn = wave_incl_scan(n), rc = wave_incl_scan(c);
  const uint32_t ra = wave_incl_minmax<true>(a), rb = wave_incl_minmax<false>(b);
  const uint32_t rf = __ballot(f != 0u) != 0ull;
  if (lane == 63) {
    red[wv][0] = rn;
    red[wv][1] = rf;
    red[wv][2] = ra;
    red[wv][3] = rb;
    red[wv][4] = rc;
  }
  __syncthreads();
  n = f = a = c = 0u;
  b = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < kDecNT / 64; ++w) {
    n += red[w][0];
    f |= red[w][1];
    a = a > red[w][2] ? a : red[w][2];
    b = b < red[w][3] ? b : red[w][3];
    c += red[w][4];
  }
}

// the kept list in LDS (DSA_TOPK_MAX entries; positions at or past p1 are
// read clamped and masked, see IdxList)
struct LdsList {
  const int32_t* sel;
  int64_t n_rows;
  __device__ int64_t row(int p, int p1) const {
    const int32_t j = sel[p < DSA_TOPK_MAX ? p : DSA_TOPK_MAX - 1];
    const bool ok = (p < p1) & (j >= 0) & ((int64_t)j < n_rows);   // no short-circuit branch
    return ok ? (int64_t)j : -1;
  }
};

// ascending bitonic sort of a[0..2048) in LDS (NT threads)
template <int NT>
__device__ __forceinline__ void bitonic_sort_2048(int32_t* a) {
  for (int size = 2; size <= DSA_TOPK_MAX; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int p = threadIdx.x; p < DSA_TOPK_MAX / 2; p += NT) {
        const int i = 2 * p - (p & (stride - 1));
        const int j = i + stride;
        const bool up = (i & size) == 0;
        const int32_t x = a[i], y = a[j];
        if ((x > y) == up) {
          a[i] = y;
          a[j] = x;
        }
      }
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(kDecNT) void decode_attend_kernel(DecodeArgs d) {
  __shared__ DecodeShared sh;
  const int c = blockIdx.x, g = blockIdx.y, t = blockIdx.z;
  const int tid = threadIdx.x;
  const AttnArgs& a = d.a;
  const int64_t n_vis = d.Lk - a.T + t + 1;
  const int k = d.k;
  const int nl = d.nlists;

  // ---- 1. this thread's lists tid + 512 q: keys and indices in registers
  // (coalesced over the threads for every entry), clamped so that every load
  // is in flight at once
  const uint32_t* key_row = d.lkeys + (size_t)t * kListM * nl;
  const uint32_t* idx_row = d.lidx + (size_t)t * kListM * nl;
  // cth = ceil(k / lists): the cth-th entry of every list bounds the threshold
  // from below (loaded with the lists, see step 2)
  const uint32_t cth = (uint32_t)((k + nl - 1) / nl);
  const int cj = cth < (uint32_t)kListM ? (int)cth - 1 : kListM - 1;
  uint32_t kA[kLPT][kListM], iA[kLPT][kListM], n[kLPT], kc[kLPT];
  bool full[kLPT];
#pragma unroll
  for (int q = 0; q < kLPT; ++q) {
    const int lq = tid + kDecNT * q;
    const int l = lq < nl ? lq : nl - 1;
    const uint32_t w = d.lcount[(size_t)t * nl + l];
#pragma unroll
    for (int j = 0; j < kListM; ++j) {
      kA[q][j] = key_row[j * nl + l];
      iA[q][j] = idx_row[j * nl + l];
    }
    kc[q] = key_row[cj * nl + l];
    n[q] = lq < nl ? w & 0x7FFFFFFFu : 0u;
    full[q] = lq < nl && (w >> 31) != 0u;
    // A list's entries past its count hold key 0 (the scan writes them so),
    // and so do those of a thread without a list, so that below every bound
    // (L0 and what derives from it, all real keys, at least 1) a test of the
    // key alone also excludes them.
    if (lq >= nl) {
#pragma unroll
      for (int j = 0; j < kListM; ++j) kA[q][j] = 0u;
    }
  }
  // the block's entries M, whether any list is capped, the largest key
  // kmax, the smallest cth-th entry xc and the lists nc holding cth entries;
  // meanwhile the first digit's histogram is cleared
  uint32_t M = 0u, full_any = 0u, kmax = 0u, xc = 0xFFFFFFFFu, nc = 0u;
#pragma unroll
  for (int q = 0; q < kLPT; ++q) {
    M += n[q];
    full_any |= (uint32_t)full[q];
    if (n[q]) kmax = kmax > kA[q][0] ? kmax : kA[q][0];
    if (n[q] >= cth) {
      ++nc;
      xc = xc < kc[q] ? xc : kc[q];
    }
  }
  for (int i = tid; i < kHistBins; i += kDecNT) sh.s.rs.hist[i] = 0;
  reduce_lists(M, full_any, kmax, xc, nc, sh.red);
  const bool any_full = full_any != 0u;

  // ---- 2. the k-th entry (tk, ti) of the union: keep key > tk, or key == tk and index <= ti
  bool fallback;
  bool direct = false;                         // the kept set is already in sel
  uint32_t n_sel_direct = 0;
  uint32_t tk = 0u, ti = 0xFFFFFFFFu;
  if (n_vis <= (int64_t)k) {
    fallback = any_full;                       // the lists hold every visible key only when uncapped
  } else if (M < (uint32_t)k) {
    fallback = true;
  } else {
    // The histogram covers [L0, Kmax]: Kmax is the largest key, and L0 a
    // lower bound of the threshold -- c = ceil(k / lists) entries of every
    // list with at least c entries reach the smallest c-th entry, and when
    // those lists hold k entries or more that entry bounds the threshold;
    // otherwise the smallest entry of all does.  Spreading the candidates
    // over the bins of this range keeps the LDS atomics apart.
    // Every pass below visits a list's entries only while they can matter:
    // the lists are sorted, so the entries at or above a bound form a prefix,
    // and a wave skips each block of 8 entries that starts past the longest
    // such prefix among its lanes (the gate `go`, wave-uniform).
    RadixShared& rs = sh.s.rs;
    uint32_t L0 = xc;
    if ((uint64_t)nc * cth < (uint64_t)k) {    // block-uniform: the smallest entry of all bounds instead
      uint32_t z0 = 0u, z1 = 0xFFFFFFFFu, z2 = 0u, xl = 0xFFFFFFFFu;
#pragma unroll
      for (int q = 0; q < kLPT; ++q)
#pragma unroll
        for (int j = 0; j < kListM; ++j)
          if ((uint32_t)j + 1 == n[q]) xl = xl < kA[q][j] ? xl : kA[q][j];
      block_reduce_mmms<kDecNT>(z0, z1, xl, z2, sh.scan);
      L0 = xl;
    }
    const uint32_t span = kmax - L0;
    const int bits = span ? 32 - __builtin_clz(span) : 0;
    const int s1 = bits > 12 ? bits - 12 : 0;   // bits of u = key - L0 below the first digit
    const int s2 = s1 > 12 ? s1 - 12 : 0;       // below the second (at most 8)
    // histogram of ((u >> shift) & mask) over the entries >= L0 with u >> mshift == prefix
    auto level = [&](int shift, uint32_t mask, int mshift, uint32_t prefix, int nbins) {
      for (int i = tid; i < nbins; i += kDecNT) rs.hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kLPT; ++q)
#pragma unroll
        for (int j0 = 0, go = 1; j0 < kListM; j0 += 8) {
          go = go && __ballot(kA[q][j0] >= L0) != 0ull;
          if (go) {
#pragma unroll
            for (int j = j0; j < j0 + 8; ++j) {
              const uint32_t u = kA[q][j] - L0;
              if (kA[q][j] >= L0 && (uint32_t)((uint64_t)u >> mshift) == prefix)
                atomicAdd(&rs.hist[(u >> shift) & mask], 1u);
            }
          }
        }
      __syncthreads();
    };
    // first digit: (key - L0) >> s1 over every entry >= L0 (cleared in step 1)
#pragma unroll
    for (int q = 0; q < kLPT; ++q)
#pragma unroll
      for (int j0 = 0, go = 1; j0 < kListM; j0 += 8) {
        go = go && __ballot(kA[q][j0] >= L0) != 0ull;
        if (go) {
#pragma unroll
          for (int j = j0; j < j0 + 8; ++j)
            if (kA[q][j] >= L0) atomicAdd(&rs.hist[(kA[q][j] - L0) >> s1], 1u);
        }
      }
    __syncthreads();
    uint32_t b1, above1, cnt1;                 // the bin, the entries in the bins above it, in it
    find_threshold_bin_once<kDecNT, kHistBins>(rs.hist, (uint32_t)k, sh.bscan, sh.bout, &b1, &above1, &cnt1);
    uint32_t need = (uint32_t)k - above1;      // entries still to take from bin b1
    const uint32_t lo = L0 + (b1 << s1);       // bin b1 holds the keys lo .. hi
    const uint32_t wid = (1u << s1) - 1u;
    const uint32_t hi = lo > 0xFFFFFFFFu - wid ? 0xFFFFFFFFu : lo + wid;
    auto in_b1 = [&](int q, int j) {
      return (uint32_t)(kA[q][j] >= lo) & (uint32_t)(kA[q][j] <= hi);
    };
    if (cnt1 <= (uint32_t)kC1Cap) {
      // Few entries in bin b1: the entries above the bin (a prefix of every
      // list) are kept, and the bin's entries are ranked directly -- those of
      // rank < need are kept too.  One packed prefix sum places both groups:
      // [entries above the bin, in list order] then [kept bin entries by rank].
      // A capped list that keeps its last entry may hide winners: then the
      // whole selection falls back (step 3).
      uint32_t ndq[kLPT], nd = 0, nb = 0;
      bool hides = false;
#pragma unroll
      for (int q = 0; q < kLPT; ++q) {
        ndq[q] = 0;
#pragma unroll
        for (int j0 = 0, go = 1; j0 < kListM; j0 += 8) {
          go = go && __ballot(kA[q][j0] >= lo) != 0ull;
          if (go) {
#pragma unroll
            for (int j = j0; j < j0 + 8; ++j) {
              const bool in = kA[q][j] >= lo;
              ndq[q] += (uint32_t)(in && kA[q][j] > hi);
              nb += (uint32_t)(in && kA[q][j] <= hi);
            }
          }
        }
        nd += ndq[q];
        hides |= full[q] && n[q] == (uint32_t)kListM && kA[q][kListM - 1] > hi;
      }
      uint32_t tot;
      const uint32_t packed = block_excl_scan_once<kDecNT>((nd << 16) | nb, sh.pscan, &tot);
      uint32_t pd = packed >> 16, pb = packed & 0xFFFFu;
#pragma unroll
      for (int q = 0; q < kLPT; ++q) {
#pragma unroll
        for (int j0 = 0, go = 1; j0 < kListM; j0 += 8) {   // the entries above the bin lead the list
          go = go && __ballot(kA[q][j0] >= lo) != 0ull;
          if (go) {
#pragma unroll
            for (int j = j0; j < j0 + 8; ++j) {
              if ((uint32_t)j < ndq[q] && pd + j < (uint32_t)DSA_TOPK_MAX) sh.sel[pd + j] = (int32_t)iA[q][j];
              if (in_b1(q, j)) {
                sh.s.ck[pb] = kA[q][j];
                sh.s.ci[pb] = iA[q][j];
                sh.cf[pb] = (uint32_t)(full[q] && (uint32_t)j + 1 == n[q]);
                ++pb;
              }
            }
          }
        }
        pd += ndq[q];
      }
      const uint32_t ncp = (cnt1 + 15u) & ~15u;  // padded with key 0, which ranks below every entry
      if ((uint32_t)tid >= cnt1 && (uint32_t)tid < ncp) {
        sh.s.ck[tid] = 0u;
        sh.s.ci[tid] = 0xFFFFFFFFu;
      }
      __syncthreads();
      if ((uint32_t)tid < cnt1) {
        const uint32_t key = sh.s.ck[tid], id = sh.s.ci[tid];
        auto before = [&](uint32_t kj, uint32_t ij) {
          return (uint32_t)(kj > key) | ((uint32_t)(kj == key) & (uint32_t)(ij < id));
        };
        uint32_t rank = 0;
        for (uint32_t j0 = 0; j0 < ncp; j0 += 16) {
          uint4 k4[4], i4[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            k4[q] = *reinterpret_cast<const uint4*>(&sh.s.ck[j0 + 4 * q]);
            i4[q] = *reinterpret_cast<const uint4*>(&sh.s.ci[j0 + 4 * q]);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q)
            rank += before(k4[q].x, i4[q].x) + before(k4[q].y, i4[q].y) + before(k4[q].z, i4[q].z) +
                    before(k4[q].w, i4[q].w);
        }
        if (rank < need) {
          if (above1 + rank < (uint32_t)DSA_TOPK_MAX) sh.sel[above1 + rank] = (int32_t)id;
          hides |= sh.cf[tid] != 0u;
        }
      }
      fallback = __syncthreads_or(hides);
      if (!fallback) {
        n_sel_direct = (uint32_t)k;
        direct = true;
      }
    } else {
      // a crowded bin: radix descent over its keys, then over the tied indices
      uint32_t known = b1, eq = cnt1;
      if (s1 > 0) {
        level(s2, (1u << (s1 - s2)) - 1u, s1, known, kHistBins);
        find_threshold_bin<kDecNT, kHistBins>(rs.hist, need, rs.scan, &rs.bin, &rs.above);
        known = (known << (s1 - s2)) | rs.bin;
        need -= rs.above;
        eq = rs.hist[rs.bin];
        __syncthreads();
      }
      if (s2 > 0) {
        level(0, (1u << s2) - 1u, s2, known, kHist3Bins);
        find_threshold_bin<kDecNT, kHist3Bins>(rs.hist, need, rs.scan, &rs.bin, &rs.above);
        known = (known << s2) | rs.bin;
        need -= rs.above;
        eq = rs.hist[rs.bin];
        __syncthreads();
      }
      tk = L0 + known;
      if (eq > need) {                         // keep the `need` lowest indices among the ties
        uint32_t tau2, r2, eq2;
        radix_threshold<kDecNT>([&](int i) { return key_row[i] == tk ? ~idx_row[i] : 0u; }, kListM * nl, need,
                                rs, &tau2, &r2, &eq2);
        ti = ~tau2;
      }
      fallback = false;
    }
  }

  // ---- 3. the kept prefix of each list; a capped list keeping its last entry may hide winners
  uint32_t n_sel = n_sel_direct;
  if (!direct) {
    uint32_t cnt[kLPT];
#pragma unroll
    for (int q = 0; q < kLPT; ++q) cnt[q] = 0u;
    if (!fallback) {
      bool hides = false;
#pragma unroll
      for (int q = 0; q < kLPT; ++q) {
        if (n_vis <= (int64_t)k) {
          cnt[q] = n[q];
        } else {
#pragma unroll
          for (int j0 = 0, go = 1; j0 < kListM; j0 += 8) {
            go = go && __ballot(kA[q][j0] >= tk) != 0ull;
            if (go) {
#pragma unroll
              for (int j = j0; j < j0 + 8; ++j)
                cnt[q] += (uint32_t)(kA[q][j] >= tk && (kA[q][j] > tk || iA[q][j] <= ti));
            }
          }
        }
        hides |= full[q] && cnt[q] == n[q];
      }
      fallback = __syncthreads_or(hides);
    }
    __syncthreads();

    if (!fallback) {
      uint32_t cnt_all = 0;
#pragma unroll
      for (int q = 0; q < kLPT; ++q) cnt_all += cnt[q];
      uint32_t base = block_excl_scan<kDecNT>(cnt_all, sh.scan, &n_sel);
#pragma unroll
      for (int q = 0; q < kLPT; ++q) {
#pragma unroll
        for (int j0 = 0, go = 1; j0 < kListM; j0 += 8) {
          go = go && __ballot((uint32_t)j0 < cnt[q]) != 0ull;
          if (go) {
#pragma unroll
            for (int j = j0; j < j0 + 8; ++j)
              if ((uint32_t)j < cnt[q] && base + j < (uint32_t)DSA_TOPK_MAX) sh.sel[base + j] = (int32_t)iA[q][j];
          }
        }
        base += cnt[q];
      }
      if (n_sel > (uint32_t)DSA_TOPK_MAX) n_sel = DSA_TOPK_MAX;
    } else {
      const float* row = d.scores + (int64_t)t * d.ld;
      if (d.rescore) {
        rescore_row(d, t, n_vis, d.rescore + (int64_t)t * d.ld);
        __syncthreads();
      }
      auto row_key = [&](int i) {
        return order_key(__uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(row) + i,
                                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)));
      };
      uint32_t tau = 0, r = 0, eq = 0;
      if (n_vis > (int64_t)k) radix_threshold<kDecNT>(row_key, (int)n_vis, (uint32_t)k, sh.s.rs, &tau, &r, &eq);
      n_sel = ordered_keep<kDecNT>(row_key, (int)n_vis, tau, r, sh.scan,
                                   [&](uint32_t pos, int i) { sh.sel[pos] = i; });
    }
    __syncthreads();
  }
  // (on the direct path the fallback vote was the barrier after the last write of sel)

  // ---- optional idx output, ascending, written by one workgroup per row
  if (d.idx_out && c == 0 && g == 0) {
    for (int i = tid; i < DSA_TOPK_MAX; i += kDecNT) sh.sorted[i] = (uint32_t)i < n_sel ? sh.sel[i] : 0x7FFFFFFF;
    __syncthreads();
    bitonic_sort_2048<kDecNT>(sh.sorted);
    int32_t* o = d.idx_out + (size_t)t * k;
    for (int i = tid; i < k; i += kDecNT) o[i] = (uint32_t)i < n_sel ? sh.sorted[i] : -1;
    __syncthreads();                           // sorted shares its memory with the attention's
  }

  // ---- 4. attention over this workgroup's chunk of the kept list
  const int p0 = c * kDecChunk < (int)n_sel ? c * kDecChunk : (int)n_sel;
  const int p1 = p0 + kDecChunk < (int)n_sel ? p0 + kDecChunk : (int)n_sel;
  LdsList src{sh.sel, a.n_rows};
  attend_chunk<DSA_KV_HEADS, kDecNW, LdsList, kDecNT>(a, src, t, g, c, d.n_chunks, p0, p1, d.part, sh.attn);
}

}  // namespace

int decode_chunks(int k) { return (int)cdiv(k, kDecChunk); }

hipError_t launch_decode_attend(const DecodeArgs& d, hipStream_t st) {
  if (d.nlists < 1 || d.nlists > kMaxLists || d.k > DSA_TOPK_MAX || d.n_chunks > kDecMaxChunks)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(decode_attend_kernel, dim3(d.n_chunks, DSA_KV_HEADS, d.a.T), dim3(kDecNT), 0, st, d);
  return hipGetLastError();
}

}  // namespace dsa
