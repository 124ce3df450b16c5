// decode.hip -- the tail of the fused DSA decode step: top-k selection and
// sparse GQA-4 attention with sink in one kernel ("Naive-N0.5-Flash: no
// full-attention layers, and a runtime built by AI", Figure 1: the main heads
// attend to the top-2,048 positions the indexer picked).
//
// The decode scan leaves, for every query row, one list per scan workgroup
// holding that workgroup's exact local top-32 keys sorted by (score desc,
// index asc), with a flag when more than 32 of its keys were visible.  Every
// workgroup of this kernel then, redundantly and without communicating:
//   1. copies the row's list keys into LDS (512 x 32 at most, entry-major);
//   2. finds the exact top-k threshold of that union by a radix descent of
//      up to three digits over the key range between a lower bound of the
//      threshold and the largest key (ties at the threshold are split by a
//      second descent on the key index);
//   3. takes from every list the prefix it keeps, and checks that the union
//      held the true top-k: when a capped list keeps its last entry, keys it
//      dropped may belong to the top-k, and only then the workgroup
//      re-selects from the whole scores row instead (same result, slower);
//   4. attends over its chunk of 128 kept keys for one KV head (the same tile
//      loop as sparse_gqa_attn) and writes a partial (max, sum, output);
//   5. the last workgroup of each (token, KV head) merges the partials with
//      the sink.
// Every workgroup derives the same kept list in the same order, so the
// result is deterministic; the list is sorted only for the optional idx
// output.  The scan deals 16-key tiles round-robin to its workgroups, so a run
// of up to 2,048 consecutive winners puts at most 16 in any one list.
#include "attn_core.hpp"
#include "dsa_common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace dsa {

namespace {

constexpr int kDecNW = 4;                          // waves per workgroup
constexpr int kDecChunk = kDecNW * kTileKeys;      // kept keys per workgroup
constexpr int kMaxLists = 512;
constexpr int kDecMaxChunks = DSA_TOPK_MAX / kDecChunk;
constexpr int kBatch = 8;                          // list entries read per round trip

struct DecodeShared {
  union {
    struct {
      uint32_t key[kListM * kMaxLists];            // entry j of list l at [j * nlists + l]
      RadixShared rs;
    } s;
    int32_t sorted[DSA_TOPK_MAX];
    char attn[AttnSmem<kDecNW>::bytes];
    float mrg[kDecMaxChunks * 32 + kDecMaxChunks * 16 + 16];
  };
  int32_t sel[DSA_TOPK_MAX];
  uint32_t scan[16];
  uint32_t flag;
};

struct LdsList {
  const int32_t* sel;
  int64_t n_rows;
  __device__ int64_t row(int p) const {
    const int32_t j = sel[p];
    return (j >= 0 && (int64_t)j < n_rows) ? (int64_t)j : -1;
  }
};

// ascending bitonic sort of a[0..2048) in LDS (256 threads)
__device__ __forceinline__ void bitonic_sort_2048(int32_t* a) {
  for (int size = 2; size <= DSA_TOPK_MAX; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int p = threadIdx.x; p < DSA_TOPK_MAX / 2; p += 256) {
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

__global__ __launch_bounds__(256) void decode_attend_kernel(DecodeArgs d) {
  __shared__ DecodeShared sh;
  const int c = blockIdx.x, g = blockIdx.y, t = blockIdx.z;
  const int tid = threadIdx.x;
  const AttnArgs& a = d.a;
  const int64_t n_vis = d.Lk - a.T + t + 1;
  const int k = d.k;
  const int nl = d.nlists;

  // ---- 1. the row's list keys (entry-major) and this thread's two lists;
  // every load is unconditional (clamped) so that all are in flight at once
  const uint32_t* cnt_row = d.lcount + (size_t)t * nl;
  const uint32_t* idx_row = d.lidx + (size_t)t * kListM * nl;
  const int la = tid, lb = tid + 256;
  const int lca = la < nl ? la : nl - 1, lcb = lb < nl ? lb : nl - 1;
  uint32_t wa = cnt_row[lca], wb = cnt_row[lcb];
  uint32_t pia[kBatch], pib[kBatch];                 // the first key indices of both lists
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    pia[j] = idx_row[j * nl + lca];
    pib[j] = idx_row[j * nl + lcb];
  }
  {
    const uint4* src = reinterpret_cast<const uint4*>(d.lkeys + (size_t)t * kListM * nl);
    uint4* dst = reinterpret_cast<uint4*>(sh.s.key);
    constexpr int kCopy = kListM * kMaxLists / 4 / 256;   // uint4 per thread at the largest list count
    const int n4 = kListM * nl / 4;
    uint4 v[kCopy];
#pragma unroll
    for (int b = 0; b < kCopy; ++b) {
      const int i = b * 256 + tid;
      v[b] = src[i < n4 ? i : n4 - 1];
    }
#pragma unroll
    for (int b = 0; b < kCopy; ++b) dst[b * 256 + tid] = v[b];   // beyond n4: unread LDS
  }
  if (la >= nl) wa = 0u;
  if (lb >= nl) wb = 0u;
  const uint32_t na = wa & 0x7FFFFFFFu, nb = wb & 0x7FFFFFFFu;
  uint32_t M;
  block_excl_scan<256>(na + nb, sh.scan, &M);
  const bool any_full = __syncthreads_or(((wa | wb) >> 31) != 0u);   // also publishes the keys

  // ---- 2. threshold of the top-k of the lists' union
  const uint32_t* U = sh.s.key;
  uint32_t kA[kListM], kB[kListM];             // this thread's lists, in registers
#pragma unroll
  for (int j = 0; j < kListM; ++j) {
    kA[j] = U[j * nl + lca];
    kB[j] = U[j * nl + lcb];
  }
  bool fallback;
  uint32_t tau = 0, tau2 = 0;
  bool split = false;
  if (n_vis <= (int64_t)k) {
    fallback = any_full;                       // the lists hold every visible key only when uncapped
  } else if (M < (uint32_t)k) {
    fallback = true;
  } else {
    // The digits cover only [L0, Kmax]: Kmax is the largest key, and L0 a
    // lower bound of the threshold -- c = ceil(k / lists) entries of every
    // list with at least c entries reach the smallest c-th entry, and when
    // those lists hold k entries or more that entry bounds the threshold;
    // otherwise the smallest entry of all does.  Spreading the candidates
    // over the bins of this range keeps the LDS atomics apart.
    RadixShared& rs = sh.s.rs;
    const uint32_t c = (uint32_t)((k + nl - 1) / nl);
    uint32_t kmax = na ? kA[0] : 0u, kmax_b = nb ? kB[0] : 0u;
    kmax = kmax > kmax_b ? kmax : kmax_b;
    uint32_t xc = 0xFFFFFFFFu, xl = 0xFFFFFFFFu, nc = 0u;
    if (na >= c) { xc = U[(c - 1) * nl + lca]; ++nc; }
    if (nb >= c) { const uint32_t v = U[(c - 1) * nl + lcb]; xc = xc < v ? xc : v; ++nc; }
    if (na) xl = U[(na - 1) * nl + lca];
    if (nb) { const uint32_t v = U[(nb - 1) * nl + lcb]; xl = xl < v ? xl : v; }
    block_reduce_mmms<256>(kmax, xc, xl, nc, sh.scan);
    const uint32_t L0 = (uint64_t)nc * c >= (uint64_t)k ? xc : xl;
    const uint32_t span = kmax - L0;
    const int bits = span ? 32 - __builtin_clz(span) : 0;
    const int s1 = bits > 12 ? bits - 12 : 0;   // bits of u = key - L0 below level 1
    const int s2 = s1 > 12 ? s1 - 12 : 0;       // below level 2 (at most 8)
    // histogram of ((u >> shift) & mask) over the candidates with u >> mshift == prefix
    auto level = [&](int shift, uint32_t mask, int mshift, uint32_t prefix, int nbins) {
      for (int i = tid; i < nbins; i += 256) rs.hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kListM; ++j) {
        const uint32_t ua = kA[j] - L0, ub = kB[j] - L0;
        if ((uint32_t)j < na && kA[j] >= L0 && (uint32_t)((uint64_t)ua >> mshift) == prefix)
          atomicAdd(&rs.hist[(ua >> shift) & mask], 1u);
        if ((uint32_t)j < nb && kB[j] >= L0 && (uint32_t)((uint64_t)ub >> mshift) == prefix)
          atomicAdd(&rs.hist[(ub >> shift) & mask], 1u);
      }
      __syncthreads();
    };
    level(s1, 0xFFFu, 32, 0u, kHistBins);
    find_threshold_bin<256, kHistBins>(rs.hist, (uint32_t)k, rs.scan, &rs.bin, &rs.above);
    uint32_t known = rs.bin;                   // u >> s1
    uint32_t need = (uint32_t)k - rs.above;
    uint32_t eq = rs.hist[known];
    __syncthreads();
    if (s1 > 0) {
      level(s2, (1u << (s1 - s2)) - 1u, s1, known, kHistBins);
      find_threshold_bin<256, kHistBins>(rs.hist, need, rs.scan, &rs.bin, &rs.above);
      known = (known << (s1 - s2)) | rs.bin;   // u >> s2
      need -= rs.above;
      eq = rs.hist[rs.bin];
      __syncthreads();
    }
    if (s2 > 0) {
      level(0, (1u << s2) - 1u, s2, known, kHist3Bins);
      find_threshold_bin<256, kHist3Bins>(rs.hist, need, rs.scan, &rs.bin, &rs.above);
      known = (known << s2) | rs.bin;          // u
      need -= rs.above;
      eq = rs.hist[rs.bin];
      __syncthreads();
    }
    tau = L0 + known;
    const uint32_t r = need;
    if (eq > r) {                              // keep the r lowest key indices among the ties
      uint32_t r2, eq2;
      radix_threshold<256>([&](int i) { return U[i] == tau ? ~idx_row[i] : 0u; }, kListM * nl, r, rs, &tau2,
                           &r2, &eq2);
      split = true;
    }
    fallback = false;
  }

  // ---- 3. the kept prefix of each list (kept entries lead a sorted list); a
  // capped list that keeps its last entry may hide winners
  uint32_t ca = 0, cb = 0;
  if (!fallback) {
    if (n_vis <= (int64_t)k) {
      ca = na;
      cb = nb;
    } else {
      if (!split) {
#pragma unroll
        for (int j = 0; j < kListM; ++j) {
          ca += (uint32_t)((uint32_t)j < na) & (uint32_t)(kA[j] >= tau);
          cb += (uint32_t)((uint32_t)j < nb) & (uint32_t)(kB[j] >= tau);
        }
      } else {                                 // ties at tau split by key index: rare
        for (int j = 0; j < kListM; ++j) {
          const uint32_t ka = U[j * nl + lca], kb = U[j * nl + lcb];
          ca += (uint32_t)j < na && (ka > tau || (ka == tau && ~idx_row[j * nl + lca] >= tau2));
          cb += (uint32_t)j < nb && (kb > tau || (kb == tau && ~idx_row[j * nl + lcb] >= tau2));
        }
      }
    }
    const bool hides = ((wa >> 31) && ca == na) || ((wb >> 31) && cb == nb);
    fallback = __syncthreads_or(hides);
  }
  __syncthreads();                             // the keys are dead from here

  uint32_t n_sel;
  if (!fallback) {
    const uint32_t base = block_excl_scan<256>(ca + cb, sh.scan, &n_sel);
    auto put = [&](uint32_t pos, uint32_t id) {
      if (pos < (uint32_t)DSA_TOPK_MAX) sh.sel[pos] = (int32_t)id;
    };
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if ((uint32_t)j < ca) put(base + j, pia[j]);
      if ((uint32_t)j < cb) put(base + ca + j, pib[j]);
    }
    for (uint32_t j = kBatch; j < ca; ++j) put(base + j, idx_row[j * nl + lca]);        // long prefixes: rare
    for (uint32_t j = kBatch; j < cb; ++j) put(base + ca + j, idx_row[j * nl + lcb]);
    if (n_sel > (uint32_t)DSA_TOPK_MAX) n_sel = DSA_TOPK_MAX;
  } else {
    const float* row = d.scores + (int64_t)t * d.ld;
    auto row_key = [&](int i) { return order_key(row[i]); };
    uint32_t r = 0, eq = 0;
    tau = 0;
    if (n_vis > (int64_t)k) radix_threshold<256>(row_key, (int)n_vis, (uint32_t)k, sh.s.rs, &tau, &r, &eq);
    n_sel = ordered_keep<256>(row_key, (int)n_vis, tau, r, sh.scan,
                              [&](uint32_t pos, int i) { sh.sel[pos] = i; });
  }
  __syncthreads();

  // ---- optional idx output, ascending, written by one workgroup per row
  if (d.idx_out && c == 0 && g == 0) {
    for (int i = tid; i < DSA_TOPK_MAX; i += 256) sh.sorted[i] = (uint32_t)i < n_sel ? sh.sel[i] : 0x7FFFFFFF;
    __syncthreads();
    bitonic_sort_2048(sh.sorted);
    int32_t* o = d.idx_out + (size_t)t * k;
    for (int i = tid; i < k; i += 256) o[i] = (uint32_t)i < n_sel ? sh.sorted[i] : -1;
  }
  __syncthreads();

  // ---- 4. attention over this workgroup's chunk of the kept list
  const int p0 = c * kDecChunk < (int)n_sel ? c * kDecChunk : (int)n_sel;
  const int p1 = p0 + kDecChunk < (int)n_sel ? p0 + kDecChunk : (int)n_sel;
  LdsList src{sh.sel, a.n_rows};
  attend_chunk<DSA_KV_HEADS, kDecNW>(a, src, t, g, c, d.n_chunks, p0, p1, d.part, sh.attn);
  if (d.n_chunks == 1) return;

  // ---- 5. the last workgroup of this (token, KV head) merges the partials
  __threadfence();
  __syncthreads();
  if (tid == 0) sh.flag = atomicAdd(&d.unit_ctr[t * DSA_KV_HEADS + g], 1u) == (uint32_t)(d.n_chunks - 1);
  __syncthreads();
  if (!sh.flag) return;
  __threadfence();
  const int nc = d.n_chunks;
  const float* pp = d.part + (size_t)(t * DSA_KV_HEADS + g) * nc * kPartFloats;
  float* mc = sh.mrg;                              // [nc][32]: m then l of 16 heads
  float* fw = sh.mrg + kDecMaxChunks * 32;         // [nc][16]: chunk weights
  float* inv = fw + kDecMaxChunks * 16;            // [16]
  {
    const int e0 = tid, e1 = tid + 256, ne = nc * 32;
    const float v0 = pp[(size_t)((e0 < ne ? e0 : ne - 1) >> 5) * kPartFloats + (e0 & 31)];
    const float v1 = pp[(size_t)((e1 < ne ? e1 : ne - 1) >> 5) * kPartFloats + (e1 & 31)];
    mc[e0] = v0;                                   // beyond ne: unread
    mc[e1] = v1;
  }
  __syncthreads();
  if (tid < 16) {
    const int h = g * 16 + tid;
    const float s2 = a.sink ? a.sink[h] * kLog2e : -INFINITY;
    float mv[kDecMaxChunks], lv[kDecMaxChunks];
#pragma unroll
    for (int cc = 0; cc < kDecMaxChunks; ++cc) {
      const float m = mc[cc * 32 + tid], l = mc[cc * 32 + 16 + tid];
      mv[cc] = cc < nc ? m : -INFINITY;
      lv[cc] = cc < nc ? l : 0.f;
    }
    float Mx = s2;
#pragma unroll
    for (int cc = 0; cc < kDecMaxChunks; ++cc) Mx = fmaxf(Mx, mv[cc]);
    float L = 0.f;
#pragma unroll
    for (int cc = 0; cc < kDecMaxChunks; ++cc) {
      const float f = (Mx == -INFINITY || mv[cc] == -INFINITY) ? 0.f : exp2f(mv[cc] - Mx);
      fw[cc * 16 + tid] = f;
      L += f * lv[cc];
    }
    if (a.sink && Mx != -INFINITY) L += exp2f(s2 - Mx);
    const bool ok = Mx != -INFINITY && L > 0.f;
    inv[tid] = ok ? 1.f / L : 0.f;
    if (a.lse) a.lse[(size_t)t * 64 + h] = Mx == -INFINITY ? -INFINITY : (Mx + log2f(L)) * kLn2;
  }
  __syncthreads();
  const int dv = tid & 127;
  const int h0 = tid >> 7;                         // heads h0, h0 + 2, ..., h0 + 14
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
#pragma unroll
  for (int cc = 0; cc < kDecMaxChunks; ++cc) {
    const float* q = pp + (size_t)(cc < nc ? cc : nc - 1) * kPartFloats + 32 + dv;   // weight 0 beyond nc
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += fw[cc * 16 + h0 + 2 * j] * q[(h0 + 2 * j) * 128];
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int hc = h0 + 2 * j;
    a.out[((size_t)t * 64 + g * 16 + hc) * 128 + dv] = f32_to_bf16_rne(acc[j] * inv[hc]);
  }
  if (tid == 0) d.unit_ctr[t * DSA_KV_HEADS + g] = 0;
}

}  // namespace

int decode_chunks(int k) { return (int)cdiv(k, kDecChunk); }

hipError_t launch_decode_attend(const DecodeArgs& d, hipStream_t st) {
  if (d.nlists < 1 || d.nlists > kMaxLists || d.k > DSA_TOPK_MAX || d.n_chunks > kDecMaxChunks)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(decode_attend_kernel, dim3(d.n_chunks, DSA_KV_HEADS, d.a.T), dim3(256), 0, st, d);
  return hipGetLastError();
}

}  // namespace dsa
