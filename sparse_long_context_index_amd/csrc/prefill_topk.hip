// prefill_topk.hip -- per-row top-k of the index scores of a prefill chunk
// without writing the score matrix ("Naive-N0.5-Flash: no full-attention
// layers, and a runtime built by AI", section "Inside a DSA layer: the
// lightning indexer": every visible key is scored, the top index_top_k are
// kept; section "What 'no full-attention layers' means": the selection is a
// stable descending argsort).
//
// Three kernels around the prefill contraction (prefill_scores.hip):
//  1. the contraction over a strided sample of the keys writes a small score
//     matrix (every 64th key); prefill_theta_kernel takes per row the r-th
//     largest sampled score as the row's threshold theta (r chosen so that
//     about max(2.5 k, 4096) keys of the whole row reach it, against 8192
//     candidate slots), or no threshold when the row's visible keys fit in
//     its slots;
//  2. the contraction over all keys appends every visible key whose score
//     reaches theta to the row's candidate slots (no score matrix);
//  3. prefill_refine_kernel selects the exact top-k of each row from its
//     candidates by (score desc, index asc) and writes it in ascending index
//     order.  The candidates hold every key at or above theta, so whenever
//     they number at least min(k, visible keys) and all fit, the result is the
//     exact top-k of the row.  A row for which that fails is listed; the host
//     side recomputes listed rows one by one with the same arithmetic.
#include "dsa_common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace dsa {

namespace {

constexpr int kPtNT = 1024;
constexpr int kSortN = DSA_TOPK_MAX;                 // bitonic sort width (k <= 2048)

__global__ __launch_bounds__(kPtNT) void prefill_theta_kernel(const float* __restrict__ sample, int64_t ld,
                                                              int64_t Lk, int T, int step, int rank, int cap,
                                                              uint32_t* __restrict__ theta) {
  __shared__ RadixShared rs;
  const int t = blockIdx.x;
  const int64_t p = Lk - T + t;
  if (p + 1 <= cap) {                                  // every visible key fits: no threshold
    if (threadIdx.x == 0) theta[t] = 0u;
    return;
  }
  const int ns = (int)(p / step) + 1;                  // sampled keys j * step <= p
  const uint32_t need = (uint32_t)(rank < ns ? rank : ns);
  const float* row = sample + (size_t)t * ld;
  uint32_t tau, r, eq;
  radix_threshold<kPtNT>([&](int j) { return j < ns ? order_key(row[j]) : 0u; }, ns, need, rs, &tau, &r, &eq);
  if (threadIdx.x == 0) theta[t] = tau;
}

struct RefineShared {
  RadixShared rs;
  uint32_t sel[kSortN];
  uint32_t nsel;
};

__global__ __launch_bounds__(kPtNT) void prefill_refine_kernel(PrefillCand pc, int64_t Lk, int T, int k,
                                                               int32_t* __restrict__ idx, uint32_t* __restrict__ nfail,
                                                               uint32_t* __restrict__ failed) {
  extern __shared__ __attribute__((aligned(16))) char dyn[];
  RefineShared& sh = *reinterpret_cast<RefineShared*>(dyn);
  uint32_t* ckey = reinterpret_cast<uint32_t*>(dyn + sizeof(RefineShared));
  uint32_t* cidx = ckey + pc.cap;
  const int t = blockIdx.x;
  const int64_t nvis = Lk - T + t + 1;
  const uint32_t need = (uint32_t)(nvis < k ? nvis : k);
  const uint32_t n = pc.count[t];
  int32_t* out = idx + (size_t)t * k;
  if (n > (uint32_t)pc.cap || n < need) {              // block-uniform
    if (threadIdx.x == 0) failed[atomicAdd(nfail, 1u)] = (uint32_t)t;
    return;
  }
  const uint2* src = pc.cand + (size_t)t * pc.cap;
  for (uint32_t i = threadIdx.x; i < n; i += kPtNT) {
    const uint2 e = src[i];
    ckey[i] = e.x;
    cidx[i] = e.y;
  }
  __syncthreads();
  select_sorted<kPtNT>(ckey, cidx, (int)n, need, k, sh.rs, sh.sel, &sh.nsel, out);
}

}  // namespace

size_t prefill_refine_lds(int cap) { return sizeof(RefineShared) + (size_t)cap * 8; }

hipError_t launch_prefill_theta(const float* sample, int64_t ld, int64_t Lk, int T, int step, int k, int cap,
                                uint32_t* theta, hipStream_t st) {
  // about 2.5 k (at least 64 step) keys of the whole row reach the rank-th
  // largest sampled score; a rank of 64 or more keeps the estimate steady
  int rank = (int)cdiv((int64_t)5 * k, 2 * (int64_t)step);
  if (rank < 64) rank = 64;
  if ((int64_t)rank * step * 3 / 2 > cap) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prefill_theta_kernel, dim3(T), dim3(kPtNT), 0, st, sample, ld, Lk, T, step, rank, cap, theta);
  return hipGetLastError();
}

hipError_t launch_prefill_refine(const PrefillCand& pc, int64_t Lk, int T, int k, int32_t* idx, uint32_t* nfail,
                                 uint32_t* failed, hipStream_t st) {
  if (k < 1 || k > kSortN) return hipErrorInvalidValue;
  const size_t lds = prefill_refine_lds(pc.cap);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prefill_refine_kernel, dim3(T), dim3(kPtNT), lds, st, pc, Lk, T, k, idx, nfail, failed);
  return hipGetLastError();
}

}  // namespace dsa
