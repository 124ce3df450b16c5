// prefill_topk.hip -- per-row top-k of the index scores of a prefill chunk
// without writing the score matrix ("Naive-N0.5-Flash: no full-attention
// layers, and a runtime built by AI", section "Inside a DSA layer: the
// lightning indexer": every visible key is scored, the top index_top_k are
// kept; section "What 'no full-attention layers' means": the selection is a
// stable descending argsort).
//
// The fp8 MFMA contraction (prefill_scores.hip) only locates candidates; the
// selection is made on exact scores (the decode scan's arithmetic), so the
// result is the top-k of the exact scores, row for row:
//  1. key_norm_kernel: an upper bound n_s of every key's Euclidean norm;
//  2. the contraction over a strided sample of the keys (every 64th) writes a
//     small score matrix; prefill_theta_kernel takes per row the r-th largest
//     sampled score as the row's threshold theta (about max(2 k, 4096) keys
//     of the row reach it, against 12,288 candidate slots; no threshold when
//     the row's visible keys fit the slots), and the row's error factor
//     c_t = c |u| with u_d = sum_h |w_h| |q_hd| (c bounds the contraction's
//     error relative to sum_h |w_h| sum_d |q_hd k_d| = u . |k|, which
//     Cauchy-Schwarz bounds by |u| |k|);
//  3. the contraction over all keys appends every visible key s whose score
//     plus c_t n_s plus 0.01 sum_h |w_h| R_h reaches theta to the row's slots
//     (the last term covers the bf16 head sums of this pass, R_h its rounded
//     ReLU logits): no key whose exact score reaches theta is missed;
//  4. prefill_rescore_kernel recomputes the candidates' scores exactly;
//  5. prefill_refine_kernel checks that at least min(k, visible keys)
//     candidates reach theta on their exact scores -- then every key left out
//     scores below theta and the row's top-k lies among the candidates -- and
//     selects it by (exact score desc, index asc) in ascending index order.
//     Rows whose candidates overflow the slots or fail the check are listed;
//  6. prefill_fallback_kernel (topk.hip) recomputes each listed row's exact
//     scores and selects from them (a launch with no listed row ends at once).
// No step reads anything back to the host, so the call can be captured.
#include "dsa_common.hpp"
#include "indexer.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace dsa {

namespace {

constexpr int kPtNT = 1024;
constexpr int kSortN = DSA_TOPK_MAX;                 // bitonic sort width (k <= 2048)

// Relative bound used for the candidate margin: the contraction adds each
// group of 8 products after aligning them to the group's largest exponent and
// keeps at least 13 fraction bits below it, so a group loses at most
// 8 * 2^-13 of its largest product (2^-10 of the absolute sum); fp32 sums and
// the exact path's own rounding add below 1e-4.  2^-9 doubles the whole.
constexpr double kCandRel = 1.0 / 512.0;

__global__ __launch_bounds__(kPtNT) void prefill_theta_kernel(const float* __restrict__ sample, int64_t ld,
                                                              const uint8_t* __restrict__ q_idx,
                                                              const float* __restrict__ w, int64_t Lk, int T, int step,
                                                              int rank, int cap, uint32_t* __restrict__ theta,
                                                              float* __restrict__ cw) {
  __shared__ RadixShared rs;
  __shared__ double usq[2];
  const int t = blockIdx.x;
  const int64_t p = Lk - T + t;
  if (threadIdx.x < 128) {
    // u_d = sum_h |w_h| |q_hd| and |u|^2 in double (thread d; two waves)
    double u = 0.0;
    for (int h = 0; h < 16; ++h) {
      const uint8_t code = q_idx[((size_t)t * 16 + h) * 128 + threadIdx.x];
      const bf16x2 v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)code, 1.0f, false);
      u += fabs((double)w[(size_t)t * 16 + h]) * fabs((double)(float)v[0]);
    }
    double sq = u * u;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sq += __shfl_xor(sq, o, 64);
    if ((threadIdx.x & 63) == 0) usq[threadIdx.x >> 6] = sq;
  }
  __syncthreads();
  if (threadIdx.x == 0) cw[t] = __double2float_ru(sqrt(usq[0] + usq[1]) * kCandRel * (1.0 + 1.0 / 1048576.0));
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

// Upper bound of every key's Euclidean norm: four lanes per key each widen 32
// bytes and sum their squares in double (exact), the key's sum of 128
// squares is exact, its square root rounded up to float.
__global__ __launch_bounds__(256) void key_norm_kernel(const uint8_t* __restrict__ k_idx, int64_t Lk,
                                                       float* __restrict__ knorm) {
  const int64_t key = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 2);
  double ss = 0.0;
  if (key < Lk) {
    bf16x8 v[4];
    widen_fp8(load_frag32_cached(k_idx + key * 128 + 32 * (threadIdx.x & 3)), v);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double x = (double)(float)v[s4][e];
        ss += x * x;
      }
  }
  ss += __shfl_xor(ss, 1, 64);
  ss += __shfl_xor(ss, 2, 64);
  if (key < Lk && (threadIdx.x & 3) == 0) knorm[key] = __double2float_ru(sqrt(ss) * (1.0 + 1.0 / 1048576.0));
}

// Exact scores of the candidates: block (t, y) takes candidates 256 y ..
// 256 y + 255 of row t, 16 per wave-step (one per lane column), four steps'
// key loads in flight, and replaces each candidate's order key with that of
// its exact score.
constexpr int kRescoreNT = 256;
constexpr int kRescorePer = 256;

__global__ __launch_bounds__(kRescoreNT) void prefill_rescore_kernel(PrefillCand pc, const uint8_t* __restrict__ q_idx,
                                                                     const float* __restrict__ w,
                                                                     const uint8_t* __restrict__ k_idx) {
  const int t = blockIdx.x;
  uint32_t n = pc.count[t];
  n = n < (uint32_t)pc.cap ? n : (uint32_t)pc.cap;
  const uint32_t i0 = blockIdx.y * kRescorePer;
  if (i0 >= n) return;                                 // block-uniform
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  ExactQuery eq;
  load_exact_query(q_idx + (size_t)t * 16 * 128, w + (size_t)t * 16, eq);
  uint2* c = pc.cand + (size_t)t * pc.cap;
  constexpr int U = kRescorePer / (kRescoreNT / 64) / 16;   // 16-candidate steps per wave
  i32x8 kr[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t i = i0 + (uint32_t)(wave * U + u) * 16 + col;
    const uint32_t key = c[i < n ? i : n - 1].y;
    kr[u] = load_frag32_cached(k_idx + (size_t)key * 128 + 32 * grp);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t i = i0 + (uint32_t)(wave * U + u) * 16 + col;
    const float s = exact_score(eq, kr[u]);
    if (grp == 0 && i < n) c[i].x = order_key(s);
  }
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
  const uint32_t th = pc.theta[t];
  int32_t* out = idx + (size_t)t * k;
  bool ok = n <= (uint32_t)pc.cap && n >= need;        // block-uniform
  if (ok) {
    // the exact keys, and how many reach the threshold
    const uint2* src = pc.cand + (size_t)t * pc.cap;
    uint32_t reach = 0;
    for (uint32_t i = threadIdx.x; i < n; i += kPtNT) {
      const uint2 e = src[i];
      ckey[i] = e.x;
      cidx[i] = e.y;
      reach += e.x >= th;
    }
    uint32_t tot;
    (void)block_excl_scan<kPtNT>(reach, sh.rs.scan, &tot);
    ok = tot >= need;
  }
  if (!ok) {
    if (threadIdx.x == 0) failed[atomicAdd(nfail, 1u)] = (uint32_t)t;
    return;
  }
  select_sorted<kPtNT>(ckey, cidx, (int)n, need, k, sh.rs, sh.sel, &sh.nsel, out);
}

}  // namespace

size_t prefill_refine_lds(int cap) { return sizeof(RefineShared) + (size_t)cap * 8; }

hipError_t launch_key_norms(const uint8_t* k_idx, int64_t Lk, float* knorm, hipStream_t st) {
  const int64_t blocks = cdiv(Lk, 64);
  if (blocks < 1 || blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(key_norm_kernel, dim3((unsigned)blocks), dim3(256), 0, st, k_idx, Lk, knorm);
  return hipGetLastError();
}

hipError_t launch_prefill_theta(const float* sample, int64_t ld, const uint8_t* q_idx, const float* w, int64_t Lk,
                                int T, int step, int k, int cap, uint32_t* theta, float* cw, hipStream_t st) {
  // about 2 k (at least 64 step) keys of the whole row reach the rank-th
  // largest sampled score; a rank of 64 or more keeps the estimate steady
  int rank = (int)cdiv((int64_t)2 * k, (int64_t)step);
  if (rank < 64) rank = 64;
  if ((int64_t)rank * step * 3 / 2 > cap) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prefill_theta_kernel, dim3(T), dim3(kPtNT), 0, st, sample, ld, q_idx, w, Lk, T, step, rank, cap,
                     theta, cw);
  return hipGetLastError();
}

hipError_t launch_prefill_rescore(const PrefillCand& pc, const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                                  int T, hipStream_t st) {
  if (pc.cap < 1 || T < 1 || cdiv(pc.cap, kRescorePer) > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prefill_rescore_kernel, dim3((unsigned)T, (unsigned)cdiv(pc.cap, kRescorePer)), dim3(kRescoreNT),
                     0, st, pc, q_idx, w, k_idx);
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
