// attn.hip -- gathered GQA attention with a sink logit on gfx950.
//
// "Naive-N0.5-Flash: no full-attention layers, and a runtime built by AI",
// section "Inside a DSA layer: the lightning indexer": the main heads attend
// only to the selected keys (the rest are masked before the softmax), GQA
// with 4 KV heads on DSA layers and 8 on SWA layers, and a sink column; the
// section "What 'no full-attention layers' means" gives the SWA mask (offset
// from the query below the window).  Both are one kernel here: a DSA unit
// reads its key list from idx, an SWA unit uses the window of its sequence.
//
// Work unit: one query token (or sequence) t and one KV head g, i.e. the 16
// (DSA) or 8 (SWA) query heads sharing K/V rows.  A unit's key list may be
// split into chunks over several workgroups (decode); each chunk yields a
// partial (max, sum, unnormalised output) that a merge kernel combines with
// the sink.  Inside a workgroup each wave takes 32-key tiles:
//   QK : K rows are gathered straight into the A operand of two 16x16x32 bf16
//        MFMA chains (keys x head-columns), 6 k-steps over qk dim 192;
//   softmax: online, base-2, per head column, fp32;
//   PV : P (heads x 32 keys) is already in A-operand order; V rows are staged
//        through LDS (after the QK and the softmax, which wait for the K rows
//        only) and read as the B operand, 8 MFMAs over v dim 128 for each of
//        P's two bf16 parts (high, and the rounding remainder), so the
//        products keep ~16 bits of every probability.
// Empty slots (idx < 0, idx >= Lk, positions past the window) read a clamped
// valid row but use none of it: their V lanes are staged as zeros and their
// logits set to -inf, so poisoned cache rows outside the set can never reach
// the output.
#include "attn_core.hpp"
#include "dsa_common.hpp"
#include "kernels.hpp"

namespace dsa {

namespace {

template <int HKV, int NW>
__global__ __launch_bounds__(NW * 64) void sparse_attn_kernel(AttnArgs a, int n_chunks, int chunk_keys,
                                                             float* part) {
  __shared__ __attribute__((aligned(16))) char smem[AttnSmem<NW>::bytes];
  const int c = blockIdx.x, g = blockIdx.y, t = blockIdx.z;
  const int p0 = c * chunk_keys;
  const int p1 = p0 + chunk_keys < a.k_len ? p0 + chunk_keys : a.k_len;
  IdxList src{a.idx + (size_t)t * a.k_len, a.k_len, a.n_rows};
  attend_chunk<HKV, NW>(a, src, t, g, c, n_chunks, p0, p1, part, smem);
}

template <int HKV, int NW>
__global__ __launch_bounds__(NW * 64) void swa_attn_kernel(AttnArgs a, int n_chunks, int chunk_keys,
                                                          float* part) {
  __shared__ __attribute__((aligned(16))) char smem[AttnSmem<NW>::bytes];
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int64_t s = a.seq_start[b];              // issued first: both scalar loads are in flight before
  const int64_t n = a.seq_len[b];                // the wait that the first use of either needs
  const int len = n <= 0 ? 0 : (int)(n < a.window ? n : a.window);
  const int64_t first = s + n - len;
  // Positions whose rows lie at or past the cache's end read as empty slots
  // either way; leaving them out of the range also makes the loop bound need
  // both descriptor words, so both loads leave before the first branch (one
  // round trip before the K/V addresses are known, not two).
  const int64_t room = a.n_rows - first;
  const int lenc = room < (int64_t)len ? (room > 0 ? (int)room : 0) : len;
  Window src{first, len, a.n_rows};
  const int p0 = c * chunk_keys;
  const int p1 = p0 + chunk_keys < lenc ? p0 + chunk_keys : lenc;
  attend_chunk<HKV, NW>(a, src, b, g, c, n_chunks, p0 < p1 ? p0 : p1, p1, part, smem);
}

// merge the chunk partials of every (t, head) and add the sink.  All loads
// go out together as vector loads: lane c of each wave fetches chunk c's
// (max, sum) and the sink, and the values are then read across the wave, so
// the kernel waits for one memory round trip.
constexpr int kMaxChunks = 32;

template <int HKV, int MAXC>
__global__ __launch_bounds__(128) void attn_merge_kernel(AttnArgs a, int n_chunks, const float* part) {
  static_assert(MAXC <= 64, "one chunk per lane");
  constexpr int GH = 64 / HKV;
  const int h = blockIdx.x, t = blockIdx.y;
  const int g = h / GH, hc = h % GH;
  const int dv = threadIdx.x;
  const int lane = dv & 63;
  const float* pp = part + ((size_t)(t * HKV + g) * n_chunks) * kPartFloats;
  const int cl = lane < n_chunks ? lane : 0;                   // chunk 0 stands in beyond n_chunks
  const float ml = pp[(size_t)cl * kPartFloats + hc];
  const float ll = pp[(size_t)cl * kPartFloats + 16 + hc];
  // lane 63 fetches the sink (a lane-dependent address keeps it a vector load
  // issued with the others); the other lanes re-read a word of the partials
  const float sl = *((a.sink && lane == 63) ? a.sink + h : pp + hc);
  float oc[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const float* q = pp + (size_t)(c < n_chunks ? c : 0) * kPartFloats;
    oc[c] = q[32 + hc * 128 + dv];                             // loaded unconditionally, masked below
  }
  float mc[MAXC], lc[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const bool ok = c < n_chunks;
    mc[c] = ok ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ml), c)) : -INFINITY;
    lc[c] = ok ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ll), c)) : 0.f;
    oc[c] = ok ? oc[c] : 0.f;
  }
  const float s2 = a.sink ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sl), 63)) * kLog2e : -INFINITY;
  float M = s2;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) M = fmaxf(M, mc[c]);
  float L = 0.f, O = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const float f = mc[c] == -INFINITY ? 0.f : exp2_hw(mc[c] - M);
      L += f * lc[c];
      O += f * oc[c];
    }
    if (a.sink) L += exp2_hw(s2 - M);
  }
  const float outv = (M != -INFINITY && L > 0.f) ? O / L : 0.f;
  a.out[((size_t)t * 64 + h) * 128 + dv] = f32_to_bf16_rne(outv);
  if (a.lse && dv == 0) a.lse[(size_t)t * 64 + h] = M == -INFINITY ? -INFINITY : (M + log2f(L)) * kLn2;
}

constexpr int kNW = 4;                          // waves per workgroup, unsplit units
constexpr int kSplitNW = 2;                     // waves per workgroup when a unit is split
constexpr int kSplitChunk = kSplitNW * kTileKeys;

int sparse_chunks(int T, int k_len) {
  // split a unit's key list over several workgroups until the grid has about
  // 1,024 of them (4 per CU), with at least one 64-key tile pair per chunk
  const int units = T * DSA_KV_HEADS;
  if (units >= 1024) return 1;
  int c = (1024 + units - 1) / units;
  const int by_keys = (k_len + kSplitChunk - 1) / kSplitChunk;
  c = c < by_keys ? c : by_keys;
  return c < kMaxChunks ? (c > 1 ? c : 1) : kMaxChunks;
}

}  // namespace

size_t attn_scratch_bytes(int T, int k_len, int hkv) {
  const int c = hkv == DSA_KV_HEADS ? sparse_chunks(T, k_len) : 1;
  if (c <= 1) return 256;
  return (size_t)T * hkv * c * kPartFloats * sizeof(float) + 256;
}

hipError_t launch_sparse_attn(const AttnArgs& a, void* scratch, hipStream_t st) {
  const int n_chunks = sparse_chunks(a.T, a.k_len);
  float* part = reinterpret_cast<float*>(scratch);
  if (n_chunks == 1) {
    hipLaunchKernelGGL((sparse_attn_kernel<DSA_KV_HEADS, kNW>), dim3(1, DSA_KV_HEADS, a.T), dim3(kNW * 64), 0,
                       st, a, 1, a.k_len, part);
    return hipGetLastError();
  }
  const int chunk = (int)cdiv(cdiv(a.k_len, n_chunks), kTileKeys) * kTileKeys;
  const int n_used = (int)cdiv(a.k_len, chunk);
  hipLaunchKernelGGL((sparse_attn_kernel<DSA_KV_HEADS, kSplitNW>), dim3(n_used, DSA_KV_HEADS, a.T),
                     dim3(kSplitNW * 64), 0, st, a, n_used, chunk, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attn_merge(a, n_used, part, st);
}

hipError_t launch_attn_merge(const AttnArgs& a, int n_chunks, const float* part, hipStream_t st) {
  if (n_chunks < 1 || n_chunks > kMaxChunks) return hipErrorInvalidValue;
  if (n_chunks <= 8)
    hipLaunchKernelGGL((attn_merge_kernel<DSA_KV_HEADS, 8>), dim3(64, a.T), dim3(128), 0, st, a, n_chunks, part);
  else if (n_chunks <= 16)
    hipLaunchKernelGGL((attn_merge_kernel<DSA_KV_HEADS, 16>), dim3(64, a.T), dim3(128), 0, st, a, n_chunks, part);
  else
    hipLaunchKernelGGL((attn_merge_kernel<DSA_KV_HEADS, kMaxChunks>), dim3(64, a.T), dim3(128), 0, st, a,
                       n_chunks, part);
  return hipGetLastError();
}

hipError_t launch_swa_attn(const AttnArgs& a, void* scratch, hipStream_t st) {
  (void)scratch;
  const int chunk = (int)cdiv(a.window, kTileKeys) * kTileKeys;
  hipLaunchKernelGGL((swa_attn_kernel<SWA_KV_HEADS, kNW>), dim3(1, SWA_KV_HEADS, a.T), dim3(kNW * 64), 0, st, a,
                     1, chunk, (float*)nullptr);
  return hipGetLastError();
}

}  // namespace dsa
