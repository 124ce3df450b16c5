// api.hip -- the extern "C" entry points of libdsa.so: host-side validation,
// workspace carving and launch sequencing.  Every check happens before the
// first launch, so a rejected call enqueues nothing and touches no output.
#include <cmath>
#include <mutex>

#include "dsa_common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace dsa {

namespace {

__global__ void zero_kernel(uint4* __restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline dsa_status hip_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

constexpr int64_t kMaxLk = (int64_t)1 << 31;

dsa_status check_index_args(const void* q_idx, const void* w, const void* k_idx, int64_t Lk, int32_t T) {
  if (!q_idx || !w || !k_idx) return DSA_ERR_NULL;
  if (!aligned16(q_idx) || !aligned16(w) || !aligned16(k_idx)) return DSA_ERR_ALIGN;
  if (T < 1 || Lk < T || Lk >= kMaxLk) return DSA_ERR_SHAPE;
  return DSA_OK;
}

dsa_status check_attn_args(const void* q, const void* k, const void* v, const void* out, const void* sink,
                           const void* lse, float sm_scale) {
  if (!q || !k || !v || !out) return DSA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return DSA_ERR_ALIGN;
  if ((sink && !aligned16(sink)) || (lse && !aligned16(lse))) return DSA_ERR_ALIGN;
  if (!std::isfinite(sm_scale)) return DSA_ERR_SHAPE;
  return DSA_OK;
}

struct DecodeLayout {
  size_t scores, idx, topk, attn, lkeys, lidx, lcount, part, total;
};

constexpr size_t kScanListLdsMax = 80 * 1024;   // keeps two scan workgroups per CU
constexpr int kScanListsMax = 512;

// The fused path: the scan writes per-workgroup top lists and one kernel
// selects, attends and merges.  It needs the scan's LDS to stay small and
// about k / 8 or more scan workgroups, so that a list of 32 rarely fills up
// (a full list that keeps its last entry sends the selection to the slow
// full-row re-selection).  Otherwise: histogram top-k, then attention.
bool use_list_path(int64_t Lk, int T, int k) {
  if (T > kScanListTMax) return false;
  const int grid = scan_grid(Lk);
  const size_t lds = scan_lds_bytes(Lk, T, true);
  return lds <= kScanListLdsMax && grid <= kScanListsMax && (int64_t)k <= (int64_t)8 * grid;
}

DecodeLayout decode_layout(int64_t Lk, int T, int k) {
  DecodeLayout d;
  size_t off = kCounterRegionBytes;
  d.scores = off;
  off += align_up((size_t)T * Lk * sizeof(float));
  d.idx = off;
  off += align_up((size_t)T * k * sizeof(int32_t));
  d.topk = off;
  off += align_up(topk_scratch_bytes(Lk, T, k));
  d.attn = off;
  off += align_up(attn_scratch_bytes(T, k, DSA_KV_HEADS));
  d.lkeys = off;
  off += align_up((size_t)T * kScanListsMax * kListM * sizeof(uint32_t));
  d.lidx = off;
  off += align_up((size_t)T * kScanListsMax * kListM * sizeof(uint32_t));
  d.lcount = off;
  off += align_up((size_t)T * kScanListsMax * sizeof(uint32_t));
  d.part = off;
  off += align_up((size_t)T * DSA_KV_HEADS * decode_chunks(k) * (16 + 16 + 16 * 128) * sizeof(float));
  d.total = off;
  return d;
}

// workspace of the fused prefill top-k
struct PrefillLayout {
  size_t sample, theta, cw, knorm, count, failed, cand, fb, total;
  int64_t ld_sample, ld_fb;
  int fb_blocks;
};

PrefillLayout prefill_layout(int64_t Lk, int T) {
  PrefillLayout d;
  d.ld_sample = (cdiv(Lk, kPrefillStep) + 3) / 4 * 4;
  d.ld_fb = (Lk + 63) / 64 * 64;
  d.fb_blocks = T < kPrefillFallbackBlocks ? T : kPrefillFallbackBlocks;
  size_t off = kCounterRegionBytes;
  d.sample = off;
  off += align_up((size_t)T * d.ld_sample * sizeof(float));
  d.theta = off;
  off += align_up((size_t)T * sizeof(uint32_t));
  d.cw = off;
  off += align_up((size_t)T * sizeof(float));
  d.knorm = off;
  off += align_up((size_t)Lk * sizeof(float));
  d.count = off;                               // T row counters, then the failure count
  off += align_up(((size_t)T + 4) * sizeof(uint32_t));
  d.failed = off;
  off += align_up((size_t)T * sizeof(uint32_t));
  d.cand = off;
  off += align_up((size_t)T * kPrefillCap * sizeof(uint2));
  d.fb = off;                                  // score rows of the exact fallback
  off += align_up((size_t)d.fb_blocks * d.ld_fb * sizeof(float));
  d.total = off;
  return d;
}

// workspace of the batched decode step
struct BatchLayout {
  size_t scores, idx, rows, attn, total;
  int64_t ld;
};

BatchLayout batch_layout(int64_t max_len, int T, int k, int B) {
  BatchLayout d;
  d.ld = (max_len + 3) / 4 * 4;
  const size_t R = (size_t)B * T;
  size_t off = kCounterRegionBytes;
  d.scores = off;
  off += align_up(R * d.ld * sizeof(float));
  d.idx = off;
  off += align_up(R * k * sizeof(int32_t));
  d.rows = off;
  off += align_up(R * k * sizeof(int32_t));
  d.attn = off;
  off += align_up(attn_scratch_bytes((int)R, k, DSA_KV_HEADS));
  d.total = off;
  return d;
}

constexpr int kBatchTMax = 16;

// workspace of the recall measurement
struct RecallLayout {
  size_t attn, out, lse, part, total;
};

RecallLayout recall_layout(int64_t Lk, int T, int k) {
  RecallLayout d;
  size_t off = kCounterRegionBytes;
  d.attn = off;
  off += align_up(attn_scratch_bytes(T, k, DSA_KV_HEADS));
  d.out = off;
  off += align_up((size_t)T * DSA_Q_HEADS * DSA_V_DIM * sizeof(uint16_t));
  d.lse = off;
  off += align_up((size_t)T * DSA_Q_HEADS * sizeof(float));
  d.part = off;
  off += align_up((size_t)T * DSA_KV_HEADS * recall_chunks(Lk) * 32 * sizeof(float));
  d.total = off;
  return d;
}

}  // namespace

hipError_t launch_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, reinterpret_cast<uint4*>(p), n16);
  return hipGetLastError();
}

namespace {

// ---- static scratch of the no-allocation decode step
// Each GPU that runs the library holds one copy of this array until the
// process ends.  Host code never passes the name itself to a kernel: on the
// host it is only a stand-in for the symbol; the device address of each GPU's
// copy comes from hipGetSymbolAddress at set-up.
static __device__ __align__(256) uint8_t scratch[DSA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`: its address is looked up once per
// device, with that device current, and kept.  Returns null on a HIP error.
void* static_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev]) return g_scratch_ptr[dev];
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
  g_scratch_ptr[dev] = ptr;
  return ptr;
}

}  // namespace

}  // namespace dsa

using namespace dsa;

extern "C" {

const char* dsa_status_string(dsa_status s) {
  switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_NULL: return "DSA_ERR_NULL: a required pointer is NULL";
    case DSA_ERR_SHAPE: return "DSA_ERR_SHAPE: a size or value is out of range";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED: request not implemented";
    case DSA_ERR_ALIGN: return "DSA_ERR_ALIGN: a pointer is not 16-byte aligned";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace missing or too small";
    case DSA_ERR_HIP: return "DSA_ERR_HIP: the HIP runtime reported an error";
    case DSA_ERR_SCRATCH: return "DSA_ERR_SCRATCH: the request needs more than the static scratch holds";
  }
  return "unknown dsa_status";
}

const char* dsa_version(void) { return "dsa-mi355x 0.1.0 gfx950"; }

size_t dsa_workspace_bytes(dsa_op op, int64_t Lk, int32_t T, int32_t k, int32_t B) {
  switch (op) {
    case DSA_OP_INDEX_SCORES:
      return 0;
    case DSA_OP_TOPK:
      if (T < 1 || Lk < T || Lk >= kMaxLk || k < 1 || k > DSA_TOPK_MAX) return 0;
      return kCounterRegionBytes + align_up(topk_scratch_bytes(Lk, T, k));
    case DSA_OP_SPARSE_ATTN:
      if (T < 1 || k < 1 || k > DSA_TOPK_MAX) return 0;
      return kCounterRegionBytes + align_up(attn_scratch_bytes(T, k, DSA_KV_HEADS));
    case DSA_OP_SWA_ATTN:
      if (B < 1) return 0;
      return kCounterRegionBytes + align_up(attn_scratch_bytes(B, SWA_WINDOW_MAX, SWA_KV_HEADS));
    case DSA_OP_DECODE_STEP:
      if (T < 1 || T > DSA_DECODE_T_MAX || Lk < T || Lk >= kMaxLk || k < 1 || k > DSA_TOPK_MAX) return 0;
      return decode_layout(Lk, T, k).total;
    case DSA_OP_DECODE_BATCH:
      if (B < 1 || B > 65535 || T < 1 || T > kBatchTMax || Lk < T || Lk >= kMaxLk || k < 1 || k > DSA_TOPK_MAX ||
          (int64_t)B * T > 0x7FFFFFFF)
        return 0;
      return batch_layout(Lk, T, k, B).total;
    case DSA_OP_INDEX_RECALL:
      if (T < 1 || Lk < T || Lk >= kMaxLk || k < 1 || k > DSA_TOPK_MAX || T > 65535) return 0;
      return recall_layout(Lk, T, k).total;
    case DSA_OP_PREFILL_TOPK:
      if (T < 1 || Lk < T || Lk >= kMaxLk || k < 1 || k > DSA_TOPK_MAX) return 0;
      return prefill_layout(Lk, T).total;
  }
  return 0;
}

dsa_status dsa_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return DSA_ERR_NULL;
  if (!aligned16(ws)) return DSA_ERR_ALIGN;
  if (ws_bytes < kCounterRegionBytes) return DSA_ERR_WORKSPACE;
  return hip_status(launch_zero(ws, kCounterRegionBytes, as_stream(stream)));
}

dsa_status dsa_index_scores(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t Lk, int32_t T,
                            float* scores, int64_t ld_scores, void* stream) {
  dsa_status s = check_index_args(q_idx, w, k_idx, Lk, T);
  if (s != DSA_OK) return s;
  if (!scores) return DSA_ERR_NULL;
  if (!aligned16(scores)) return DSA_ERR_ALIGN;
  if (ld_scores < Lk) return DSA_ERR_SHAPE;
  return hip_status(launch_index_scores(q_idx, w, k_idx, Lk, T, scores, ld_scores, as_stream(stream)));
}

dsa_status dsa_topk(const float* scores, int64_t ld_scores, int64_t Lk, int32_t T, int32_t k, int32_t* idx,
                    void* ws, size_t ws_bytes, void* stream) {
  if (!scores || !idx) return DSA_ERR_NULL;
  if (!aligned16(scores) || !aligned16(idx)) return DSA_ERR_ALIGN;
  if (T < 1 || Lk < T || Lk >= kMaxLk || ld_scores < Lk || k < 1 || k > DSA_TOPK_MAX) return DSA_ERR_SHAPE;
  if (!ws || ws_bytes < dsa_workspace_bytes(DSA_OP_TOPK, Lk, T, k, 0)) return DSA_ERR_WORKSPACE;
  if (!aligned16(ws)) return DSA_ERR_ALIGN;
  char* base = static_cast<char*>(ws);
  return hip_status(launch_topk(scores, ld_scores, Lk, T, k, idx, base, base + kCounterRegionBytes,
                                as_stream(stream)));
}

dsa_status sparse_gqa_attn(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, int64_t Lk,
                           const int32_t* idx, int32_t T, int32_t k, const float* sink, float sm_scale,
                           uint16_t* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  dsa_status s = check_attn_args(q, k_cache, v_cache, out, sink, lse, sm_scale);
  if (s != DSA_OK) return s;
  if (!idx) return DSA_ERR_NULL;
  if (!aligned16(idx)) return DSA_ERR_ALIGN;
  if (T < 1 || k < 1 || k > DSA_TOPK_MAX || Lk < 1 || Lk >= kMaxLk) return DSA_ERR_SHAPE;
  if (!ws || ws_bytes < dsa_workspace_bytes(DSA_OP_SPARSE_ATTN, Lk, T, k, 0)) return DSA_ERR_WORKSPACE;
  if (!aligned16(ws)) return DSA_ERR_ALIGN;
  AttnArgs a{};
  a.q = q; a.k = k_cache; a.v = v_cache; a.n_rows = Lk;
  a.idx = idx; a.k_len = k; a.T = T;
  a.sink = sink; a.sm_scale = sm_scale; a.out = out; a.lse = lse;
  return hip_status(launch_sparse_attn(a, static_cast<char*>(ws) + kCounterRegionBytes, as_stream(stream)));
}

dsa_status swa_attn(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, int64_t n_rows,
                    const int64_t* seq_start, const int32_t* seq_len, int32_t B, int32_t window,
                    const float* sink, float sm_scale, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                    void* stream) {
  dsa_status s = check_attn_args(q, k_cache, v_cache, out, sink, lse, sm_scale);
  if (s != DSA_OK) return s;
  if (!seq_start || !seq_len) return DSA_ERR_NULL;
  if (!aligned16(seq_start) || !aligned16(seq_len)) return DSA_ERR_ALIGN;
  if (B < 1 || window < 1 || window > SWA_WINDOW_MAX || n_rows < 1) return DSA_ERR_SHAPE;
  if (!ws || ws_bytes < dsa_workspace_bytes(DSA_OP_SWA_ATTN, 0, 0, 0, B)) return DSA_ERR_WORKSPACE;
  if (!aligned16(ws)) return DSA_ERR_ALIGN;
  AttnArgs a{};
  a.q = q; a.k = k_cache; a.v = v_cache; a.n_rows = n_rows;
  a.seq_start = seq_start; a.seq_len = seq_len; a.window = window; a.T = B;
  a.sink = sink; a.sm_scale = sm_scale; a.out = out; a.lse = lse;
  return hip_status(launch_swa_attn(a, static_cast<char*>(ws) + kCounterRegionBytes, as_stream(stream)));
}

dsa_status dsa_decode_step(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, const uint16_t* q,
                           const uint16_t* k_cache, const uint16_t* v_cache, int64_t Lk, int32_t T, int32_t k,
                           const float* sink, float sm_scale, uint16_t* out, float* lse, int32_t* idx_out,
                           float* scores_out, int64_t ld_scores, void* ws, size_t ws_bytes, void* stream) {
  dsa_status s = check_index_args(q_idx, w, k_idx, Lk, T);
  if (s != DSA_OK) return s;
  s = check_attn_args(q, k_cache, v_cache, out, sink, lse, sm_scale);
  if (s != DSA_OK) return s;
  if (T > DSA_DECODE_T_MAX || k < 1 || k > DSA_TOPK_MAX) return DSA_ERR_SHAPE;
  if ((idx_out && !aligned16(idx_out)) || (scores_out && !aligned16(scores_out))) return DSA_ERR_ALIGN;
  if (scores_out && ld_scores < Lk) return DSA_ERR_SHAPE;
  const size_t need = dsa_workspace_bytes(DSA_OP_DECODE_STEP, Lk, T, k, 0);
  if (!ws || ws_bytes < need) return DSA_ERR_WORKSPACE;
  if (!aligned16(ws)) return DSA_ERR_ALIGN;

  const DecodeLayout L = decode_layout(Lk, T, k);
  char* base = static_cast<char*>(ws);
  float* scores = scores_out ? scores_out : reinterpret_cast<float*>(base + L.scores);
  const int64_t ld = scores_out ? ld_scores : Lk;
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(base + L.idx);
  hipStream_t st = as_stream(stream);

  if (use_list_path(Lk, T, k)) {
    ScanLists sl;
    sl.keys = reinterpret_cast<uint32_t*>(base + L.lkeys);
    sl.idx = reinterpret_cast<uint32_t*>(base + L.lidx);
    sl.count = reinterpret_cast<uint32_t*>(base + L.lcount);
    sl.store_scores = scores_out != nullptr;     // else only a re-selection needs them, and recomputes them
    hipError_t e = launch_index_scores(q_idx, w, k_idx, Lk, T, scores, ld, st, nullptr, sl);
    if (e != hipSuccess) return DSA_ERR_HIP;
    DecodeArgs d{};
    d.a.q = q; d.a.k = k_cache; d.a.v = v_cache; d.a.n_rows = Lk; d.a.T = T; d.a.k_len = k;
    d.a.sink = sink; d.a.sm_scale = sm_scale; d.a.out = out; d.a.lse = lse;
    d.scores = scores; d.ld = ld; d.Lk = Lk; d.k = k;
    d.rescore = sl.store_scores ? nullptr : scores;
    d.q_idx = q_idx; d.w = w; d.k_idx = k_idx;
    d.lkeys = sl.keys; d.lidx = sl.idx; d.lcount = sl.count; d.nlists = scan_grid(Lk);
    d.idx_out = idx_out;
    d.part = reinterpret_cast<float*>(base + L.part);
    d.n_chunks = decode_chunks(k);
    e = launch_decode_attend(d, st);
    if (e != hipSuccess || d.n_chunks == 1) return hip_status(e);
    return hip_status(launch_attn_merge(d.a, d.n_chunks, d.part, st));
  }
  // up to kScanHistTMax tokens the scan also builds the top-k's level-1 histogram
  const bool fused = T <= kScanHistTMax && topk_multi_block(Lk, T, k);
  hipError_t e = launch_index_scores(q_idx, w, k_idx, Lk, T, scores, ld, st, fused ? base : nullptr);
  if (e != hipSuccess) return DSA_ERR_HIP;
  e = launch_topk(scores, ld, Lk, T, k, idx, base, base + L.topk, st, fused);
  if (e != hipSuccess) return DSA_ERR_HIP;
  AttnArgs a{};
  a.q = q; a.k = k_cache; a.v = v_cache; a.n_rows = Lk;
  a.idx = idx; a.k_len = k; a.T = T;
  a.sink = sink; a.sm_scale = sm_scale; a.out = out; a.lse = lse;
  return hip_status(launch_sparse_attn(a, base + L.attn, st));
}

dsa_status dsa_decode_step_noalloc(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, const uint16_t* q,
                                   const uint16_t* k_cache, const uint16_t* v_cache, int64_t Lk, int32_t T, int32_t k,
                                   const float* sink, float sm_scale, uint16_t* out, float* lse, int32_t* idx_out,
                                   float* scores_out, int64_t ld_scores, void* stream) {
  // the same checks as dsa_decode_step, then the size limit, before any set-up
  dsa_status s = check_index_args(q_idx, w, k_idx, Lk, T);
  if (s != DSA_OK) return s;
  s = check_attn_args(q, k_cache, v_cache, out, sink, lse, sm_scale);
  if (s != DSA_OK) return s;
  if (T > DSA_DECODE_T_MAX || k < 1 || k > DSA_TOPK_MAX) return DSA_ERR_SHAPE;
  if ((idx_out && !aligned16(idx_out)) || (scores_out && !aligned16(scores_out))) return DSA_ERR_ALIGN;
  if (scores_out && ld_scores < Lk) return DSA_ERR_SHAPE;
  const size_t need = dsa_workspace_bytes(DSA_OP_DECODE_STEP, Lk, T, k, 0);
  if (need == 0 || need > (size_t)DSA_STATIC_SCRATCH_BYTES) return DSA_ERR_SCRATCH;
  void* ws = static_scratch();
  if (!ws) return DSA_ERR_HIP;
  // the scratch keeps whatever the last call left: the histogram path needs
  // its counter region cleared first (a fill kernel, so the call can be
  // captured); the list path reads nothing it did not write
  if (!use_list_path(Lk, T, k) && launch_zero(ws, kCounterRegionBytes, as_stream(stream)) != hipSuccess)
    return DSA_ERR_HIP;
  return dsa_decode_step(q_idx, w, k_idx, q, k_cache, v_cache, Lk, T, k, sink, sm_scale, out, lse, idx_out,
                         scores_out, ld_scores, ws, need, stream);
}

dsa_status dsa_cache_append(const uint16_t* idx_q, const uint16_t* idx_k, const float* ln_gamma,
                            const float* ln_beta, float ln_eps, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, int64_t Lk, int32_t T, int32_t rot_idx, int32_t rot_main,
                            double rope_base, uint8_t* q_idx_out, uint8_t* k_idx_cache, uint16_t* q_out,
                            uint16_t* k_cache, uint16_t* v_cache, void* stream) {
  const void* req[] = {idx_q, idx_k, q, k, v, q_idx_out, k_idx_cache, q_out, k_cache, v_cache};
  for (const void* ptr : req) {
    if (!ptr) return DSA_ERR_NULL;
    if (!aligned16(ptr)) return DSA_ERR_ALIGN;
  }
  if ((ln_gamma && !aligned16(ln_gamma)) || (ln_beta && !aligned16(ln_beta))) return DSA_ERR_ALIGN;
  if (T < 1 || T > 8192 || Lk < T || Lk >= kMaxLk) return DSA_ERR_SHAPE;
  if (rot_idx < 2 || rot_idx > DSA_IDX_DIM || (rot_idx & 1) || rot_main < 2 || rot_main > DSA_QK_DIM ||
      (rot_main & 1))
    return DSA_ERR_SHAPE;
  if (!(rope_base > 0.0) || !std::isfinite(rope_base) || !(ln_eps >= 0.f) || !std::isfinite(ln_eps))
    return DSA_ERR_SHAPE;
  return hip_status(launch_cache_append(idx_q, idx_k, ln_gamma, ln_beta, ln_eps, q, k, v, Lk, T, rot_idx,
                                        rot_main, rope_base, q_idx_out, k_idx_cache, q_out, k_cache, v_cache,
                                        as_stream(stream)));
}

dsa_status dsa_decode_batch(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, const uint16_t* q,
                            const uint16_t* k_cache, const uint16_t* v_cache, int64_t n_rows,
                            const int64_t* seq_start, const int32_t* seq_len, int32_t B, int32_t T,
                            int64_t max_len, int32_t k, const float* sink, float sm_scale, uint16_t* out,
                            float* lse, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  if (!q_idx || !w || !k_idx || !seq_start || !seq_len) return DSA_ERR_NULL;
  if (!aligned16(q_idx) || !aligned16(w) || !aligned16(k_idx) || !aligned16(seq_start) || !aligned16(seq_len))
    return DSA_ERR_ALIGN;
  dsa_status s = check_attn_args(q, k_cache, v_cache, out, sink, lse, sm_scale);
  if (s != DSA_OK) return s;
  if (idx_out && !aligned16(idx_out)) return DSA_ERR_ALIGN;
  if (B < 1 || B > 65535 || T < 1 || T > kBatchTMax || max_len < T || max_len >= kMaxLk || n_rows < 1 ||
      n_rows >= kMaxLk || k < 1 || k > DSA_TOPK_MAX)
    return DSA_ERR_SHAPE;
  const BatchLayout d = batch_layout(max_len, T, k, B);
  if (!ws || ws_bytes < d.total) return DSA_ERR_WORKSPACE;
  if (!aligned16(ws)) return DSA_ERR_ALIGN;
  hipStream_t st = as_stream(stream);
  char* base = static_cast<char*>(ws);
  float* scores = reinterpret_cast<float*>(base + d.scores);
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(base + d.idx);
  int32_t* rows = reinterpret_cast<int32_t*>(base + d.rows);
  SeqBatch sb;
  sb.start = seq_start;
  sb.len = seq_len;
  sb.n_rows = n_rows;
  sb.max_len = max_len;
  hipError_t e = launch_index_scores_batch(q_idx, w, k_idx, sb, B, T, scores, d.ld, st);
  if (e == hipSuccess) e = launch_topk_batch(scores, d.ld, sb, B, T, k, idx, rows, st);
  if (e == hipSuccess) {
    AttnArgs a{};
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.n_rows = n_rows;
    a.idx = rows;
    a.k_len = k;
    a.T = B * T;
    a.sink = sink;
    a.sm_scale = sm_scale;
    a.out = out;
    a.lse = lse;
    e = launch_sparse_attn(a, base + d.attn, st);
  }
  return hip_status(e);
}

dsa_status dsa_index_recall(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, int64_t Lk,
                            const int32_t* idx, int32_t T, int32_t k, float sm_scale, float* recall,
                            float* lse_dense, void* ws, size_t ws_bytes, void* stream) {
  if (!idx || !recall) return DSA_ERR_NULL;
  if (!aligned16(idx) || !aligned16(recall) || (lse_dense && !aligned16(lse_dense))) return DSA_ERR_ALIGN;
  // the output check needs a non-null pointer; the attention output lives in ws
  dsa_status s = check_attn_args(q, k_cache, v_cache, recall, nullptr, nullptr, sm_scale);
  if (s != DSA_OK) return s;
  if (T < 1 || T > 65535 || Lk < T || Lk >= kMaxLk || k < 1 || k > DSA_TOPK_MAX) return DSA_ERR_SHAPE;
  const RecallLayout d = recall_layout(Lk, T, k);
  if (!ws || ws_bytes < d.total) return DSA_ERR_WORKSPACE;
  if (!aligned16(ws)) return DSA_ERR_ALIGN;
  hipStream_t st = as_stream(stream);
  char* base = static_cast<char*>(ws);
  float* lse_sel = reinterpret_cast<float*>(base + d.lse);
  AttnArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.n_rows = Lk;
  a.idx = idx;
  a.k_len = k;
  a.T = T;
  a.sink = nullptr;
  a.sm_scale = sm_scale;
  a.out = reinterpret_cast<uint16_t*>(base + d.out);
  a.lse = lse_sel;
  hipError_t e = launch_sparse_attn(a, base + d.attn, st);
  if (e == hipSuccess)
    e = launch_index_recall(q, k_cache, Lk, T, sm_scale, lse_sel, reinterpret_cast<float*>(base + d.part), recall,
                            lse_dense, st);
  return hip_status(e);
}

dsa_status dsa_prefill_topk(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t Lk, int32_t T,
                            int32_t k, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  dsa_status s = check_index_args(q_idx, w, k_idx, Lk, T);
  if (s != DSA_OK) return s;
  if (!idx) return DSA_ERR_NULL;
  if (!aligned16(idx)) return DSA_ERR_ALIGN;
  if (k < 1 || k > DSA_TOPK_MAX) return DSA_ERR_SHAPE;
  const PrefillLayout d = prefill_layout(Lk, T);
  if (!ws || ws_bytes < d.total) return DSA_ERR_WORKSPACE;
  if (!aligned16(ws)) return DSA_ERR_ALIGN;
  hipStream_t st = as_stream(stream);
  char* base = static_cast<char*>(ws);
  float* sample = reinterpret_cast<float*>(base + d.sample);
  uint32_t* theta = reinterpret_cast<uint32_t*>(base + d.theta);
  uint32_t* count = reinterpret_cast<uint32_t*>(base + d.count);
  uint32_t* nfail = count + T;
  uint32_t* failed = reinterpret_cast<uint32_t*>(base + d.failed);
  PrefillCand pc{theta, count, reinterpret_cast<uint2*>(base + d.cand), kPrefillCap};
  pc.cw = reinterpret_cast<float*>(base + d.cw);
  pc.knorm = reinterpret_cast<float*>(base + d.knorm);
  hipError_t e = launch_zero(count, align_up(((size_t)T + 4) * sizeof(uint32_t)), st);
  if (e == hipSuccess) e = launch_key_norms(k_idx, Lk, const_cast<float*>(pc.knorm), st);
  if (e == hipSuccess) e = launch_idx_gemm_sample(q_idx, w, k_idx, Lk, T, kPrefillStep, sample, d.ld_sample, st);
  if (e == hipSuccess)
    e = launch_prefill_theta(sample, d.ld_sample, q_idx, w, Lk, T, kPrefillStep, k, kPrefillCap, theta,
                             const_cast<float*>(pc.cw), st);
  if (e == hipSuccess) e = launch_idx_gemm_cand(q_idx, w, k_idx, Lk, T, pc, st);
  if (e == hipSuccess) e = launch_prefill_rescore(pc, q_idx, w, k_idx, T, st);
  if (e == hipSuccess) e = launch_prefill_refine(pc, Lk, T, k, idx, nfail, failed, st);
  // rows whose candidates did not fit or did not hold their top-k: recomputed
  // exactly on the device (the launch ends at once when there are none)
  if (e == hipSuccess)
    e = launch_prefill_fallback(q_idx, w, k_idx, Lk, T, k, nfail, failed, reinterpret_cast<float*>(base + d.fb),
                                d.ld_fb, d.fb_blocks, idx, st);
  return hip_status(e);
}

}  // extern "C"
