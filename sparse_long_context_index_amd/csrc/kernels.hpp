// kernels.hpp -- launchers of the HIP kernels (internal to libdsa.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

constexpr int kDecodeTMax = 8;            // streaming-scan limit of the indexer
constexpr int kScanHistTMax = 4;          // the scan also builds the top-k histogram up to here
constexpr int kTopkMultiRowsMax = 8;      // rows handled by the multi-block top-k

constexpr int kListM = 32;                // per-workgroup local top list of the decode scan
constexpr int kScanListTMax = 4;          // query rows the list scan (and the fused decode step) serves

// A batch of ragged sequences over shared caches: sequence b owns cache rows
// start[b] .. start[b] + len[b] - 1 (its history and its T new tokens).  A
// sequence whose length lies outside [0, max_len] or whose rows leave
// [0, n_rows) is treated as empty.
struct SeqBatch {
  const int64_t* start = nullptr;   // [B] device
  const int32_t* len = nullptr;     // [B] device
  int64_t n_rows = 0;
  int64_t max_len = 0;
  int32_t spread = 0;               // the batch scan: B when its workgroups are dealt by length (B <= 256)
  // the batch scan over a group of a sequence's tokens: tstride tokens per
  // sequence in the query, weight and score layouts (0: the launch's T), and
  // `tail` more tokens after the group (its keys end tail rows before the
  // sequence's last)
  int32_t tstride = 0;
  int32_t tail = 0;
};

// keys of sequence b (0 when its descriptor is invalid); *first receives its first row
__device__ __forceinline__ int64_t seq_keys(const SeqBatch& sb, int b, int64_t* first) {
  const int64_t s = sb.start[b];
  const int64_t n = sb.len[b];
  const bool ok = n >= 0 && n <= sb.max_len && s >= 0 && s + n <= sb.n_rows;
  *first = ok ? s : 0;
  return ok ? n : 0;
}

// ---- index scores
// Per-workgroup local top lists of the decode scan.  Entry j of workgroup b's
// list for row t sits at [(t * kListM + j) * scan_grid + b]; entries are in
// (score desc, index asc) order, unused entries have key 0.
struct ScanLists {
  uint32_t* keys = nullptr;    // [T][kListM][scan_grid] order keys
  uint32_t* idx = nullptr;     // [T][kListM][scan_grid] key indices
  uint32_t* count = nullptr;   // [T][scan_grid] kept | (more than kListM visible) << 31
  bool store_scores = true;    // also write the scores (else the selection recomputes them if it must)
};
int scan_grid(int64_t Lk);     // workgroups of the decode scan
int scan_list_cap(int64_t Lk); // keys a workgroup of the scan without lists scores per row (at most)
size_t scan_lds_bytes(int64_t Lk, int T, bool lists);   // dynamic LDS of the decode scan
// topk_counters: optional workspace counter region; when given (T <=
// kScanHistTMax) the scan also builds the top-k's level-1 histogram there.
// lists: optional per-workgroup local top lists (exclusive with the histogram).
hipError_t launch_index_scores(const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                               int64_t Lk, int T, float* scores, int64_t ld, hipStream_t st,
                               void* topk_counters = nullptr, ScanLists lists = ScanLists{});
// scores of B sequences at once: q_idx [B][T][16][128], w [B][T][16], scores
// [B][T][ld] (ld >= max_len); row (b, t) sees keys 0 .. len[b] - T + t of its
// sequence.  T <= 8 takes the streaming scan, larger T the contraction.
hipError_t launch_index_scores_batch(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, const SeqBatch& sb,
                                     int B, int T, float* scores, int64_t ld, hipStream_t st);

// ---- top-k
size_t topk_scratch_bytes(int64_t Lk, int T, int k);
bool topk_multi_block(int64_t Lk, int T, int k);   // few long rows: the multi-block path
// hist_ready: the level-1 histogram of these scores is already in the counter
// region (built by the scan); otherwise launch_topk builds it first.
hipError_t launch_topk(const float* scores, int64_t ld, int64_t Lk, int T, int k, int32_t* idx,
                       void* ws_counters, void* scratch, hipStream_t st, bool hist_ready = false);
// top-k of the B * T rows of a batch ([B][T][ld] scores): idx [B][T][k]
// positions within each sequence, idx_rows the same as cache rows (-1 kept)
hipError_t launch_topk_batch(const float* scores, int64_t ld, const SeqBatch& sb, int B, int T, int k, int32_t* idx,
                             int32_t* idx_rows, hipStream_t st);

// ---- gathered attention
struct AttnArgs {
  const uint16_t* q;       // [units_t][64][192]
  const uint16_t* k;       // [rows][Hkv][192]
  const uint16_t* v;       // [rows][Hkv][128]
  int64_t n_rows;          // rows of k / v
  // index source: explicit list (idx != nullptr) or a window per sequence
  const int32_t* idx;      // [T][k]
  int k_len;               // entries per idx row
  const int64_t* seq_start;  // [B]
  const int32_t* seq_len;    // [B]
  int window;
  int T;                   // query tokens (DSA) or sequences (SWA)
  const float* sink;       // [64] or null
  float sm_scale;
  uint16_t* out;           // [T][64][128]
  float* lse;              // [T][64] or null
};
size_t attn_scratch_bytes(int T, int k_len, int hkv);
hipError_t launch_sparse_attn(const AttnArgs& a, void* scratch, hipStream_t st);
hipError_t launch_swa_attn(const AttnArgs& a, void* scratch, hipStream_t st);
// merge of per-chunk partials [(t * 4 + g) * n_chunks + c] of the GQA-4 attention, with the sink
hipError_t launch_attn_merge(const AttnArgs& a, int n_chunks, const float* part, hipStream_t st);

// ---- fused decode tail: selection from the scan's lists + attention (partials
// merged by launch_attn_merge when there is more than one chunk)
struct DecodeArgs {
  AttnArgs a;                  // q, k, v, n_rows = Lk, T, sink, sm_scale, out, lse
  const float* scores;         // [T][ld] (re-selection when the lists may miss a winner)
  int64_t ld;
  float* rescore;              // null, or [T][ld]: the scan stored no scores, the re-selection recomputes them here
  const uint8_t* q_idx;        // the scan's inputs, for the recomputation
  const float* w;
  const uint8_t* k_idx;
  int64_t Lk;
  int k;
  const uint32_t* lkeys;       // scan lists (ScanLists layout)
  const uint32_t* lidx;
  const uint32_t* lcount;
  int nlists;                  // scan workgroups
  int32_t* idx_out;            // [T][k] or null
  float* part;                 // [T][4][n_chunks] partials
  int n_chunks;
};
int decode_chunks(int k);
hipError_t launch_decode_attend(const DecodeArgs& d, hipStream_t st);

// ---- prefill contraction of the index scores (T > 8; any T >= 1 works)
hipError_t launch_idx_gemm(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t Lk, int T,
                           float* scores, int64_t ld, hipStream_t st);
// the same for the B sequences of a batch (grid dimension y = sequence)
hipError_t launch_idx_gemm_batch(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, const SeqBatch& sb,
                                 int B, int T, float* scores, int64_t ld, hipStream_t st);
// scores of the sampled keys 0, step, 2 step, ...: column j of a row is key j * step
hipError_t launch_idx_gemm_sample(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t Lk, int T,
                                  int step, float* scores, int64_t ld, hipStream_t st);
// candidate emission: every visible key whose order key reaches theta[t] is
// appended to row t's slots as (order key, index); count[t] counts them all
// (slots past cap are not written)
// A key s is a candidate of row t when the contraction's score plus
// cw[t] * knorm[s] reaches theta[t]: cw[t] bounds, per unit of key norm, how
// far the contraction's score of row t can lie from the exact one (see the
// fused prefill top-k), knorm[s] bounds the key's norm.
constexpr int kPrefillTileKeys = 2048;
struct PrefillCand {
  const uint32_t* theta;   // [T]
  uint32_t* count;         // [T], zero before the launch
  uint2* cand;             // [T][cap]
  int cap;
  const float* cw = nullptr;     // [T]
  const float* knorm = nullptr;  // [Lk]
};
hipError_t launch_idx_gemm_cand(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t Lk, int T,
                                const PrefillCand& pc, hipStream_t st);

// ---- fused prefill top-k (prefill_topk.hip)
constexpr int kPrefillStep = 64;           // key sample stride of the threshold estimate
constexpr int kPrefillCap = 12288;         // candidate slots per row
constexpr int kPrefillFallbackBlocks = 64; // workgroups (and score rows of workspace) of the exact fallback
size_t prefill_refine_lds(int cap);
// knorm[s]: an upper bound of the Euclidean norm of key s
hipError_t launch_key_norms(const uint8_t* k_idx, int64_t Lk, float* knorm, hipStream_t st);
// theta[t]: order key of the row's threshold (0: every visible key); cw[t]:
// the row's error factor (|u| with u_d = sum_h |w[t,h]| |q_idx[t,h,d]|, times
// the relative error bound of the contraction, rounded up)
hipError_t launch_prefill_theta(const float* sample, int64_t ld, const uint8_t* q_idx, const float* w, int64_t Lk,
                                int T, int step, int k, int cap, uint32_t* theta, float* cw, hipStream_t st);
// the candidates' order keys recomputed with the exact index arithmetic (in place)
hipError_t launch_prefill_rescore(const PrefillCand& pc, const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                                  int T, hipStream_t st);
// exact top-k of each row from its candidates into idx [T][k]; rows whose
// candidates do not fit, or of which fewer than min(k, visible) reach the
// row's threshold, are appended to failed (nfail counts)
hipError_t launch_prefill_refine(const PrefillCand& pc, int64_t Lk, int T, int k, int32_t* idx, uint32_t* nfail,
                                 uint32_t* failed, hipStream_t st);
// the listed rows (failed[0 .. *nfail)) recomputed exactly: scores of every
// visible key into buf ([blocks][ld] floats), then the row top-k (topk.hip)
hipError_t launch_prefill_fallback(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t Lk, int T,
                                   int k, const uint32_t* nfail, const uint32_t* failed, float* buf, int64_t ld,
                                   int blocks, int32_t* idx, hipStream_t st);

// ---- index-selection recall (recall.hip)
int recall_chunks(int64_t Lk);
// part: [T][4][recall_chunks(Lk)][32] floats; lse_sel [T][64] from the
// gathered attention without sink; lse_dense optional
hipError_t launch_index_recall(const uint16_t* q, const uint16_t* k, int64_t Lk, int T, float sm_scale,
                               const float* lse_sel, float* part, float* recall, float* lse_dense, hipStream_t st);

// ---- cache append (LayerNorm / partial RoPE / fp8 of the indexer, RoPE of attention q, k)
hipError_t launch_cache_append(const uint16_t* idx_q, const uint16_t* idx_k, const float* ln_gamma,
                               const float* ln_beta, float ln_eps, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, int64_t Lk, int T, int rot_idx, int rot_main, double base,
                               uint8_t* q_idx_out, uint8_t* k_idx_cache, uint16_t* q_out, uint16_t* k_cache,
                               uint16_t* v_cache, hipStream_t st);

// ---- workspace
hipError_t launch_zero(void* p, size_t bytes, hipStream_t st);

}  // namespace dsa
