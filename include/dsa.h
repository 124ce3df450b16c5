/*
 * dsa.h -- C ABI of libdsa.so: the single-GPU hot path of a DeepSeek-Sparse-
 * Attention (DSA) layer and of a sliding-window (SWA) layer, built for AMD
 * Instinct MI355X (gfx950).
 *
 * Citation keys (web pages about the Naive-N0.5-Flash release):
 *   [NoFA]   "Naive-N0.5-Flash: no full-attention layers, and a runtime built
 *            by AI" (ai.thesatyajit.com) -- property table; section "What 'no
 *            full-attention layers' means"; section "Inside a DSA layer: the
 *            lightning indexer" and its Figure 1; section "The runtime is the
 *            actual claim"; section "How much of this did AI actually build?".
 *   [Master] "Naive-N0.5-Flash: the open-weight 309B MoE with no full-attention
 *            layers at all aims for 2,000 tokens/s per user" (ai-master.dev),
 *            section "Zero full-attention: what it really changes".
 *   [Reading] "2,122 tok/s, Zero Full-Attention Layers: Reading
 *            Naive-N0.5-Flash Carefully" (sheldonwangrjt.github.io), section
 *            "The 42x footnote".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors) unless a
 *   parameter says otherwise.  `stream` is a hipStream_t passed as void*; NULL
 *   means the default stream.  Every call only enqueues work on `stream` and
 *   returns without synchronising (so every call can be captured into a HIP
 *   graph); outputs are ready when the stream reaches that point.
 * - Index-score arithmetic.  Every selection (dsa_decode_step,
 *   dsa_decode_batch, dsa_prefill_topk) is made on EXACT index scores: fp8
 *   bytes widened losslessly to bf16, exact products, float32 sums of the 128
 *   terms and of the 16 weighted heads (error at most 2e-5 of
 *   sum_h |w_h| sum_d |q_hd k_d|), the same bits on every path.
 *   dsa_index_scores returns those scores for T <= 8; for T > 8 it returns
 *   the fp8 MFMA contraction's scores, whose error is at most
 *   (2^-10 + 4e-5) sum_h |w_h| sum_d |q_hd k_d| (the matrix cores add each
 *   group of 8 fp8 products after aligning them to the group's largest
 *   exponent, keeping at least 13 fraction bits below it).
 * - Ownership: the caller owns every buffer.  The library never allocates or
 *   frees memory on a call path.  Scratch space is the caller's workspace `ws`
 *   of at least dsa_workspace_bytes() bytes (see the workspace contract
 *   below); the one exception, dsa_decode_step_noalloc, uses a static device
 *   array per GPU instead, the library's only global mutable state.
 * - Layouts are dense, row-major, C order, with the shapes given per call.
 *   fp8 values are OCP E4M3FN bytes; bf16 values are raw 16-bit patterns.
 * - Alignment: every pointer must be 16-byte aligned (torch gives 256 B).
 * - Query positions: T query tokens are the LAST T of Lk cached tokens, so
 *   query t (0 <= t < T) sits at position p_t = Lk - T + t and sees keys
 *   [0, p_t] (causal, including itself; [NoFA] Figure 1 "index sweep over all
 *   visible keys").
 * - Errors: arguments are validated on the host before anything is enqueued;
 *   on a validation failure nothing is launched and outputs are untouched.  A
 *   failed launch returns DSA_ERR_HIP.  Faults inside kernels surface at the
 *   caller's next synchronisation.  No C++ exception crosses the ABI.
 * - Outputs are fully overwritten (never accumulated).  Results are bitwise
 *   deterministic: the same inputs give the same bits on every run.
 *
 * Workspace contract
 * ------------------
 * Calls that take `ws` use it for histograms, per-block candidate lists,
 * split-softmax partials and completion counters.  A fresh workspace must be
 * prepared ONCE with dsa_workspace_init() (it zero-fills the counter region
 * on `stream`); every call leaves the counter region zeroed again when its
 * work completes, so a workspace can be reused by any sequence of calls on one
 * stream.  Calls that overlap in time (e.g. on two streams) need separate
 * workspaces.  If a call's kernels fault, re-initialise the workspace.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Fixed model constants ([NoFA] property table: index_n_heads, the single
 * fp8 index-key head, num_attention_heads, head_dim / v head dim,
 * num_key_value_heads (DSA) and swa_num_key_value_heads, index_top_k,
 * sliding_window). */
#define DSA_IDX_HEADS 16
#define DSA_IDX_DIM 128
#define DSA_Q_HEADS 64
#define DSA_QK_DIM 192
#define DSA_V_DIM 128
#define DSA_KV_HEADS 4
#define SWA_KV_HEADS 8
#define DSA_TOPK_MAX 2048
#define SWA_WINDOW_DEFAULT 128
#define SWA_WINDOW_MAX 2048
#define DSA_DECODE_T_MAX 8

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_NULL = 1,        /* a required pointer is NULL                      */
  DSA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent          */
  DSA_ERR_UNSUPPORTED = 3, /* a valid request this build does not implement   */
  DSA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                */
  DSA_ERR_WORKSPACE = 5,   /* ws is NULL or smaller than dsa_workspace_bytes  */
  DSA_ERR_HIP = 6,         /* the HIP runtime reported an error at launch     */
  DSA_ERR_SCRATCH = 7      /* the request needs more than the static scratch  */
} dsa_status;

typedef enum dsa_op {
  DSA_OP_INDEX_SCORES = 0,
  DSA_OP_TOPK = 1,
  DSA_OP_SPARSE_ATTN = 2,
  DSA_OP_SWA_ATTN = 3,
  DSA_OP_DECODE_STEP = 4,
  DSA_OP_PREFILL_TOPK = 5,
  DSA_OP_DECODE_BATCH = 6,
  DSA_OP_INDEX_RECALL = 7
} dsa_op;

/*
 * dsa_index_scores -- lightning-indexer scores ([NoFA] "Inside a DSA layer":
 * 16 fp8 query heads against one shared fp8 key head, ReLU of the dot
 * product, combined into one score per key by per-head weights):
 *
 *   S[t,s] = sum_{h<16} w[t,h] * max( sum_{d<128} q_idx[t,h,d] * k_idx[s,d], 0 )
 *            for s <= p_t,   S[t,s] = -inf for p_t < s < Lk.
 *
 *   q_idx   [T][16][128] fp8 e4m3   (2 KiB per query token)
 *   w       [T][16] float32
 *   k_idx   [Lk][128] fp8 e4m3      (key s at byte offset 128*s)
 *   scores  [T][ld_scores] float32, ld_scores >= Lk; columns >= Lk untouched.
 *
 * Precision depends on T (see "Index-score arithmetic" above): T <= 8 runs the
 * streaming scan (decode) with exact fp8 products and float32 sums; T > 8 runs
 * the fp8 MFMA contraction (prefill), whose sums drop low-order bits (bound
 * (2^-10 + 4e-5) sum_h |w_h| sum_d |q_hd k_d| per score).  To score many rows
 * exactly, call it on groups of at most 8 consecutive rows (group [r0, r1)
 * with Lk - (T - r1) keys).  Limits: 1 <= T <= Lk < 2^31.
 */
dsa_status dsa_index_scores(const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                            int64_t Lk, int32_t T, float* scores, int64_t ld_scores,
                            void* stream);

/*
 * dsa_topk -- per query row, the min(k, p_t + 1) visible keys with the
 * largest scores, ties broken towards the lower key index ([NoFA] "What 'no
 * full-attention layers' means": first index_top_k entries of a descending
 * argsort; "How much of this did AI actually build?": stable ties).
 *
 *   scores  [T][ld_scores] float32; only columns [0, p_t] of row t are read.
 *   idx     [T][k] int32 output: the kept key indices in ASCENDING order,
 *           padded with -1 when p_t + 1 < k.
 *
 * -0.0 and +0.0 compare equal.  NaN scores are outside the contract.
 * Limits: 1 <= k <= 2048, 1 <= T <= Lk < 2^31.  Needs ws (DSA_OP_TOPK).
 */
dsa_status dsa_topk(const float* scores, int64_t ld_scores, int64_t Lk, int32_t T, int32_t k,
                    int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/*
 * sparse_gqa_attn -- gathered GQA-4 attention with an optional sink
 * ([NoFA] "Inside a DSA layer": the main heads attend only to the selected
 * keys, everything else masked before the softmax; GQA with 4 KV heads on DSA
 * layers; a sink column per head.  [Master]: sink bias on both attention
 * types).  For query token t, head h < 64, KV head g = h / 16:
 *
 *   z_j    = sm_scale * <q[t,h,:], k_cache[j,g,:]>      for every j in idx[t]
 *   out    = sum_j e^{z_j} v_cache[j,g,:] / (sum_j e^{z_j} + e^{sink[h]})
 *   lse    = ln(sum_j e^{z_j} + e^{sink[h]})
 *
 * (the sink terms vanish when sink == NULL; the sink is NOT multiplied by
 * sm_scale).
 *
 *   q        [T][64][192] bf16
 *   k_cache  [Lk][4][192] bf16,  v_cache [Lk][4][128] bf16
 *   idx      [T][k] int32; entries outside [0, Lk) (e.g. -1 padding) are empty
 *            slots and are skipped.  Entries must be distinct within a row;
 *            causality is the caller's business (idx from dsa_topk is causal).
 *   sink     [64] float32 or NULL
 *   out      [T][64][128] bf16 (fp32 accumulation, round-to-nearest-even)
 *   lse      [T][64] float32 or NULL (natural log; -inf for an empty row
 *            without sink)
 *
 * An empty row gives out = 0.  Limits: 1 <= k <= 2048, 1 <= T, Lk < 2^31.
 * Needs ws (DSA_OP_SPARSE_ATTN).
 */
dsa_status sparse_gqa_attn(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                           int64_t Lk, const int32_t* idx, int32_t T, int32_t k,
                           const float* sink, float sm_scale, uint16_t* out, float* lse,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * swa_attn -- single-token sliding-window decode for a ragged batch, GQA-8
 * ([NoFA] "What 'no full-attention layers' means": the SWA path keeps keys
 * whose offset from the query is below sliding_window = 128, the query itself
 * included).  Sequence b has seq_len[b] = n_b >= 1 tokens stored at rows
 * [seq_start[b], seq_start[b] + n_b) of the ragged caches; its query is the
 * token at position n_b - 1 and attends to positions
 * [max(0, n_b - window), n_b - 1].  Head h uses KV head h / 8.  The formula is
 * the one of sparse_gqa_attn over that index set.
 *
 *   q          [B][64][192] bf16
 *   k_cache    [n_rows][8][192] bf16,  v_cache [n_rows][8][128] bf16
 *   seq_start  [B] int64 (device),  seq_len [B] int32 (device)
 *   sink       [64] float32 or NULL
 *   out        [B][64][128] bf16,  lse [B][64] float32 or NULL
 *
 * Rows outside [0, n_rows) are never read: a window row outside the cache is
 * skipped (a sequence with n_b <= 0 is empty).  Limits: 1 <= B,
 * 1 <= window <= 2048.  Needs ws (DSA_OP_SWA_ATTN).
 */
dsa_status swa_attn(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                    int64_t n_rows, const int64_t* seq_start, const int32_t* seq_len, int32_t B,
                    int32_t window, const float* sink, float sm_scale, uint16_t* out, float* lse,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * dsa_decode_step -- one DSA decode (or speculative-verify) step, fused:
 * index scores -> top-k -> sparse GQA-4 attention, with no host round trip
 * ([NoFA] Figure 1, the order of one DSA module).  Arguments are those of the
 * three calls above; idx_out ([T][k] int32) optionally receives the selected
 * set; scores_out ([T][ld_scores] float32) optionally receives the scores.
 * Without scores_out the step may store no scores at all (the results are the
 * same; only a rare slow re-selection then recomputes them in ws), so asking
 * for them costs time.
 * Limits: 1 <= T <= 8, 1 <= k <= 2048.  Needs ws (DSA_OP_DECODE_STEP).
 */
dsa_status dsa_decode_step(const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                           const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                           int64_t Lk, int32_t T, int32_t k, const float* sink, float sm_scale,
                           uint16_t* out, float* lse, int32_t* idx_out,
                           float* scores_out, int64_t ld_scores,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * dsa_decode_step_noalloc -- dsa_decode_step without a caller workspace and
 * without any allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Arguments, results and bits are those of dsa_decode_step.
 *
 * Scratch: a static device array of DSA_STATIC_SCRATCH_BYTES (64 MiB) per GPU,
 * held from the library's first use on that GPU until the process ends; its
 * address is looked up at the first call on each device, with that device
 * current.  Every call on a GPU shares that GPU's array, which keeps the last
 * call's contents: a call clears on `stream` what it needs zeroed (the
 * counter region, on the histogram path taken for T > 4), so calls in
 * sequence are independent, but calls that overlap in time on one GPU (two
 * streams, two threads) race and must be serialised by the caller.  A request
 * whose workspace (dsa_workspace_bytes(DSA_OP_DECODE_STEP, Lk, T, k, 0))
 * exceeds the array returns DSA_ERR_SCRATCH before anything is enqueued
 * (about 15 M keys for T = 1, 1.2 M keys for T = 8).
 */
#define DSA_STATIC_SCRATCH_BYTES (64u << 20)
dsa_status dsa_decode_step_noalloc(const uint8_t* q_idx, const float* w, const uint8_t* k_idx,
                                   const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                                   int64_t Lk, int32_t T, int32_t k, const float* sink, float sm_scale,
                                   uint16_t* out, float* lse, int32_t* idx_out,
                                   float* scores_out, int64_t ld_scores, void* stream);

/*
 * dsa_decode_batch -- dsa_decode_step for B sequences of different lengths
 * at once, T query tokens each (serving many users, T = 1: [Reading] "The
 * 42x footnote" on the Standard-mode figure; the verify step of a
 * speculative round, T up to 16: [NoFA] "The runtime is the actual claim").  The sequences share one index-key cache and one K/V
 * cache: sequence b owns rows seq_start[b] .. seq_start[b] + seq_len[b] - 1,
 * its history followed by its T new tokens, so its token t sits at position
 * seq_len[b] - T + t and sees the sequence's keys 0 .. seq_len[b] - T + t.
 *
 *   q_idx [B][T][16][128] fp8, w [B][T][16] f32, q [B][T][64][192] bf16
 *   k_idx [n_rows][128] fp8, k_cache [n_rows][4][192], v_cache [n_rows][4][128] bf16
 *   seq_start [B] int64, seq_len [B] int32   (device arrays)
 *   max_len   an upper bound of every seq_len (sizes the workspace)
 *   out [B][T][64][128] bf16, lse [B][T][64] f32 (optional)
 *   idx_out   [B][T][k] int32 (optional): positions within each sequence,
 *             ascending, -1 padded
 *
 * Each row's selection is the top-k rule of dsa_topk over its own exact
 * scores, and its attention that of sparse_gqa_attn over the selected rows.
 * A sequence with seq_len outside [0, max_len] or rows outside [0, n_rows) is
 * treated as empty (its outputs are those of an empty selection).  The scores
 * come from the streaming scan per sequence; T > 8 scans the keys once per
 * group of 8 tokens.
 * Limits: 1 <= B <= 65535, 1 <= T <= 16, T <= max_len < 2^31, n_rows < 2^31,
 * 1 <= k <= 2048.  Needs ws (DSA_OP_DECODE_BATCH with Lk = max_len).
 */
dsa_status dsa_decode_batch(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, const uint16_t* q,
                            const uint16_t* k_cache, const uint16_t* v_cache, int64_t n_rows,
                            const int64_t* seq_start, const int32_t* seq_len, int32_t B, int32_t T,
                            int64_t max_len, int32_t k, const float* sink, float sm_scale, uint16_t* out,
                            float* lse, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);

/*
 * dsa_index_recall -- how much of dense attention an index set keeps ([NoFA]
 * "How much of this did AI actually build?": the indexer's top-k was checked
 * against a full-attention reference).  For every query token t and head h:
 *
 *   recall[t,h] = sum_{j in idx[t]} e^{z_j} / sum_{j <= p_t} e^{z_j},
 *   z_j = sm_scale * <q[t,h], k_cache[j, h / 16]>   (no sink on either side)
 *
 *   q [T][64][192], k_cache [Lk][4][192], v_cache [Lk][4][128] bf16 (v is
 *   read for the selected rows only); idx [T][k] as dsa_topk writes it;
 *   recall [T][64] f32; lse_dense [T][64] f32 (optional): log of the
 *   denominator.  An empty set has recall 0.
 * The numerator comes from the gathered attention over idx, the denominator
 * from a QK-only pass over every visible key (Lk * 1.5 KiB of K per token).
 * Limits: 1 <= T <= min(Lk, 65535), Lk < 2^31, 1 <= k <= 2048.  Needs ws
 * (DSA_OP_INDEX_RECALL).
 */
dsa_status dsa_index_recall(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, int64_t Lk,
                            const int32_t* idx, int32_t T, int32_t k, float sm_scale, float* recall,
                            float* lse_dense, void* ws, size_t ws_bytes, void* stream);

/*
 * dsa_prefill_topk -- index scores and top-k for many query rows (the
 * prefill chunk) without writing the [T][Lk] score matrix ([NoFA] "Inside a
 * DSA layer": every visible key is scored and the top index_top_k kept; "What
 * 'no full-attention layers' means": a stable descending argsort).
 * idx [T][k] int32 receives, per row, the min(k, p_t+1) best keys by
 * (exact score desc, index asc) in ascending index order, -1 padded -- the
 * same set, element for element, as dsa_topk over the exact scores
 * (dsa_index_scores on groups of at most 8 rows).
 *
 * Internally the fp8 MFMA contraction only locates candidates: scores of
 * every 64th key give each row a threshold theta; one pass over all keys
 * (fp8 logits, head sums on the bf16 matrix cores) keeps the keys whose
 * approximate score reaches theta minus the largest error that score can
 * have (bounded per key from the row's query and weights, the key's norm and
 * the pass's own sum of |weight| x rounded ReLU logit), up to 12,288 per
 * row; the candidates are
 * re-scored exactly and the top-k selected from them once at least min(k,
 * p_t+1) of them reach theta (then no key left out can belong).  A row that
 * fails this is recomputed exactly on the device, so the result never
 * depends on the threshold.  Nothing is read back to the host.
 * Limits: 1 <= T <= Lk < 2^31, 1 <= k <= 2048.  Needs ws (DSA_OP_PREFILL_TOPK,
 * about T * (Lk / 16 + 96 KiB) + (min(T, 64) + 1) * Lk * 4 bytes).
 */
dsa_status dsa_prefill_topk(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t Lk, int32_t T,
                            int32_t k, int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/*
 * dsa_cache_append -- the step before the index sweep for T new tokens at
 * positions p_t = Lk - T + t ([NoFA] "Inside a DSA layer" and Figure 1, panel
 * B: the index key is layer-normalised, rotated by partial RoPE and rounded to
 * fp8; the index queries are rotated and rounded to fp8; the attention
 * queries and keys are rotated (RoPE on a third of each head, rope base
 * 10,000,000 on the sparse layers, same section); keys and values are
 * appended to the cache):
 *
 *   idx_k' = rope(LayerNorm(idx_k) * ln_gamma + ln_beta, p)  -> fp8 -> k_idx_cache[p]
 *   idx_q' = rope(idx_q, p)                                   -> fp8 -> q_idx_out
 *   q'     = rope(q, p)                                       -> bf16 -> q_out
 *   k'     = rope(k, p)                                       -> bf16 -> k_cache[p]
 *   v                                                         -> v_cache[p]
 *
 * rope(x, p) rotates the first R dims of every head, pairing dim i with dim
 * i + R/2: x_i cos a_i - x_{i+R/2} sin a_i and x_{i+R/2} cos a_i + x_i sin a_i,
 * a_i = p * rope_base^(-2i/R); the angles are formed in float64 at the
 * absolute position ("How much of this did AI actually build?" reports
 * precision issues in positional encoding).  Dims >= R pass through.
 *
 *   idx_q        [T][16][128] bf16   index query heads (post-projection)
 *   idx_k        [T][128] bf16       index key
 *   ln_gamma, ln_beta [128] float32  LayerNorm gain and bias (NULL: 1 and 0)
 *   ln_eps       LayerNorm epsilon (>= 0)
 *   q            [T][64][192] bf16   attention queries
 *   k, v         [T][4][192], [T][4][128] bf16  attention keys and values
 *   rot_idx, rot_main  rotated dims of the 128- and 192-dim heads (even,
 *                      0 < R <= head dim; the pages' third: 42 and 64)
 *   rope_base    > 0 (DSA_ROPE_BASE for the sparse layers)
 *   q_idx_out    [T][16][128] fp8    the scan's query (dsa_index_scores q_idx)
 *   k_idx_cache  [Lk][128] fp8       rows Lk-T .. Lk-1 written
 *   q_out        [T][64][192] bf16
 *   k_cache      [Lk][4][192] bf16   rows Lk-T .. Lk-1 written
 *   v_cache      [Lk][4][128] bf16   rows Lk-T .. Lk-1 written
 *
 * fp8 results round to nearest even after clamping to +-448; bf16 results
 * round to nearest even.  Arithmetic is float32 (LayerNorm moments float64).
 * Limits: 1 <= T <= Lk < 2^31, T <= 8192.  Needs no workspace.
 */
#define DSA_ROPE_BASE 10000000.0
dsa_status dsa_cache_append(const uint16_t* idx_q, const uint16_t* idx_k, const float* ln_gamma,
                            const float* ln_beta, float ln_eps, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, int64_t Lk, int32_t T, int32_t rot_idx, int32_t rot_main,
                            double rope_base, uint8_t* q_idx_out, uint8_t* k_idx_cache, uint16_t* q_out,
                            uint16_t* k_cache, uint16_t* v_cache, void* stream);

/* Workspace bytes needed by `op` for the given sizes (B is the SWA batch; the
 * other sizes are ignored where they do not apply).  Returns 0 for an invalid
 * request.  Sizes are upper bounds: a workspace sized for (Lk, T, k, B) serves
 * every call with smaller sizes of the same op. */
size_t dsa_workspace_bytes(dsa_op op, int64_t Lk, int32_t T, int32_t k, int32_t B);

/* Prepare a fresh workspace (zero-fills its counter region) on `stream`. */
dsa_status dsa_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Static, human-readable name of a status code. */
const char* dsa_status_string(dsa_status s);

/* Library version string, e.g. "dsa-mi355x 0.1.0 gfx950". */
const char* dsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
