/* spec_verify.h -- batched speculative-sampling verification on AMD Instinct MI355X (gfx950).
 *
 * One speculative round per request: the draft proposed y_1..y_g from q_1..q_g, the target
 * scored p_1..p_{g+1} in one forward pass.  The library turns the logit rows into the
 * tempered, top-k/top-p-filtered distributions, accepts y_i with probability
 * min(1, p_i(y_i)/q_i(y_i)) (or by argmax equality when greedy), stops at the first
 * rejection, draws the correction token from the residual [p_i - q_i]_+ / sum [p_i - q_i]_+
 * or a bonus token from p_{g+1}, and emits per-position draft entropy, draft max-probability
 * and 1 - TV(p, q).
 *
 * Sources: the guide page "5.1 投机解码核心原理" (speculative decoding: core principles),
 * sections 2.1-2.2 (inputs), 3.1 (greedy rule), 3.2 (acceptance ratio, residual formula),
 * 3.3 (token-only drafts), 4.1-4.3 (beta = sum [p-q]_+ = 1 - A, A = 1 - TV), 5.1-5.2 (first
 * rejection, bonus token); the page "SpecKV: Adaptive Speculative Decoding with
 * Compression-Aware Gamma Selection", section on draft-model signals (entropy in bits,
 * max probability, their mean / max / min over the draft block).
 *
 * Conventions shared by every entry point
 *  - Every pointer argument is DEVICE memory owned by the caller; structs are by value.
 *    The library allocates nothing and writes only the outputs and the workspace.
 *  - Calls are asynchronous and ordered on `hip_stream` (a hipStream_t; NULL = the null
 *    stream).  They are re-entrant when concurrent calls use different workspaces.
 *  - Workspaces: zero-fill once before first use; sizes come from the *_workspace_bytes
 *    functions (each covers every path a call can take).  Nothing a call does depends on an
 *    earlier call: the library keeps no settings between calls (per-call options travel in
 *    spec_call_options) and no environment variable changes a path.  Its one piece of
 *    process-wide data is a call sequence number, atomically incremented, that tags the
 *    records a call writes into its workspace so that records of an earlier call are never
 *    taken for this call's.
 *  - Logit rows are dense, row-major, `ld` ELEMENTS apart (ld >= V).  dtype SPEC_BF16 rows
 *    hold bf16 bit patterns, SPEC_F32 rows hold floats.  A 16-byte aligned base with a
 *    16-byte multiple row stride takes the vector path; anything else takes a scalar path
 *    with identical results.  -inf logits are allowed (masked tokens).
 *  - Return codes are synchronous argument / launch checks; per-request problems found on
 *    the device are reported in `out_status` bit flags.
 *  - Randomness is Philox4x64-10 with key (seed, step); see each entry point for its
 *    counters.  A uniform is (word >> 11) * 2^-53.  Equal inputs give bitwise equal outputs.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define SPEC_OK 0
#define SPEC_ERR_INVALID (-1)     /* null / inconsistent argument, bad size, bad parameter */
#define SPEC_ERR_UNSUPPORTED (-2) /* a valid combination this build does not implement     */
#define SPEC_ERR_WORKSPACE (-3)   /* workspace smaller than the *_workspace_bytes figure    */
#define SPEC_ERR_LAUNCH (-4)      /* a HIP launch failed                                    */
#define SPEC_ERR_SCRATCH_LIMIT (-5) /* spec_verify_batch_noalloc: the call needs more workspace
                                       than SPEC_NOALLOC_SCRATCH_BYTES                        */

/* per-request / per-row status bits written to out_status on the device */
#define SPEC_STATUS_NONFINITE 1        /* NaN or +inf logit, or a row with no finite logit:
                                          0 accepted, tokens -1                             */
#define SPEC_STATUS_BAD_TOKEN 2        /* draft token outside [0, V): rejected there        */
#define SPEC_STATUS_ZERO_Q 4           /* q(y) = 0 after filtering: rejected there          */
#define SPEC_STATUS_RESIDUAL_EMPTY 8   /* residual mass 0 after a rejection: drawn from p   */
#define SPEC_STATUS_TIMEOUT 16         /* a bounded wait expired: 0 accepted, tokens -1     */
#define SPEC_STATUS_FILTER_OVERFLOW 32 /* not returned: a filtered row that the sparse path
                                          cannot hold is recomputed on the dense path       */
#define SPEC_STATUS_BAD_GAMMA 64       /* cu_draft inconsistent for this request: nothing
                                          read, 0 accepted, tokens -1                        */

typedef enum { SPEC_F32 = 0, SPEC_BF16 = 1 } spec_dtype;

/* Sampling parameters applied identically to target and draft rows (guide §2.1: p and q are
 * the distributions actually sampled from).  temperature 0 = greedy (argmax).  top_k <= 0 or
 * >= V = off; otherwise every logit >= the k-th largest is kept (ties kept).  top_p >= 1 =
 * off; otherwise the smallest set of largest values whose mass over the top-k set reaches
 * top_p is kept (a boundary value is kept with all its ties).  Order: temperature, top-k,
 * top-p.  Two paths serve filtered calls with the same results.  With 1 <= top_k <= 256 (top-p
 * optional) the sparse path works on per-slice top-k candidates; a request (or plain row) whose
 * top-k set (k plus boundary ties) holds more than 512 tokens, or whose slices had to drop
 * tied candidates, is recomputed in the same call on the dense path.  Every other filter
 * (top-p alone, top_k > 256) takes the dense path, which finds each row's kept-set threshold
 * exactly and has no size limit; SPEC_PATH_MULTI_KERNEL sends every filtered call there. */
typedef struct {
  float temperature;
  int top_k;
  float top_p;
} spec_sampling_params;

/* Optional per-position outputs of spec_verify_batch; each pointer may be NULL.
 * Draft-side arrays have one float per draft row (sum gamma_b, laid out like draft rows);
 * target-side arrays one per target row (sum (gamma_b + 1)).  Values are fp32. */
typedef struct {
  float* p_y;                 /* p_i(y_i); NaN if y_i is not a token                      */
  float* q_y;                 /* q_i(y_i); 1 for a token-only draft                       */
  float* one_minus_tv;        /* sum_x min(p_i, q_i) = 1 - TV(p_i, q_i)   (guide §4.3)     */
  float* draft_entropy_bits;  /* H(q_i) in bits (SpecKV signals); NaN when greedy          */
  float* draft_max_prob;      /* max_x q_i(x); NaN when greedy                             */
  float* target_entropy_bits; /* H(p_i) in bits, i = 1..gamma_b+1; 0 when greedy           */
  float* target_max_prob;     /* max_x p_i(x); 1 when greedy                               */
  /* Extra signals (both KL divergences and the L1 distance are the uncertainty features of
   * the tree-search page's selector; the forward KL is the DLite page's D_KL(p||q) =
   * sum p log(p/q)).  KL is in nats, +inf when one side puts mass where the other has none,
   * NaN when greedy; q is one-hot at y_i for a token-only draft (then NaN if y_i is not a
   * token).  Requesting either KL array routes the call off the single-kernel path.       */
  float* kl_pq;               /* D_KL(p_i || q_i)                                          */
  float* kl_qp;               /* D_KL(q_i || p_i)                                          */
  float* l1;                  /* sum_x |p_i - q_i| = 2 TV                                  */
  float* accept_prob;         /* a_i = min(1, p_i(y_i) / q_i(y_i)); 0 if y_i is not a token
                                 or q_i(y_i) = 0; greedy: 1 iff y_i is the target argmax   */
  float* expected_committed;  /* [B]: 1 + sum_{k=1..gamma_b} prod_{i<=k} a_i, the expected
                                 tokens committed given the drafts (the tree-search page's
                                 variance-free block efficiency for one chain); NaN for a
                                 non-finite request                                        */
} spec_pos_stats;

/* Per-call options of the *_ex entry points; a NULL pointer means every default.  No field
 * changes a result: the paths compute the same outputs, the wait bound and poll timing only
 * move time, and the events only observe it.
 *  path           SPEC_PATH_AUTO: the fastest path for the shape and filter.
 *                 SPEC_PATH_MULTI_KERNEL: the multi-kernel path (one pass per statistic,
 *                 filtered calls through per-row thresholds), for cross-checks.
 *  spin_limit     polls before the single-kernel path's team wait gives up and reports
 *                 SPEC_STATUS_TIMEOUT for the request (no tokens); < 0: 262144; 0: give up at
 *                 the first incomplete poll (a test of the failure path).
 *  poll_delay     10-ns ticks a streaming workgroup waits before its first team poll; <= 0: 400.
 *  poll_pause     pause between failed polls, in units of 128 cycles; <= 0: 8.
 *  profile_start  a hipEvent_t pair, or both NULL: recorded by the dispatch of the call's
 *  profile_stop   streaming kernel (the pass that reads every needed logit), right at its start
 *                 and end, so a benchmark times that kernel alone.  Owned by the caller.
 * An unknown path or exactly one NULL event gives SPEC_ERR_INVALID. */
typedef enum { SPEC_PATH_AUTO = 0, SPEC_PATH_MULTI_KERNEL = 1 } spec_path;
typedef struct {
  int path;
  int64_t spin_limit;
  int poll_delay;
  int poll_pause;
  void* profile_start;
  void* profile_stop;
} spec_call_options;

/* spec_verify_batch -- verify one speculative round for B ragged requests.
 *
 * Request b has gamma_b = cu_draft[b+1] - cu_draft[b] draft tokens (0 <= gamma_b <=
 * gamma_max).  Its target rows are target_logits rows cu_draft[b] + b + i, i = 0..gamma_b
 * (gamma_b + 1 rows, the last one for the bonus token); its draft rows and tokens are rows
 * cu_draft[b] + i, i = 0..gamma_b-1.  n_draft_rows must equal cu_draft[B] (the sum of the
 * gamma_b): it bounds every row index the device forms, so the target allocation must hold
 * n_draft_rows + B rows and the draft allocation n_draft_rows rows.
 *
 *  draft_logits NULL = token-only draft (one-hot q at y_i, guide §3.3); with temperature 0
 *  the draft logits are never read.  Outputs:
 *   out_tokens        [B, gamma_max + 1] int32: accepted draft tokens, then the correction or
 *                     bonus token, then -1 padding.
 *   out_num_accepted  [B] int32 in [0, gamma_b]; the request advances num_accepted + 1 tokens.
 *   pos_stats         optional per-position signals (see spec_pos_stats).
 *   out_req_stats     optional [B, 4] fp32: mean H(q_i), mean max q_i, max H(q_i), min max q_i
 *                     over i = 1..gamma_b (NaN when gamma_b = 0 or greedy).
 *   out_status        [B] int32 status bits (SPEC_STATUS_*).
 *  Randomness: Philox counter (b, i, 0, 0) for 1-based position i: word 0 is the accept draw
 *  at i, words 1..3 drive the three sampler levels when the emitted token is drawn at i.
 *  The sampler is a fixed-order inverse CDF in three levels (chunks of 4096 tokens, groups of
 *  64, tokens) with one uniform per level; its law is exactly the residual (or p_{g+1}).
 *  If cu_draft is not an exclusive prefix (cu_draft[0] = 0, 0 <= gamma_b <= gamma_max,
 *  cu_draft[B] = n_draft_rows) every request reports SPEC_STATUS_BAD_GAMMA; rows may still be
 *  read, but only inside the declared allocations (target rows < n_draft_rows + B, draft rows
 *  < n_draft_rows).
 *  workspace: spec_verify_workspace_bytes(B, V, gamma_max, dt, sp) bytes of device memory,
 *  256-byte aligned, ZERO-FILLED once before its first use with this library (workgroups of
 *  one call exchange records in it, tagged with a per-call sequence number that a zero-filled
 *  workspace never matches).  A workspace serves one call at a time. */
int spec_verify_batch(int B, int V, int gamma_max, spec_dtype dt,
                      const void* target_logits, int64_t target_ld,
                      const void* draft_logits, int64_t draft_ld,
                      const int32_t* draft_tokens, const int32_t* cu_draft, int n_draft_rows,
                      spec_sampling_params sp, uint64_t seed, uint64_t step,
                      int32_t* out_tokens, int32_t* out_num_accepted,
                      spec_pos_stats pos_stats, float* out_req_stats, int32_t* out_status,
                      void* workspace, size_t workspace_bytes, void* hip_stream);

/* spec_verify_batch with per-call options (NULL: defaults, the same call as above). */
int spec_verify_batch_ex(int B, int V, int gamma_max, spec_dtype dt,
                         const void* target_logits, int64_t target_ld,
                         const void* draft_logits, int64_t draft_ld,
                         const int32_t* draft_tokens, const int32_t* cu_draft, int n_draft_rows,
                         spec_sampling_params sp, uint64_t seed, uint64_t step,
                         int32_t* out_tokens, int32_t* out_num_accepted,
                         spec_pos_stats pos_stats, float* out_req_stats, int32_t* out_status,
                         void* workspace, size_t workspace_bytes, void* hip_stream,
                         const spec_call_options* options);

size_t spec_verify_workspace_bytes(int B, int V, int gamma_max, spec_dtype dt,
                                   spec_sampling_params sp);

/* spec_verify_batch_noalloc -- spec_verify_batch for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments and results without the workspace.  The workspace is a static device array of the
 * library, SPEC_NOALLOC_SCRATCH_BYTES on each GPU it runs on, held until the process ends; its
 * address is looked up once per device on the first call there, which also clears it with one
 * kernel on `hip_stream`.  The call allocates nothing (no hipMalloc, no library allocation).
 * Every call on one GPU shares that GPU's array and it keeps the last call's contents: calls
 * that overlap in time on one GPU (different streams, threads or processes' graphs) race; order
 * them, for example on one stream.  A call whose spec_verify_workspace_bytes exceeds the array
 * returns SPEC_ERR_SCRATCH_LIMIT before any launch (the batch-64 and batch-256 unfiltered
 * workloads need a few MB; top-k filtered batches of 256 requests need more than the array). */
#define SPEC_NOALLOC_SCRATCH_BYTES (32u << 20)
int spec_verify_batch_noalloc(int B, int V, int gamma_max, spec_dtype dt,
                              const void* target_logits, int64_t target_ld,
                              const void* draft_logits, int64_t draft_ld,
                              const int32_t* draft_tokens, const int32_t* cu_draft, int n_draft_rows,
                              spec_sampling_params sp, uint64_t seed, uint64_t step,
                              int32_t* out_tokens, int32_t* out_num_accepted,
                              spec_pos_stats pos_stats, float* out_req_stats, int32_t* out_status,
                              void* hip_stream);

/* spec_row_stats -- per-row statistics of R filtered, tempered logit rows (the signals of the
 * SpecKV page, computed on the distribution actually sampled from).  Each output is [R] and
 * may be NULL: max_logit, argmax (lowest index of the maximum), log_z = ln sum_kept
 * exp(l/T), entropy_bits, max_prob, kept_count (kept tokens with a finite logit).  With
 * temperature 0 the row is one-hot at the argmax: entropy 0, max_prob 1, kept 1, log_z NaN.
 * A row with a NaN / +inf logit or no finite logit gives argmax -1, NaN statistics and kept
 * count 0. */
int spec_row_stats(int R, int V, spec_dtype dt, const void* logits, int64_t ld,
                   spec_sampling_params sp,
                   float* max_logit, int32_t* argmax, float* log_z, float* entropy_bits,
                   float* max_prob, int32_t* kept_count,
                   void* workspace, size_t workspace_bytes, void* hip_stream);

/* spec_row_stats with per-call options (NULL: defaults). */
int spec_row_stats_ex(int R, int V, spec_dtype dt, const void* logits, int64_t ld,
                      spec_sampling_params sp,
                      float* max_logit, int32_t* argmax, float* log_z, float* entropy_bits,
                      float* max_prob, int32_t* kept_count,
                      void* workspace, size_t workspace_bytes, void* hip_stream,
                      const spec_call_options* options);

size_t spec_row_stats_workspace_bytes(int R, int V, spec_dtype dt, spec_sampling_params sp);

/* spec_residual_sample -- one draw per row from r(x) = [p(x) - q(x)]_+ / sum [p - q]_+
 * (guide §3.2), or from p when q_logits is NULL, with the same three-level sampler.
 *  uniforms: [R, 3] fp64 in [0, 1) on the device, or NULL for Philox counter (r, 0, 1, 0),
 *  words 1..3.  Outputs [R]: out_token, out_mass (beta = sum [p - q]_+, or 1 without q; NaN
 *  for non-finite rows), out_status (NONFINITE, RESIDUAL_EMPTY: beta = 0, drawn from p). */
int spec_residual_sample(int R, int V, spec_dtype dt,
                         const void* p_logits, int64_t p_ld, const void* q_logits, int64_t q_ld,
                         spec_sampling_params sp, const double* uniforms,
                         uint64_t seed, uint64_t step,
                         int32_t* out_token, double* out_mass, int32_t* out_status,
                         void* workspace, size_t workspace_bytes, void* hip_stream);

/* spec_residual_sample with per-call options (NULL: defaults). */
int spec_residual_sample_ex(int R, int V, spec_dtype dt,
                            const void* p_logits, int64_t p_ld, const void* q_logits, int64_t q_ld,
                            spec_sampling_params sp, const double* uniforms,
                            uint64_t seed, uint64_t step,
                            int32_t* out_token, double* out_mass, int32_t* out_status,
                            void* workspace, size_t workspace_bytes, void* hip_stream,
                            const spec_call_options* options);

size_t spec_residual_sample_workspace_bytes(int R, int V, spec_dtype dt, spec_sampling_params sp);

/* spec_lm_head_row_stats -- the statistics of spec_row_stats for logits that are never
 * materialised: l = h W^T, the projection of hidden states onto the vocabulary (the DLite page,
 * section "核心方法" (core method), projects onto the vocabulary once per round), computed in
 * 256-column tiles with bf16 MFMA (fp32 accumulation) and reduced to per-row statistics in the
 * tiles' epilogue.
 *  hidden      [R, D] bf16 on the device, row stride h_ld elements.
 *  weight      [V, D] bf16 on the device (one head row per vocabulary entry), row stride w_ld.
 *              D, h_ld and w_ld must be multiples of 8 and both bases 16-byte aligned
 *              (otherwise SPEC_ERR_UNSUPPORTED).
 *  sp          temperature T >= 0 (0: greedy); top-k and top-p must be off (SPEC_ERR_UNSUPPORTED).
 *  tokens      [R] int32 or NULL: a token per row for p_tok.
 *  outputs     [R] each, or NULL: max_logit, argmax (lowest index), log_z = ln sum exp(l / T)
 *              (NaN when greedy), entropy_bits, max_prob, p_tok = p(tokens[r]) (NaN for a
 *              token outside [0, V); requires tokens).  A row with a NaN or +inf logit, or no
 *              finite one, gets NaN everywhere and argmax -1; greedy rows report entropy 0,
 *              max_prob 1 and p_tok 1 or 0.
 *  workspace   spec_lm_head_workspace_bytes(R, V, D) bytes, 256-byte aligned.
 * The logits carry fp32 accumulation error, at most D 2^-24 sum_d |h_d W_{v,d}| each.
 * Returns SPEC_OK, SPEC_ERR_INVALID, SPEC_ERR_UNSUPPORTED, SPEC_ERR_WORKSPACE or
 * SPEC_ERR_LAUNCH. */
int spec_lm_head_row_stats(int R, int V, int D, const void* hidden, int64_t h_ld, const void* weight, int64_t w_ld,
                           spec_sampling_params sp, const int32_t* tokens, float* max_logit, int32_t* argmax,
                           float* log_z, float* entropy_bits, float* max_prob, float* p_tok, void* workspace,
                           size_t workspace_bytes, void* hip_stream);

/* spec_lm_head_row_stats with per-call options (NULL: defaults; the profile events bracket the
 * MFMA tile kernel). */
int spec_lm_head_row_stats_ex(int R, int V, int D, const void* hidden, int64_t h_ld, const void* weight,
                              int64_t w_ld, spec_sampling_params sp, const int32_t* tokens, float* max_logit,
                              int32_t* argmax, float* log_z, float* entropy_bits, float* max_prob, float* p_tok,
                              void* workspace, size_t workspace_bytes, void* hip_stream,
                              const spec_call_options* options);

size_t spec_lm_head_workspace_bytes(int R, int V, int D);

/* Weights of the draft-length predictor: the SpecKV page's acceptance-rate regressor
 * f(x, gamma), an MLP with 16 hidden units, read as h = relu(w1 [x, gamma] + b1),
 * f = w2 . h + b2 with x = [H_bar, c_bar, H_max, c_min, comp].  Device pointers, fp32;
 * w1 is [16][6] row-major, b1 and w2 are [16]. */
typedef struct {
  const float* w1;
  const float* b1;
  const float* w2;
  float b2;
} spec_gamma_mlp;

/* spec_select_gamma -- each request's next draft length (SpecKV page, acceptance prediction
 * and gamma selection): gamma* = argmax over gamma in {2, 4, 6, 8} of f(x, gamma) gamma + 1,
 * the expected tokens of a step; ties go to the smaller gamma.
 *  req_stats    [B, 4] fp32: H_bar, c_bar, H_max, c_min, as spec_verify_batch writes them.
 *  comp         [B] fp32: the caller's compression feature of each request, or NULL for 0.
 *  out_gamma    [B] int32: gamma*, or -1 when a feature is NaN (no draft tokens, greedy,
 *               non-finite rows).
 *  out_expected optional [B, 4] fp32: f(x, gamma) gamma + 1 for gamma = 2, 4, 6, 8.
 * fp32 arithmetic, one wave per request, no workspace; stream-ordered after the
 * spec_verify_batch call whose req_stats it reads.  Returns SPEC_OK, SPEC_ERR_INVALID (a
 * required pointer is NULL, B < 0) or SPEC_ERR_LAUNCH. */
int spec_select_gamma(int B, const float* req_stats, const float* comp, spec_gamma_mlp w, int32_t* out_gamma,
                      float* out_expected, void* hip_stream);

/* Benchmark instrumentation, not a verification step: a plain streaming read of `bytes` bytes of
 * device memory at `buf` (16-byte aligned, `bytes` a multiple of 16), the practical HBM read
 * ceiling that a benchmark reports beside the streaming kernel's bandwidth.  `sink` is a device
 * pointer to one uint32_t that the kernel writes only when the XOR of all words equals a fixed
 * value (it keeps the reads from being dropped).  Stream-ordered; nothing is allocated.  Returns SPEC_OK (also for bytes == 0),
 * SPEC_ERR_INVALID (bytes < 0, a NULL pointer), SPEC_ERR_UNSUPPORTED (alignment) or
 * SPEC_ERR_LAUNCH. */
int spec_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* hip_stream);

/* Benchmark instrumentation, not a verification step: the matrix cores' sustained bf16 rate on
 * the fused LM head's pattern, the practical counterpart of the dense MFMA peak that a benchmark
 * reports beside the head's rate.  `workgroups` workgroups of four waves (one wave per SIMD)
 * each issue `iters` steps of 16 independent 32x32x16 bf16 MFMAs (2^19 flop each) on register
 * operands, with no memory traffic: mode 0 all operands 1.0; mode 1 random bf16 operands of
 * normal magnitude, the same every step; mode 2 the random operands with mantissa bits flipped
 * every step.  Modes 1 and 2 show how the rate depends on the data the multipliers see.
 * `sink` is a device pointer to one float, written only if the accumulated sum is exactly
 * 2^127 (it keeps the work from being dropped).  Stream-ordered; nothing is allocated.  Returns
 * SPEC_OK (also for iters == 0 or workgroups == 0), SPEC_ERR_INVALID (mode outside 0..2,
 * iters outside 0..2^20, workgroups outside 0..65536, a NULL sink) or SPEC_ERR_LAUNCH. */
int spec_mfma_rate(int mode, int iters, int workgroups, float* sink, void* hip_stream);

/* Human-readable text for a return code (negative) or a single status bit (positive). */
const char* spec_status_string(int code);

#ifdef __cplusplus
}
#endif
#endif /* SPEC_VERIFY_H */
