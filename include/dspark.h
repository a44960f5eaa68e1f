/*
 * dspark.h — C ABI of the MI355X (gfx950) library for confidence-scheduled
 * block verification in speculative decoding.
 *
 * Three calls make up the data-parallel hot path of one decoding round:
 *
 *   dspark_schedule       survival product, threshold truncation and a global
 *                         verify-token budget (which drafted positions go to
 *                         the target model);
 *   dspark_verify         temperature softmaxes of target and draft rows,
 *                         lossless rejection sampling up to the first
 *                         rejection, and the correction (residual) or bonus
 *                         draw; requests with temperature 0 use the greedy rule;
 *   dspark_verify_greedy  the greedy (T = 0) rule for the whole batch.
 *
 * dspark_schedule_load_aware derives the schedule's threshold and budget on
 * the device from the engine's load and a stored throughput curve;
 * dspark_calibrate and dspark_calib_observe keep the confidences calibrated
 * online (per-position temperatures updated from the observed acceptance);
 * dspark_markov_draft drafts a block with the Markov logit bias.
 *
 * Sources (page title, then section):
 *   "DSpark Deep Dive: How DeepSeek Squeezed an 85% Speedup Out of Inference
 *    Without Touching a Single Model Weight" — "Speculative Decoding From First
 *    Principles" (draft, verify in one target pass, accept with probability
 *    min(1, p/q), resample a rejection from the normalised positive part of
 *    p - q), "Variable-Length Drafts", "The Optimization Logic", "GPU-Resident
 *    Scheduling" (scheduler on the GPU; maximum-length buffers plus masking so
 *    that variable lengths fit a fixed launch), "The Full Scheduling Pipeline"
 *    (1 <= L <= K; drafted tokens past L are discarded).
 *   "DSpark Guide: Confidence Speculative Decoding in LLMs" — "1. The
 *    Mathematics of Suffix Decay" (alpha_k = min(1, P/Q_k)), "2. Confidence-
 *    Scheduled Dynamic Verification" (C_k = prod_{i<=k} p_i, truncate at the
 *    first k with C_k < tau).
 *   "DSpark shows why fast AI inference is a scheduling problem, not a model
 *    trick" — prefix survival probability cut at a threshold.
 *
 * Conventions shared by every call:
 *   - All array arguments are DEVICE pointers owned by the caller; the
 *     library never allocates, frees or synchronises. Work is enqueued on
 *     `stream` (a hipStream_t passed as void*; NULL = the default stream) and
 *     outputs are valid once the stream reaches the call. Every call is a
 *     fixed sequence of kernel launches whose shape depends only on the
 *     scalar arguments, so it can be captured in a HIP graph.
 *   - Arrays are dense, row-major, with the shapes given below; logits rows
 *     must start on 16-byte boundaries for the vectorised path (a row-wise
 *     scalar path handles any other V).
 *   - Indices: b = request 0..B-1; drafted position k = 1..K is stored at
 *     column k-1. Target row j (0..K) is the target distribution for the
 *     token after the prefix plus the first j drafted tokens; row j = k-1
 *     scores drafted token y_k and row L_b is the bonus row. Draft row j
 *     (0..K-1) is the distribution drafted token y_{j+1} came from.
 *   - The return value is a synchronous status (argument checks only; no
 *     launch happens unless it is DSPARK_OK). Faults found in the DATA are
 *     OR-ed as DSPARK_DEV_* bits into *dev_status (the caller zeroes it);
 *     outputs of an affected request are then unspecified but every access
 *     stays in bounds.
 *   - `workspace` is caller-allocated device memory of at least
 *     dspark_workspace_bytes(op, B, K, V) bytes, 256-byte aligned. Calls that
 *     run concurrently need distinct workspaces. Nothing in it needs to be
 *     initialised.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define DSPARK_API __attribute__((visibility("default")))
#else
#define DSPARK_API
#endif

typedef enum {
  DSPARK_OK = 0,
  DSPARK_ERR_NULL = 1,      /* a required pointer is NULL                         */
  DSPARK_ERR_SHAPE = 2,     /* B, K or V out of range (B,K,V >= 1; K <= 64 for verify) */
  DSPARK_ERR_DTYPE = 3,     /* unknown logits dtype                               */
  DSPARK_ERR_BUDGET = 4,    /* budget >= 0 but < B*min_len, or min_len not in [0,K] */
  DSPARK_ERR_WORKSPACE = 5, /* ws_bytes too small or workspace misaligned         */
  DSPARK_ERR_LAUNCH = 6,    /* the HIP runtime rejected a launch                  */
  DSPARK_ERR_PARAM = 7,     /* a parameter out of range or misaligned (per call)  */
  DSPARK_ERR_SCRATCH = 8    /* sizes beyond the built-in scratch (no-alloc call)  */
} dspark_status;

typedef enum { DSPARK_F32 = 0, DSPARK_BF16 = 1 } dspark_dtype;

/* Device status bits (OR-ed into *dev_status). */
#define DSPARK_DEV_BAD_TOKEN 1    /* a drafted id that is read lies outside [0, V)      */
#define DSPARK_DEV_NONFINITE 2    /* a row that is read holds NaN or +Inf, or no finite logit (-Inf alone is legal) */
#define DSPARK_DEV_BAD_TEMP 4     /* temperature < 0 or NaN                              */
#define DSPARK_DEV_BAD_UNIFORM 8  /* a uniform that is read lies outside [0, 1)          */
#define DSPARK_DEV_BAD_CONF 16    /* a confidence is NaN or outside [0, 1]               */
#define DSPARK_DEV_BAD_LENGTH 32  /* lengths[b] outside [0, K] (clamped)                 */
#define DSPARK_DEV_BAD_LOAD 64    /* queue depth or memory in use NaN, infinite or < 0    */
#define DSPARK_DEV_BAD_CURVE 128  /* throughput curve breaks the rules of dspark_schedule_load_aware */
#define DSPARK_DEV_INCOMPLETE 256 /* a verify launch gave up waiting for another workgroup (1 s): outputs unspecified */

#define DSPARK_OP_SCHEDULE 0
#define DSPARK_OP_VERIFY 1
#define DSPARK_OP_VERIFY_GREEDY 2
#define DSPARK_OP_MARKOV_DRAFT 3
#define DSPARK_OP_SCHEDULE_VERIFY 4

/* Bytes of workspace `op` needs for these sizes (0 for bad sizes). */
DSPARK_API size_t dspark_workspace_bytes(int op, int B, int K, int V);

/* Static text for a dspark_status value. */
DSPARK_API const char* dspark_status_string(int status);

/*
 * dspark_schedule — which drafted positions are verified.
 *
 * Defines (DSpark Guide, "2. Confidence-Scheduled Dynamic Verification";
 * DSpark Deep Dive, "Variable-Length Drafts", "The Optimization Logic"):
 *   C[b,1] = conf[b,1];  C[b,k] = fp32(C[b,k-1] * conf[b,k])   (left to right)
 *   Lthr[b] = max(min_len, number of leading k with C[b,k] >= threshold)
 *   if budget >= 0 and sum_b Lthr[b] > budget:
 *     each request keeps min_len positions; the other budget - B*min_len
 *     slots go to candidates (b,k), min_len < k <= Lthr[b], ordered by C
 *     descending, then b ascending, then k ascending;
 *     lengths[b] = min_len + (number of row-b candidates taken)
 *   else lengths[b] = Lthr[b].
 * For confidences in [0,1] the survival is non-increasing in k, so the
 * selected set is a prefix of every row and the budget fill maximises the
 * total survival of the verified positions.
 *
 *   conf      [B,K] float32 per-position confidence, expected in [0,1]
 *   threshold survival threshold tau (compared as fp32)
 *   budget    total drafted positions to verify, < 0 = no budget
 *   min_len   positions every request keeps (1 by default; 0 allowed)
 *   lengths   [B] int32 out, min_len <= lengths[b] <= K
 *   mask      [B,K] uint8 out, mask[b,k-1] = (k <= lengths[b]); may be NULL
 *   survival  [B,K] float32 out C[b,k]; may be NULL
 * Errors: NULL conf/lengths/dev_status/workspace; B < 1 or K < 1;
 * min_len outside [0,K]; 0 <= budget < B*min_len; small workspace.
 */
DSPARK_API int dspark_schedule(const float* conf, int B, int K, float threshold, int budget, int min_len,
                    int32_t* lengths, uint8_t* mask, float* survival,
                    int32_t* dev_status, void* workspace, size_t ws_bytes, void* stream);

/*
 * dspark_schedule_load_aware — dspark_schedule with its threshold and budget
 * derived on the device from the engine's load and a stored throughput
 * curve, with no host round trip.
 *
 * Defines (DSpark Guide, "Dynamic Verification Scheduling Algorithm", steps
 * 1 and 2, and its code listing's threshold line; DSpark Deep Dive, "The
 * Throughput Curve", "The Optimization Logic", "GPU-Resident Scheduling"):
 *   LF  = clamp(0.6 * (Q / q_max) + 0.4 * (M / m_max), 0, 1)     fp32, in this order
 *   tau = tau_min + (tau_max - tau_min) * (LF * LF)               fp32, in this order
 *   with curve points (x_i tokens per target forward pass, T_i tokens/s),
 *   g_i = (T_i - T_{i-1}) / (x_i - x_{i-1}) in fp64 for i >= 1;
 *   x*  = x_{i-1} for the first i with g_i < slot_cost, else x_{n-1};
 *   budget = max(B * min_len, x* - B)   (one position per request in a
 *            forward pass is not a drafted token; no curve: budget = -1);
 *   then exactly dspark_schedule(conf, B, K, tau, budget, min_len, ...).
 * A queue depth or memory figure that is NaN, infinite or negative sets
 * DSPARK_DEV_BAD_LOAD and is read as LF = 1. A curve whose x are not whole
 * numbers in [1, 2^24], strictly ascending, or whose values are not finite,
 * sets DSPARK_DEV_BAD_CURVE and means no budget. The pages give tau_min as
 * 0.20 (prose) and 0.25 (code) and tau_max as 0.75; both are arguments.
 *
 *   load       device float32[2]: Q (queue depth) and M (GPU memory in use,
 *              in the unit of m_max), read when the kernel runs
 *   q_max, m_max   finite, > 0
 *   tau_min, tau_max   finite, 0 <= tau_min <= tau_max
 *   curve      device float32[n_curve][2], (x_i, T_i); may be NULL if n_curve == 0
 *   n_curve    0..64; 0 = no budget
 *   slot_cost  finite, tokens/s a token must add to be worth its slot
 *   tau_out    device float32[1] out, the threshold used; may be NULL
 *   budget_out device int32[1] out, the budget used (-1 = none); may be NULL
 *   other arguments as for dspark_schedule (same workspace, op
 *   DSPARK_OP_SCHEDULE).
 * Errors: as dspark_schedule (NULL conf/lengths/dev_status/workspace/load,
 * shape, min_len, workspace), and DSPARK_ERR_PARAM for a parameter above out
 * of range, n_curve outside 0..64, or n_curve > 0 with a NULL curve.
 */
DSPARK_API int dspark_schedule_load_aware(const float* conf, int B, int K, const float* load,
                                          float q_max, float m_max, float tau_min, float tau_max,
                                          const float* curve, int n_curve, float slot_cost,
                                          int min_len, int32_t* lengths, uint8_t* mask,
                                          float* survival, float* tau_out, int32_t* budget_out,
                                          int32_t* dev_status, void* workspace, size_t ws_bytes,
                                          void* stream);

/*
 * dspark_markov_draft — semi-autoregressive drafting with the Markov logit
 * bias: the block's draft logits and drafted tokens, position by position.
 *
 * Defines (DSpark Guide, the Markov logit-bias head and its code listing):
 * for k = 1..K in order, with y_0 = y0[b] (the last target token),
 *   corrected[b,k-1,:] = base[b,k-1,:] + scale * U . Vm[y_{k-1},:]^T
 *       (the rank-r sum accumulated in fp32 on the matrix cores, scaled and
 *       added to the widened base logit in fp32, stored in `dtype`, bf16
 *       rounded to nearest even)
 *   y_k = the smallest token id whose cumulative mass of
 *       softmax(corrected[b,k-1,:] / T_b) exceeds uniforms[b,k-1] (T_b = 0:
 *       the lowest-index maximum), drawn from the STORED corrected logits so
 *       that the draft distribution is exactly what dspark_verify reads as
 *       draft row k-1.
 *
 *   base       [B,K,V] dtype parallel logits
 *   U, Vm      [V,r] bf16 (uint16 bit patterns) low-rank transition factors,
 *              16-byte aligned
 *   r          rank, a multiple of 16 in [16, 256]
 *   scale      the listing's scalar on the bias
 *   y0         [B] int32 token before the block
 *   temperature [B] float32, uniforms [B,K] float32 in [0,1)
 *   corrected  [B,K,V] dtype out (the draft logits for dspark_verify)
 *   drafted    [B,K] int32 out, q_tok [B,K] float32 out softmax prob of the
 *              drafted token (1 at T = 0); q_tok may be NULL
 *   workspace  dspark_workspace_bytes(DSPARK_OP_MARKOV_DRAFT, B, K, V)
 * 2K kernel launches (a contraction and a draw per position).
 * A previous token outside [0,V) sets DSPARK_DEV_BAD_TOKEN (read as 0), a
 * non-finite corrected logit DSPARK_DEV_NONFINITE, a bad temperature
 * DSPARK_DEV_BAD_TEMP.
 * Errors: NULL pointers; B, K, V < 1; r not a multiple of 16 in [16,256];
 * unknown dtype; U or Vm misaligned (DSPARK_ERR_PARAM); small workspace.
 */
DSPARK_API int dspark_markov_draft(const void* base, int dtype, int B, int K, int V,
                                   const uint16_t* U, const uint16_t* Vm, int r, float scale,
                                   const int32_t* y0, const float* temperature,
                                   const float* uniforms, void* corrected, int32_t* drafted,
                                   float* q_tok, int32_t* dev_status, void* workspace,
                                   size_t ws_bytes, void* stream);

/*
 * dspark_calibrate — per-position temperature scaling of the confidences.
 *
 * Defines (DSpark Deep Dive, "Online Calibration", "Sequential Temperature
 * Scaling"):  calibrated[b,k] = sigmoid(logit(raw[b,k]) / theta[k]),
 * computed in fp64 and stored as fp32; scores 0 and 1 stay 0 and 1.
 *
 *   raw        [B,K] float32 confidence-head scores, expected in [0,1]
 *   theta      [K] float32 per-position temperatures, expected finite and > 0
 *   calibrated [B,K] float32 out (may alias raw)
 * A score that is NaN or outside [0,1], or a temperature that is NaN,
 * infinite or not positive, sets DSPARK_DEV_BAD_CONF and the score passes
 * through unchanged.
 * Errors: NULL raw/theta/calibrated/dev_status; B < 1, K < 1 or K > 64.
 */
DSPARK_API int dspark_calibrate(const float* raw, const float* theta, int B, int K,
                                float* calibrated, int32_t* dev_status, void* stream);

/* Bytes of calibration window state for K positions and n_bins ECE bins. */
DSPARK_API size_t dspark_calib_state_bytes(int K, int n_bins);

/*
 * dspark_calib_observe — one verification round into the calibration window,
 * and at its end the temperature step (DSpark Deep Dive, "Online
 * Calibration", "Online Adaptation" and "The Calibration Loop in Practice").
 *
 * Per round, for every request b and position k (1-based) whose accept test
 * ran — k <= lengths[b] and k <= accepted[b] + 1 — the window counts the
 * token, whether it was accepted (k <= accepted[b]) and its calibrated score,
 * per position and per score bin (n_bins equal-width bins on [0,1], a score
 * s in bin min(floor(s * n_bins), n_bins - 1), the product taken in fp64).
 * When this call completes the window (`window` rounds):
 *   theta[k] = max(theta_min, theta[k] + lr * (mean score - accepted fraction))
 *              for every position with a token in the window (fp64, stored fp32);
 *   *ece_out = sum over bins |accepted - sum of scores| / tokens (expected
 *              calibration error of the window);
 *   and the window restarts.
 *
 *   calibrated [B,K] float32, the scores the round was scheduled with
 *   lengths    [B] int32 scheduled lengths (NULL: all K)
 *   accepted   [B] int32 accepted counts from dspark_verify
 *   theta      [K] float32 in/out temperatures
 *   lr, theta_min  finite, theta_min > 0
 *   window     rounds per window, >= 1
 *   n_bins     1..64
 *   state      device memory of dspark_calib_state_bytes(K, n_bins) bytes,
 *              8-byte aligned, zero-filled before the first call; the
 *              library keeps it between calls and restarts it at each
 *              window's end. Layout in 8-byte words: rounds; per position
 *              tokens[K], accepted[K], score sums[K] (double); per bin
 *              tokens[n_bins], accepted[n_bins], score sums[n_bins] (double).
 *   ece_out    [1] float32 out, written at each window's end; may be NULL
 * Lengths or accepted counts out of range set DSPARK_DEV_BAD_LENGTH (then
 * clamped), scores outside [0,1] DSPARK_DEV_BAD_CONF. Calls that share a
 * state must be ordered (one stream).
 * Errors: NULL calibrated/accepted/theta/state/dev_status; B < 1, K < 1 or
 * K > 64; DSPARK_ERR_PARAM for lr, theta_min, window or n_bins out of range;
 * DSPARK_ERR_WORKSPACE for a small or misaligned state.
 */
DSPARK_API int dspark_calib_observe(const float* calibrated, const int32_t* lengths,
                                    const int32_t* accepted, int B, int K, float* theta, float lr,
                                    float theta_min, int window, int n_bins, void* state,
                                    size_t state_bytes, float* ece_out, int32_t* dev_status,
                                    void* stream);

/*
 * dspark_verify — lossless block verification.
 *
 * For every request b with T = temperature[b] > 0 and L = lengths[b]
 * (DSpark Deep Dive, "Speculative Decoding From First Principles";
 * DSpark Guide, "1. The Mathematics of Suffix Decay"):
 *   p_k = softmax(target[b,k-1,:] / T),  q_k = softmax(draft[b,k-1,:] / T)
 *   alpha_k = min(1, p_k(y_k) / q_k(y_k))  (0 if p_k(y_k) = 0, 1 if only q is 0)
 *   a = (first k <= L with NOT uniforms[b,k-1] < alpha_k) - 1, or L if none
 *   if a < L: t drawn from r = max(0, p_{a+1} - q_{a+1}) / sum(r)
 *             (r == 0 everywhere: drawn from p_{a+1})
 *   else:     t drawn from softmax(target[b,L,:] / T)  (the bonus token)
 *   draw = the smallest token id whose cumulative mass exceeds
 *          uniforms[b,K] * (total mass), ids in ascending order
 *   accepted[b] = a; tokens[b,:] = (y_1 .. y_a, t, -1, ...).
 * For T = 0 the greedy rule of dspark_verify_greedy applies to that request.
 * Target rows past L and draft rows past L-1 are never read; draft rows of
 * T = 0 requests are never read.
 *
 *   target_logits [B,K+1,V] dtype; draft_logits [B,K,V] dtype
 *   dtype         DSPARK_F32 or DSPARK_BF16
 *   drafted       [B,K] int32 drafted ids y_k
 *   lengths       [B] int32 verify lengths (normally dspark_schedule's);
 *                 NULL = K for every request; out-of-range values are clamped
 *                 to [0,K] and flagged
 *   temperature   [B] float32 (0 = greedy)
 *   uniforms      [B,K+1] float32 in [0,1): column k-1 is position k's
 *                 accept test, column K the final draw
 *   accepted      [B] int32 out
 *   tokens        [B,K+1] int32 out, -1 padded
 *   p_tok, q_tok  [B,K] float32 out p_k(y_k), q_k(y_k) for k <= L and T > 0,
 *                 0 elsewhere; either may be NULL
 * Errors: NULL required pointer; B,V < 1; K < 1 or K > 64; bad dtype; small
 * workspace.
 */
DSPARK_API int dspark_verify(const void* target_logits, const void* draft_logits, int dtype, int B, int K,
                  int V, const int32_t* drafted, const int32_t* lengths,
                  const float* temperature, const float* uniforms, int32_t* accepted,
                  int32_t* tokens, float* p_tok, float* q_tok, int32_t* dev_status,
                  void* workspace, size_t ws_bytes, void* stream);

/*
 * dspark_verify_greedy — greedy (T = 0) verification of the whole batch
 * (perchy.ai "The Technology": outputs match standard decoding; DSpark Guide,
 * tutorial drafter takes the argmax):
 *   g_j = lowest token id attaining max_v target[b,j,v] (compared as floats)
 *   a = (first k <= L with y_k != g_{k-1}) - 1, or L if none
 *   accepted[b] = a; tokens[b,:] = (y_1 .. y_a, g_a, -1, ...).
 * Reads target rows 0..L only.  Arguments as for dspark_verify.
 */
DSPARK_API int dspark_verify_greedy(const void* target_logits, int dtype, int B, int K, int V,
                         const int32_t* drafted, const int32_t* lengths, int32_t* accepted,
                         int32_t* tokens, int32_t* dev_status, void* workspace, size_t ws_bytes,
                         void* stream);

/*
 * dspark_schedule_verify — one verification step: dspark_schedule, then
 * dspark_verify on the lengths it produced, as one call (DSpark Deep Dive,
 * "GPU-Resident Scheduling": the schedule runs on the device and hands the
 * lengths to verification without a host round trip; the scheduling and
 * verification passages cited at those two calls define what is computed).
 *
 * Results are exactly those of
 *   dspark_schedule(conf, B, K, threshold, budget, min_len, lengths, mask,
 *                   survival, ...) followed by
 *   dspark_verify(target_logits, draft_logits, dtype, B, K, V, drafted,
 *                 lengths, temperature, uniforms, accepted, tokens, p_tok,
 *                 q_tok, ...)
 * on the same stream; the arguments mean what they mean there, and lengths
 * is required (it is the schedule's output and the verification's input).
 * With B <= 512, K <= 16 and B*K <= 12288 the schedule is worked out inside
 * the streaming pass (every workgroup computes it from the confidences while
 * its first loads are in flight, and each writes the lengths, mask rows and
 * survival rows of its share of the requests), which saves a launch; larger
 * batches launch the schedule first. Overlapping calls need distinct
 * workspaces, as for the other calls.
 *   workspace  dspark_workspace_bytes(DSPARK_OP_SCHEDULE_VERIFY, B, K, V)
 * Errors: those of the two calls (argument checks of both come before any
 * launch).
 */
DSPARK_API int dspark_schedule_verify(const float* conf, float threshold, int budget,
                                      int min_len, int32_t* lengths, uint8_t* mask,
                                      float* survival, const void* target_logits,
                                      const void* draft_logits, int dtype, int B, int K, int V,
                                      const int32_t* drafted, const float* temperature,
                                      const float* uniforms, int32_t* accepted, int32_t* tokens,
                                      float* p_tok, float* q_tok, int32_t* dev_status,
                                      void* workspace, size_t ws_bytes, void* stream);

/*
 * The calls above in two halves, for callers that want to place or time the
 * streaming pass on its own (for instance to run the streaming pass of the
 * next batch on another stream while this one finishes, or to bracket it
 * with events).  The pages define no such split; what is computed is exactly
 * what the call without the suffix computes.
 *
 *   phases  DSPARK_PHASE_STREAM: enqueue everything up to and including the
 *           streaming pass (the launch that reads every scheduled logits row
 *           once; for dspark_schedule_verify_phase with more than 512
 *           requests, the schedule's own launch first);
 *           DSPARK_PHASE_FINISH: enqueue the rest (the decision, the residual
 *           and the draw), which reads what the streaming pass left in the
 *           workspace;
 *           both bits: the whole call.
 *   other arguments: as for the call without the suffix.
 * The FINISH half must follow the STREAM half on the same stream, once, with
 * the same arguments and workspace, and nothing that writes the workspace in
 * between (the STREAM half also resets the hand-over state the FINISH half
 * uses). A split call (phases other than both bits) needs
 * B <= 2048 (the workspace holds one launch batch); larger batches return
 * DSPARK_ERR_SHAPE. phases outside 1..3 returns DSPARK_ERR_PARAM.
 */
#define DSPARK_PHASE_STREAM 1
#define DSPARK_PHASE_FINISH 2

DSPARK_API int dspark_verify_phase(int phases, const void* target_logits, const void* draft_logits,
                                   int dtype, int B, int K, int V, const int32_t* drafted,
                                   const int32_t* lengths, const float* temperature,
                                   const float* uniforms, int32_t* accepted, int32_t* tokens,
                                   float* p_tok, float* q_tok, int32_t* dev_status,
                                   void* workspace, size_t ws_bytes, void* stream);

DSPARK_API int dspark_verify_greedy_phase(int phases, const void* target_logits, int dtype, int B,
                                          int K, int V, const int32_t* drafted,
                                          const int32_t* lengths, int32_t* accepted,
                                          int32_t* tokens, int32_t* dev_status, void* workspace,
                                          size_t ws_bytes, void* stream);

DSPARK_API int dspark_schedule_verify_phase(int phases, const float* conf, float threshold,
                                            int budget, int min_len, int32_t* lengths,
                                            uint8_t* mask, float* survival,
                                            const void* target_logits, const void* draft_logits,
                                            int dtype, int B, int K, int V, const int32_t* drafted,
                                            const float* temperature, const float* uniforms,
                                            int32_t* accepted, int32_t* tokens, float* p_tok,
                                            float* q_tok, int32_t* dev_status, void* workspace,
                                            size_t ws_bytes, void* stream);

/*
 * dspark_schedule_verify_noalloc — dspark_schedule_verify for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation. It takes no workspace; its
 * kernels use the library's built-in scratch instead, a device array of
 * DSPARK_SCRATCH_BYTES (16 MiB) per GPU, held from the first call on that
 * GPU until the process ends. It allocates and frees nothing.
 *
 * Computes exactly what dspark_schedule_verify computes (the same kernels),
 * with the same arguments apart from the workspace.
 *   Sizes: dspark_workspace_bytes(DSPARK_OP_SCHEDULE_VERIFY, B, K, V) must
 *   not exceed DSPARK_SCRATCH_BYTES (for V = 151,936: B up to 330 at K = 16,
 *   up to 532 at K = 8), else DSPARK_ERR_SCRATCH before any launch.
 *   Every call on one GPU shares that GPU's scratch, and the scratch keeps
 *   what the last call left (nothing in it needs to start at zero): calls
 *   that overlap on one GPU (different streams, or different host threads
 *   without ordering) race and must not be issued.
 * Errors: those of dspark_schedule_verify except the workspace ones;
 * DSPARK_ERR_SCRATCH for sizes beyond the scratch; DSPARK_ERR_LAUNCH if the
 * scratch's device address cannot be obtained.
 */
#define DSPARK_SCRATCH_BYTES (16u << 20)

DSPARK_API int dspark_schedule_verify_noalloc(const float* conf, float threshold, int budget,
                                              int min_len, int32_t* lengths, uint8_t* mask,
                                              float* survival, const void* target_logits,
                                              const void* draft_logits, int dtype, int B, int K,
                                              int V, const int32_t* drafted,
                                              const float* temperature, const float* uniforms,
                                              int32_t* accepted, int32_t* tokens, float* p_tok,
                                              float* q_tok, int32_t* dev_status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
