/*
 * dspark.h — C ABI of the DSpark draft-round hot path on MI355X (gfx950).
 *
 * Four operations, each the data-parallel core of one step of a DSpark draft
 * round as the pages describe it:
 *
 *   dspark_block_attention  block-masked dual-source attention
 *   dspark_markov_sample    Markov-head sequential gamma-step sampler
 *   dspark_accept_rate      TV-distance accept rate (+ optional tau)
 *   dspark_eval_mask        cumulative-product eval mask
 *
 * and two training-side neighbours of the same steps:
 *
 *   dspark_markov_block_logits  teacher-forced Markov logits of a whole block
 *   dspark_markov_head_sample / dspark_markov_head_block_logits
 *                               the same for the gated and recurrent heads
 *   dspark_l1_loss              L1 (TV) alignment loss, its gradient, tau_greedy
 *   dspark_confidence_schedule  confidence head, prefix survival, verify length
 *   dspark_verify               lossless verify (rejection sampling) of a drafted block
 *
 * Sources (cited per entry point): page 1 = "03 · DSpark 建模：Markov 与
 * Confidence" (devpress.csdn.net), page 2 = "从 DFlash 到 dLLM Self-Spec
 * （三）" (r00kie-liu.github.io), page 4 = "DSpark 深度解读" (juejin.cn).
 *
 * Shape names follow page 1 §3.1: B batch, A anchors (blocks) per row,
 * gamma block size, V vocabulary, Hq / Hkv query / key-value heads,
 * D head dimension, r Markov rank, R Markov rows.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor argument is a caller-owned DEVICE pointer to contiguous
 *   row-major memory in the stated layout.  The library never allocates,
 *   frees or keeps a pointer after the call returns.
 * - Scratch memory is passed in as (ws, ws_bytes); size it with the matching
 *   *_workspace_bytes() query (a pure host function of the shapes).  A
 *   workspace may be reused by later calls on the same stream; two calls
 *   that run concurrently must not share one.
 * - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *   enqueue work on it and never synchronise the host.
 * - Arguments are validated on the host before any HIP call; an invalid
 *   argument returns DSPARK_ERR_INVALID_ARG and enqueues nothing.
 * - Data-dependent faults that only the device can see (an anchor outside
 *   its context, a token outside [0, V), ...) set bits in the optional
 *   device word *dev_status (atomic OR; pass NULL to ignore them).  Kernels
 *   clamp such indices, so they never read or write out of bounds.
 * - The human-readable reason of the last failing call on the calling host
 *   thread is returned by dspark_last_error().
 * - Outputs are bitwise deterministic for fixed inputs and launch shapes.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define DSPARK_OK               0
#define DSPARK_ERR_INVALID_ARG (-1)
#define DSPARK_ERR_WORKSPACE   (-2)
#define DSPARK_ERR_UNSUPPORTED (-3)
#define DSPARK_ERR_HIP         (-4)

/* element types */
#define DSPARK_F32  0
#define DSPARK_BF16 1

/* bits OR-ed into *dev_status */
#define DSPARK_STATUS_BAD_ANCHOR  1  /* kept block with anchor < 0 or > its context length */
#define DSPARK_STATUS_BAD_TOKEN   2  /* previous token outside [0, V) */
#define DSPARK_STATUS_BAD_OFFSETS 4  /* ctx_offsets not non-decreasing, or a context longer than max_ctx */
#define DSPARK_STATUS_BAD_LABEL   8  /* label index beyond S_stride of the loss mask */
#define DSPARK_STATUS_WAIT_TIMEOUT 16 /* a workgroup of a cooperative grid gave up waiting on its peers */

/* Library version (major*10000 + minor*100 + patch). */
int dspark_version(void);

/* Reason of the last non-zero status returned on this host thread ("" if none). */
const char* dspark_last_error(void);

/* ------------------------------------------------------------------------
 * Block-masked dual-source attention (page 1 §3.4 block attention mask and
 * §3.5 custom attention; page 4 §3.2).  Queries come from the draft blocks
 * only; keys/values are the context projections followed by the block's own
 * projections.  For draft row (b, a, k) and query head h (key/value head
 * kvh = h / (Hq / Hkv)):
 *
 *     out = sum_{j in vis} softmax_j(scale * <q, k_j>) * v_j
 *     vis = context rows [0, anchor[b,a]) of request b
 *           + the gamma own-block rows (b, a*gamma .. a*gamma+gamma-1)
 *
 * and a block with keep_mask[b,a] == 0 outputs zeros (lse = -inf).  Within a
 * block every query sees all gamma own-block keys.
 *
 *   q            [B, A*gamma, Hq, D]    dtype
 *   k_ctx, v_ctx [T, Hkv, D]            dtype, T = ctx_offsets[B]; request b
 *                                        owns rows ctx_offsets[b] .. ctx_offsets[b+1]-1
 *   ctx_offsets  [B+1] int32, non-decreasing, ctx_offsets[0] = 0
 *   k_blk, v_blk [B, A*gamma, Hkv, D]   dtype
 *   anchor_pos   [B, A] int32: 0 <= anchor <= context length of request b
 *   keep_mask    [B, A] uint8 (0 = masked block; its anchor is ignored)
 *   out          [B, A*gamma, Hq, D]    dtype (written for every row)
 *   lse          [B, Hq, A*gamma] float32, natural-log log-sum-exp of the
 *                scaled logits, -inf for masked rows (nullable)
 *   max_ctx      host upper bound of every request's context length
 *   total_ctx    rows allocated in k_ctx / v_ctx (T); every request's range
 *                is clamped into [0, total_ctx) and a clamp is flagged
 *                DSPARK_STATUS_BAD_OFFSETS, so bad offsets never read out of
 *                bounds
 *   scale        logit scale > 0 (1/sqrt(D) for Qwen3-style, 1.0 for Gemma4-style)
 *   dtype        DSPARK_BF16 (fp32 accumulate, bf16 out) or DSPARK_F32
 * Limits: D in {64, 128}; Hq % Hkv == 0; 1 <= gamma <= 64; A*gamma*Hq/Hkv
 * rows per (b, kvh) below 2^31.  Out-of-range anchors are clamped into
 * [0, context length] and flagged DSPARK_STATUS_BAD_ANCHOR.
 * ---------------------------------------------------------------------- */
size_t dspark_block_attention_workspace_bytes(int B, int A, int gamma, int Hq, int Hkv,
                                              int D, int max_ctx);
int dspark_block_attention(const void* q, const void* k_ctx, const void* v_ctx,
                           const int32_t* ctx_offsets, const void* k_blk, const void* v_blk,
                           const int32_t* anchor_pos, const uint8_t* keep_mask,
                           void* out, float* lse,
                           int B, int A, int gamma, int Hq, int Hkv, int D, int max_ctx,
                           int total_ctx, float scale, int dtype,
                           void* ws, size_t ws_bytes, int32_t* dev_status, void* stream);

/* ------------------------------------------------------------------------
 * Markov-head sequential sampler (page 1 §3.7, the paper's Eq. 5; page 2
 * §3.4 and §3.8.2 sample_block_tokens).  For every row, left to right over
 * i = 0 .. gamma-1, with prev = first_prev[row] at i = 0:
 *
 *     l[v]  = base_logits[row, i, v] + sum_j W1[prev, j] * W2[j, v]
 *     tok   = argmax_v l[v]                      (temperature == 0, greedy)
 *           = argmax_v l[v] / T + G(seed,row,i,v) (temperature T > 0)
 *     tokens[row, i] = tok;  prev = tok
 *
 * Ties go to the lowest index.  G is Gumbel(0,1) noise -ln(-ln u) with
 * u = ((x >> 9) + 1/2) * 2^-23, x = word (v & 3) of Philox4x32-10 (Salmon
 * et al., SC'11) at counter (v >> 2, i, row, 0) and key (seed mod 2^32,
 * seed >> 32); `row` is the row's index in this call.
 *
 *   base_logits [R, gamma, V] float32
 *   w1          [V, r]  wdtype (embedding table)
 *   w2          [r, V]  wdtype (row j holds the rank-j output weights)
 *   first_prev  [R] int32, in [0, V) (the anchor tokens)
 *   tokens      [R, gamma] int32 (out)
 *   step_logits [R, gamma, V] float32 (out, nullable): the l[v] above
 *   wdtype      DSPARK_BF16 (MFMA path) or DSPARK_F32 (vector-ALU path)
 * Limits: V >= 1, 1 <= r <= 1024 (bf16: r % 32 == 0), 1 <= gamma <= 1024,
 * temperature >= 0 and finite.  Tokens outside [0, V) read as 0 and set
 * DSPARK_STATUS_BAD_TOKEN.
 * ---------------------------------------------------------------------- */
size_t dspark_markov_sample_workspace_bytes(int R, int gamma, int V, int r, int wdtype);
int dspark_markov_sample(const float* base_logits, const void* w1, const void* w2,
                         const int32_t* first_prev, int32_t* tokens, float* step_logits,
                         int R, int gamma, int V, int r, int wdtype,
                         float temperature, uint64_t seed,
                         void* ws, size_t ws_bytes, int32_t* dev_status, void* stream);

/* ------------------------------------------------------------------------
 * Allocation-free Markov sampler, for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, semantics and
 * results as dspark_markov_sample, without (ws, ws_bytes): its per-step
 * argmax keys live in a fixed device array of DSPARK_NOALLOC_SCRATCH_BYTES
 * inside the library (one per GPU the library runs on, held until the
 * process ends, cleared at the start of every call).  It calls no
 * allocator.
 *   - Sizes whose dspark_markov_sample_workspace_bytes(R, gamma, V, r,
 *     wdtype) exceeds DSPARK_NOALLOC_SCRATCH_BYTES return
 *     DSPARK_ERR_WORKSPACE (e.g. R = 128 rows allow gamma <= 64).
 *   - All calls on one GPU share that array: two calls whose executions
 *     overlap on one GPU (different streams, or host threads without
 *     ordering) race and give undefined tokens.  Serialise them.
 *   - DSPARK_ERR_HIP if the array's device address cannot be looked up on
 *     the current device (done once per device, on its first call).
 * ---------------------------------------------------------------------- */
#define DSPARK_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
int dspark_markov_sample_noalloc(const float* base_logits, const void* w1, const void* w2,
                                 const int32_t* first_prev, int32_t* tokens, float* step_logits,
                                 int R, int gamma, int V, int r, int wdtype,
                                 float temperature, uint64_t seed,
                                 int32_t* dev_status, void* stream);

/* ------------------------------------------------------------------------
 * TV-distance accept rate (page 1 §3.9, the paper's Eq. 8; page 2 §3.5 and
 * §3.8.3) and the tau statistic (page 1 §3.10).  Per row of V logits:
 *
 *     accept = clamp(1 - 1/2 * sum_v |softmax(draft)_v - softmax(target)_v|, 0, 1)
 *
 * softmaxes in float32 on the upcast stored values.  If tau != NULL:
 *
 *     tau[b, a] = 1 + sum_k prod_{i <= k} accept[b,a,i] * eval_mask[b,a,i]
 *
 * (eval_mask NULL = all ones).
 *
 *   draft_logits, target_logits [B, A, gamma, V] dtype
 *   accept     [B, A, gamma] float32 (out)
 *   eval_mask  [B, A, gamma] uint8 (nullable; only read for tau)
 *   tau        [B, A] float32 (out, nullable)
 *   dev_status int32 device word (nullable): DSPARK_STATUS_WAIT_TIMEOUT
 * Limits: V >= 2, gamma <= 1024.  Launched cooperatively: the call fails
 * with DSPARK_ERR_HIP if the device cannot host its persistent grid.
 * Accept values of poisoned rows (see dspark_set_wait_limit) stay NaN
 * through the clamp.
 * ---------------------------------------------------------------------- */
size_t dspark_accept_rate_workspace_bytes(int B, int A, int gamma, int V, int dtype);
int dspark_accept_rate(const void* draft_logits, const void* target_logits, float* accept,
                       const uint8_t* eval_mask, float* tau,
                       int B, int A, int gamma, int V, int dtype,
                       void* ws, size_t ws_bytes, int32_t* dev_status, void* stream);

/* Poll limit of the bounded waits inside cooperative grids (the accept rate's
 * exchange of row statistics between the workgroups of a row).  A wait that
 * exceeds it sets DSPARK_STATUS_WAIT_TIMEOUT and the workgroup goes on without
 * waiting: the rows it finishes from then on are NaN and every accept / tau
 * of that call is unreliable.  With a co-resident grid the waits end long
 * before the default limit (2^20 polls); a smaller limit exists so that
 * tests can drive the timeout path with every kernel still exiting normally.
 * polls = 0 restores the default.  Process-wide; takes effect for calls
 * enqueued afterwards. */
void dspark_set_wait_limit(uint32_t polls);

/* ------------------------------------------------------------------------
 * Cumulative-product eval mask (page 1 §3.1 and §3.6).  For block (b, a)
 * and block position k the label index is L = anchor + 1 + k, and
 *
 *     valid(k) = keep[b,a] != 0 && anchor >= 0 && L < seq_lens[b]
 *                && (loss_mask == NULL || loss_mask[b, L] != 0)
 *     eval_mask[b,a,k] = valid(0) && ... && valid(k)
 *
 *   anchor_pos [B, A] int32, keep_mask [B, A] uint8, seq_lens [B] int32
 *   loss_mask  [B, S_stride] uint8 (nullable)
 *   eval_mask  [B, A, gamma] uint8 (out, 0/1)
 * A label index >= S_stride (possible only if seq_lens[b] > S_stride) is
 * invalid and sets DSPARK_STATUS_BAD_LABEL.
 * ---------------------------------------------------------------------- */
int dspark_eval_mask(const int32_t* anchor_pos, const uint8_t* keep_mask,
                     const int32_t* seq_lens, const uint8_t* loss_mask, uint8_t* eval_mask,
                     int B, int A, int gamma, int S_stride,
                     int32_t* dev_status, void* stream);

/* ------------------------------------------------------------------------
 * Teacher-forced Markov block logits (page 1 §3.7: apply_block_logits in
 * training, every position's bias from its given previous token; page 4
 * §3.3; optional soft cap from page 1 §3.12).  For rows n = 0 .. N-1:
 *
 *     logits[n, v] = base[n, v] + sum_j W1[prev[n], j] * W2[j, v]
 *     logits       = softcap * tanh(logits / softcap)      if softcap > 0
 *
 *   base_logits   [N, V] float32 (N = B * A * gamma for a training batch)
 *   w1 [V, r], w2 [r, V]   wdtype (bf16 or float32); r <= 1024
 *   prev          [N] int32 teacher tokens (outside [0, V): row uses token 0
 *                 and DSPARK_STATUS_BAD_TOKEN is set)
 *   logits        [N, V] float32 (out)
 *   argmax_tokens [N] int32 (out, nullable): argmax_v logits, lowest index on ties
 * Workspace from dspark_markov_block_logits_workspace_bytes (8-byte aligned).
 * ---------------------------------------------------------------------- */
size_t dspark_markov_block_logits_workspace_bytes(int N, int V, int r, int wdtype);
int dspark_markov_block_logits(const float* base_logits, const void* w1, const void* w2,
                               const int32_t* prev, float* logits, int32_t* argmax_tokens,
                               int N, int V, int r, int wdtype, float softcap,
                               void* ws, size_t ws_bytes, int32_t* dev_status, void* stream);

/* ------------------------------------------------------------------------
 * Gated and recurrent Markov heads (page 1 §3.7, the paper's Eq. 6; page 4
 * §3.3, the table of head variants).  They replace the vanilla head's W1[x]
 * by a rank-r row E of the position that also sees the backbone hidden
 * state h (length d); the bias is E @ W2 as for the vanilla head:
 *
 *   DSPARK_HEAD_GATED (1):  E = sigmoid(W_g [h; W1[x]]) * W1[x]
 *       whead = W_g [r, d + r] bf16 (input order h, then W1[x])
 *   DSPARK_HEAD_RNN (2):    z = [s; W1[x]; h],  E = tanh(W_o z),
 *       s <- sigmoid(W_g z) * s + (1 - sigmoid(W_g z)) * tanh(W_c z)
 *       whead = [W_g; W_c; W_o] stacked [3, r, 2r + d] bf16
 *
 * No bias terms; the state s is zero at the first position of every block
 * and runs along it.  x is the previous token: for the sampler, the supplied
 * first previous token at position 0 and the token just sampled after
 * that; for the block logits, the caller's teacher token of the position.
 * Precision: the hidden-state part of the maps is a bf16 matrix-core
 * product with float32 accumulation; the recurrent part, the state and E
 * are float32; E is rounded to bf16 for the vocabulary product when W2 is
 * bf16 (float32 W2 uses float32 E).
 *
 *   base_logits  [R, gamma, V] float32
 *   hidden       [R, gamma, d] bf16, 16-byte aligned; d a multiple of 8
 *   w1 [V, r] (16-byte aligned), w2 [r, V]   wdtype (bf16 or float32); r a
 *                multiple of 8, <= 512
 *   whead        as above, bf16, 16-byte aligned
 *
 * dspark_markov_head_sample: the gamma-step sampler with the state carried
 * between steps; token choice, Gumbel noise (seed, row, step, column) and
 * the step_logits output exactly as dspark_markov_sample.
 *   first_prev [R] int32; tokens [R, gamma] int32 (out);
 *   step_logits [R, gamma, V] float32 (out, nullable)
 * dspark_markov_head_block_logits: teacher-forced logits of B blocks
 * (R = B rows of the state, N = B * gamma output rows), soft cap and argmax
 * as dspark_markov_block_logits.
 *   prev [B, gamma] int32 (prev[b, k] is x_{k-1} of position k);
 *   logits [B, gamma, V] float32 (out); argmax_tokens [B, gamma] (out, nullable)
 * Out-of-range previous tokens are replaced by 0 and set
 * DSPARK_STATUS_BAD_TOKEN in *dev_status (nullable).  Workspaces from the
 * matching *_workspace_bytes (256-byte aligned; 0 for an invalid kind).
 * ---------------------------------------------------------------------- */
#define DSPARK_HEAD_GATED 1
#define DSPARK_HEAD_RNN 2
size_t dspark_markov_head_sample_workspace_bytes(int kind, int R, int gamma, int V, int r);
int dspark_markov_head_sample(int kind, const float* base_logits, const void* hidden, const void* w1,
                              const void* w2, const void* whead, const int32_t* first_prev, int32_t* tokens,
                              float* step_logits, int R, int gamma, int V, int r, int d, int wdtype,
                              float temperature, uint64_t seed, void* ws, size_t ws_bytes,
                              int32_t* dev_status, void* stream);
size_t dspark_markov_head_block_logits_workspace_bytes(int kind, int B, int gamma, int V, int r);
int dspark_markov_head_block_logits(int kind, const float* base_logits, const void* hidden, const void* w1,
                                    const void* w2, const void* whead, const int32_t* prev, float* logits,
                                    int32_t* argmax_tokens, int B, int gamma, int V, int r, int d, int wdtype,
                                    float softcap, void* ws, size_t ws_bytes, int32_t* dev_status,
                                    void* stream);

/* ------------------------------------------------------------------------
 * Lossless verify step (page 3's speculative-decoding primer; page 4 §1.2):
 * rejection sampling of R drafted blocks of K tokens against the target.
 * The pages give the outline; the steps are the published speculative-
 * sampling rule: q_k = softmax(draft[k] / T), p_k = softmax(target[k] / T);
 * keep x_k while u_k < p_k(x_k) / q_k(x_k); at the first rejected k draw
 * from max(0, p_k - q_k) normalised; if all K are kept draw one more token
 * from p_K.  T = 0: keep x_k while it is the target's argmax (lowest index
 * on ties); the extra token is that argmax at the stopping position.
 * Random numbers: Philox4x32-10 keyed by seed; u_k = word 0 at counter
 * (k, 0, row, 2) as ((x >> 9) + 1/2) 2^-23; draws are Gumbel-max with word
 * v & 3 at counter (v >> 2, k, row, 1).  float32 arithmetic.
 *
 *   draft_logits  [R, K, V] float32 (the draft's step logits)
 *   target_logits [R, K + 1, V] float32
 *   draft_tokens  [R, K] int32 (any token outside [0, V) sets
 *                 DSPARK_STATUS_BAD_TOKEN in *dev_status, nullable, wherever it
 *                 lies; one that is tested is tested as token 0)
 *   n_accepted    [R] int32 (out): kept drafts, 0 .. K
 *   next_token    [R] int32 (out): the target's token after them
 * Workspace from dspark_verify_workspace_bytes (256-byte aligned).
 * ---------------------------------------------------------------------- */
size_t dspark_verify_workspace_bytes(int R, int K);
int dspark_verify(const float* draft_logits, const float* target_logits, const int32_t* draft_tokens,
                  int32_t* n_accepted, int32_t* next_token, int R, int K, int V, float temperature,
                  uint64_t seed, void* ws, size_t ws_bytes, int32_t* dev_status, void* stream);

/* ------------------------------------------------------------------------
 * L1 (total-variation) alignment loss, its gradient and tau_greedy (page 1
 * §3.9, the paper's Eq. 10, and §3.10; page 4 §4.1).  Row n = position k of
 * block (b, a); p = softmax(draft[n]), q = softmax(target[n]) in float32:
 *
 *     l1[n]   = sum_v |p_v - q_v|
 *     c[n]    = w_k m[n] / sum_n' w_k' m[n'],  w_k = exp(-k / decay)
 *     *loss   = sum_n c[n] l1[n]                        (0 if no m[n] is set)
 *     grad[n, v] = c[n] p_v (s_v - sum_u s_u p_u),  s = sign(p - q)
 *     tau_greedy[b, a] = 1 + sum_k prod_{i <= k} [argmax draft == argmax target]_i m_i
 *
 *   draft_logits, target_logits [B, A, gamma, V] dtype (bf16 or float32)
 *   eval_mask  [B, A, gamma] uint8 (nullable = all valid)
 *   loss       device float[1] (out, required)
 *   row_l1     [B, A, gamma] float32 (out, nullable)
 *   grad       [B, A, gamma, V] float32 (out, nullable: the backward pass is skipped)
 *   tau_greedy [B, A] float32 (out, nullable)
 * Limits: gamma <= 1024, decay > 0.  Workspace from
 * dspark_l1_loss_workspace_bytes(B, A, gamma, V, dtype) (0 for an invalid
 * shape or dtype); its size depends on V and dtype because rows of 16-byte
 * vectors are split over clusters of workgroups that keep per-slice records.
 * A cooperative wait that exceeds dspark_set_wait_limit poisons the rows it
 * served (NaN loss, distances and gradients) instead of hanging.
 * ---------------------------------------------------------------------- */
size_t dspark_l1_loss_workspace_bytes(int B, int A, int gamma, int V, int dtype);
int dspark_l1_loss(const void* draft_logits, const void* target_logits, const uint8_t* eval_mask,
                   float decay, float* loss, float* row_l1, float* grad, float* tau_greedy,
                   int B, int A, int gamma, int V, int dtype,
                   void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Confidence head, prefix survival and the hardware-aware verify-length
 * scheduler (page 1 §3.8; page 4 §3.4 and §5.1).  Row n = position k
 * (1-based) of block (b, a):
 *
 *     c[n]  = sigmoid(weight_h . hidden[n] + weight_e . W1[prev[n]] + bias)
 *     a[n]  = prod_{i <= k} c[block, i]
 *     Theta_l = (1 + sum_{k <= l} a_k) * sps[l],   l = 0 .. gamma
 *     verify_len[b, a] = the last l before Theta first decreases (gamma if never)
 *
 *   hidden     [B, A, gamma, H] hdtype (bf16 or float32)
 *   weight_h   [H] float32; bias a finite float
 *   weight_e   [r] float32 (nullable: no Markov input; then w1 / prev are unused)
 *   w1 [V, r] wdtype, prev [B, A, gamma] int32 (outside [0, V): token 0 and
 *              DSPARK_STATUS_BAD_TOKEN)
 *   sps        [gamma + 1] float32: sps[l] = target steps per second when it
 *              verifies l + 1 tokens
 *   confidence, survival [B, A, gamma] float32 (out, nullable)
 *   verify_len [B, A] int32 (out, required)
 *   theta      [B, A, gamma + 1] float32 (out, nullable)
 * Limits: gamma <= 1024, H >= 1.
 * ---------------------------------------------------------------------- */
int dspark_confidence_schedule(const void* hidden, int hdtype, const float* weight_h, float bias,
                               const void* w1, int wdtype, const int32_t* prev, const float* weight_e,
                               int r, int V, const float* sps, float* confidence, float* survival,
                               int32_t* verify_len, float* theta, int B, int A, int gamma, int H,
                               int32_t* dev_status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
