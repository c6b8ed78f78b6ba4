/*
 * moe.h — C ABI of libmoe.so: the Mixture-of-Experts routing, load-balance and
 * dispatch path on AMD Instinct MI355X (gfx950).
 *
 * Page references (title, then section / equation):
 *   [Switch review] "Switch Transformers 논문 리뷰: 1.6조 파라미터 MoE 모델의 Sparse
 *                   Routing 기법 완전 분석" (tildalice.io)
 *   [Switch impl]   "Switch Transformer를 구현 관점에서 읽기: Top-1 라우팅과 Expert 병렬
 *                   처리" (molayo1419.me)
 *   [MoE tour 6]    "MoE环游记：6、最优分配促均衡" (kexue.fm/archives/11619)
 *   [Qwen global]   "Qwen 글로벌-배치 로드 밸런스 MoE LLM 훈련" (agentlenshq.com)
 *
 * Conventions shared by every call
 *   - Arrays are DEVICE pointers (HIP global memory), row-major and contiguous,
 *     owned by the caller.  The library allocates no device memory: scratch
 *     space is the caller's workspace `ws` of at least moe_workspace_size()
 *     bytes, 256-byte aligned.
 *   - The first 53248 bytes of a workspace are control words that must be
 *     zero before the workspace is first used (moe_workspace_init(), or any
 *     zero fill).  Every call leaves them zero again; a call that returns
 *     MOE_ERR_HIP after enqueueing kernels clears them with an asynchronous
 *     fill on its stream (should the stream itself be broken, re-initialise
 *     with moe_workspace_init before reusing the workspace).  Two calls that run at
 *     the same time (different streams) must not share a workspace.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work; they never synchronise with the host.  Results are ready
 *     when the stream reaches that point.
 *   - Every call validates its arguments on the host before any HIP call and
 *     returns MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED / MOE_ERR_WORKSPACE
 *     without touching device memory.  MOE_ERR_HIP reports a failed launch
 *     (hipGetLastError); device faults surface at the caller's next sync.
 *   - Integer outputs are deterministic and bit-reproducible.  Float
 *     reductions use fixed-order trees or exact fixed-point integer sums, so
 *     repeated calls give bit-identical results.
 *   - NaN / Inf inputs are outside the contract; indices stay in [0, n).
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,   /* bad size, null required pointer, inconsistent options */
  MOE_ERR_UNSUPPORTED = 2,   /* valid but beyond the library's limits (e.g. n > 4096) */
  MOE_ERR_WORKSPACE = 3,     /* ws_bytes smaller than moe_workspace_size() */
  MOE_ERR_HIP = 4            /* a kernel launch failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Router score: softmax p_i = e^{h_i}/Σ_j e^{h_j} ([Switch review] "Switch Routing
 * 메커니즘" Step 1) or sigmoid ρ_i = σ(h_i) ([MoE tour 6] "방법 회고"). */
typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score;

/* Gate of a chosen expert: its score (Switch: [Switch review] Step 3; Loss-Free:
 * [MoE tour 6] eq. (1), the bias never enters the gate), or the score divided by
 * the sum over the token's k choices (top-k softmax gating, [Switch review]
 * "Shazeer et al. (2017)의 MoE Layer"). */
typedef enum { MOE_GATE_PROB = 0, MOE_GATE_RENORM = 1 } moe_gate;

/* Balanced-assignment modes ([MoE tour 6] "교대 반복" and "함정에 주의"), with
 * optional flags OR-ed in: MOE_QB_QUANTILE, the quantile form of the page's
 * demo code ("데모 코드": each α and β the 1 − k/n quantile of its row / column
 * with linear interpolation, as numpy computes it on fp32 data); MOE_QB_BIP,
 * α and β clipped at 0 after every step (the demo's comment on BIP). */
typedef enum { MOE_QB_SOLVE = 0, MOE_QB_ONLINE = 1 } moe_qb_mode;
enum { MOE_QB_QUANTILE = 0x10, MOE_QB_BIP = 0x20 };

typedef enum { MOE_EXPERT_IDENTITY = 0, MOE_EXPERT_RELU_FFN = 1 } moe_expert_kind;

/* Problem shape, following the pages' problem statement: m tokens (batch x
 * sequence flattened), d = d_model, n experts, k experts per token. */
typedef struct {
  int64_t m;
  int32_t d;
  int32_t n;
  int32_t k;
  int32_t score;    /* moe_score */
  int32_t gate;     /* moe_gate */
  int32_t x_dtype;  /* moe_dtype of the hidden states x */
} moe_shape;

/* ------------------------------------------------------------------ host helpers */

/* Workspace bytes that every call below needs for this shape (the maximum
 * over calls), with `capacity` the per-expert capacity used by dispatch
 * (-1: no limit) and `d_ff` the expert hidden width (0: no FFN).  Returns 0
 * for an invalid shape. */
size_t moe_workspace_size(const moe_shape* shape, int32_t capacity, int32_t d_ff);

/* Zero-fills the control words of a fresh workspace (asynchronous on stream). */
moe_status moe_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for moe_balance_duals (exact != 0: with the completion);
 * 0 for invalid sizes. */
size_t moe_balance_workspace_size(int64_t m, int32_t n, int32_t k, int32_t exact);

/* Workspace bytes for moe_expert_ffn with at most rows_max rows per expert;
 * 0 for invalid sizes. */
size_t moe_expert_ffn_workspace_size(int32_t n, int32_t rows_max, int32_t d_ff);

/* Expert capacity floor(m · cf / n) on the exact binary value of cf
 * ([Switch review] "Expert Capacity와 토큰 드롭": (tokens per batch / number of
 * experts) x capacity factor).  Returns -1 if m < 0, n < 1, cf < 0 or not
 * finite, or the result exceeds INT32_MAX. */
int32_t moe_capacity(int64_t m, int32_t n, double capacity_factor);

const char* moe_status_str(int32_t status);

/* Library version string and the GPU architecture its kernels target. */
const char* moe_build_info(void);

/* ------------------------------------------------------------------ router */

/* Bytes of the prepared router weight for moe_router_prepare (0 if invalid). */
size_t moe_router_planes_bytes(int32_t d, int32_t n);

/* moe_router_prepare — re-lays the fp32 router weight W_r [d, n] for the bf16
 * matrix-core product of moe_route: three bf16 planes hi, mid, lo with
 * hi + mid + lo == W_r exactly (each plane [n_pad, d_pad], expert-major, zero
 * padded).  Prepare once per weight update and pass the planes to every
 * moe_route call that uses this W_r (for example all micro-batches of a
 * global batch).  planes: device buffer of moe_router_planes_bytes(d, n). */
moe_status moe_router_prepare(int32_t d, int32_t n, const float* w_r, void* planes, void* stream);

/* moe_route — router projection, score, top-k selection and load histogram.
 *   h = x · W_r with x upcast exactly to fp32 and fp32-accurate accumulation
 *   ([Switch review] "Switch Routing 메커니즘" Step 1, "선택적 정밀도 캐스팅":
 *   the router runs in fp32 on bf16 hidden states).  For bf16 x the product
 *   is formed on bf16 matrix cores from an exact three-way bf16 split of W_r.
 *   Selection key: h (no bias; the same order as p or σ(h)), or score + bias
 *   (Loss-Free, [MoE tour 6] eq. (1)).  Ties go to the lower expert index; a
 *   token's k choices are written by descending key.
 * x        [m, d]   fp32 or bf16 (shape->x_dtype)
 * w_r      [d, n]   fp32 router weight
 * w_planes moe_router_prepare(w_r) output, or NULL (then moe_route prepares it
 *          in the workspace on every call)
 * bias     [n]      fp32 or NULL (ranks only; never part of the gate)
 * idx      [m, k]   int32 out: chosen experts
 * gate     [m, k]   fp32 out: gate values (moe_gate)
 * counts   [n]      int32 out: c_j = number of (token, choice) pairs on expert j
 * prob_sum [n]      fp32 out or NULL: Σ_t score_j(t) (softmax p or sigmoid ρ),
 *                   the numerator of P_j ([Switch review] "로드 밸런싱 손실")
 * Limits: 1 <= k <= min(n, 64), n <= 4096, 1 <= d <= 65536, m >= 1. */
moe_status moe_route(const moe_shape* shape, const void* x, const float* w_r, const void* w_planes,
                     const float* bias, int32_t* idx, float* gate, int32_t* counts, float* prob_sum,
                     void* ws, size_t ws_bytes, void* stream);

/* moe_route_noalloc — moe_route for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments and results as moe_route without ws / ws_bytes:
 * the scratch is a static device array of moe_route_noalloc_max_bytes() bytes
 * (16 MiB) that the library holds on each GPU it runs on until the process
 * ends.  Shapes whose moe_route workspace exceeds that return
 * MOE_ERR_UNSUPPORTED (for example n > 256 at large m, whose logits pass
 * through the scratch); the Switch-Base and Loss-Free router shapes fit.  The
 * call allocates nothing.  Every call on one GPU shares that GPU's array, so
 * calls that overlap on one GPU (different streams, host threads) race; calls
 * in order on one stream do not.  The first call on a device also enqueues a
 * small kernel that clears the array's control words. */
size_t moe_route_noalloc_max_bytes(void);
moe_status moe_route_noalloc(const moe_shape* shape, const void* x, const float* w_r, const void* w_planes,
                             const float* bias, int32_t* idx, float* gate, int32_t* counts, float* prob_sum,
                             void* stream);

/* ------------------------------------------------------------------ statistics */

/* moe_stats — load statistics of one (micro-)batch, optional global-batch
 * accumulation and optional Loss-Free bias update.
 *   f_j = c_j / m; P_j = prob_sum_j / m; aux = α · n · Σ_j f_j P_j
 *   ([Switch review] "로드 밸런싱 손실"; for k > 1, f_j still counts the pairs
 *   on expert j per token).  Σ is taken in fp64 in a fixed order.
 *   global_counts[j] += c_j and global_tokens[0] += m ([Qwen global]
 *   "글로벌-배치 로드 밸런스 구현": expert frequencies are gathered over the
 *   global batch).
 *   bias[j] ← fl32(bias[j] − fl32(γ) · sign(c_j · n − m · k)), i.e. the sign of
 *   F_j − 1/n with F_j = c_j/(m·k), evaluated exactly in 64-bit integers
 *   ([MoE tour 6] eq. (2)).  Call this AFTER routing the batch with the old
 *   bias ([MoE tour 6] "함정에 주의").
 * counts [n] int32 in; prob_sum [n] fp32 in or NULL (then P and aux are skipped);
 * f [n] fp32 out or NULL; P [n] fp32 out or NULL; aux [1] fp32 out or NULL;
 * global_counts [n] int64 in/out or NULL; global_tokens [1] int64 in/out or NULL
 * (both or neither); bias [n] fp32 in/out or NULL. */
moe_status moe_stats(int64_t m, int32_t n, int32_t k, const int32_t* counts, const float* prob_sum,
                     float alpha, float* f, float* P, float* aux,
                     int64_t* global_counts, int64_t* global_tokens,
                     float* bias, float gamma, void* stream);

/* moe_route_lossfree — one Loss-Free micro-batch step in one launch: moe_route
 * with the bias as selection offset ([MoE tour 6] eq. (1)), then, in the
 * route's last workgroup, the bias update of eq. (2) and the optional
 * global-batch accumulation, exactly as moe_stats(m, n, k, counts, ...,
 * global_counts, global_tokens, bias, gamma) would do them after the route.
 * Every workgroup reads the bias before the last one updates it, so the
 * update follows the routing as [MoE tour 6] "함정에 주의" requires.
 * Arguments as moe_route, and: bias [n] fp32 in/out (required; routes with
 * the incoming value, holds the updated one afterwards); gamma: the update
 * rate; global_counts [n] int64 in/out and global_tokens [1] int64 in/out, both
 * or neither.  Results (idx, gate, counts, prob_sum, bias, global counts) are
 * bit-identical to moe_route followed by moe_stats.  Limits as moe_route.
 * Errors: MOE_ERR_INVALID_ARG for a missing bias, a non-finite gamma or only
 * one of the two global pointers (nothing is launched); otherwise as moe_route. */
moe_status moe_route_lossfree(const moe_shape* shape, const void* x, const float* w_r, const void* w_planes,
                              float* bias, float gamma, int32_t* idx, float* gate, int32_t* counts,
                              float* prob_sum, int64_t* global_counts, int64_t* global_tokens, void* ws,
                              size_t ws_bytes, void* stream);

/* moe_global_aux — the global-batch balance loss ([Qwen global] "글로벌-배치 로드
 * 밸런스 구현": synchronise f over the global batch, form each micro-batch's loss
 * with it, aggregate).  f^g_j = global_counts_j / global_tokens;
 * losses[t] = α · n · Σ_j f^g_j · P[t, j]; loss_mean = mean_t losses[t].
 * Hybrid ([Qwen global] "효율성과 효과성의 균형": the micro-batch balance loss is
 * added to the global-batch one, with a constant weight of 0.01 that the page's
 * wording can attach to either term): hybrid[t] = global_weight · losses[t] +
 * micro_weight · micro_aux[t], hybrid_mean = mean_t hybrid[t], where micro_aux[t]
 * is micro-batch t's own Switch loss (moe_stats' aux).  (1, 0.01) weights the
 * micro-batch loss, (0.01, 1) the global one.  Sums in fp64.
 * P [nb, n] fp32 (each row a micro-batch's P); f_global [n], losses [nb],
 * loss_mean [1] fp32 out (each may be NULL); micro_aux [nb] fp32 in, needed
 * only for hybrid [nb] / hybrid_mean [1] fp32 out (each may be NULL). */
moe_status moe_global_aux(int32_t n, const int64_t* global_counts, const int64_t* global_tokens,
                          const float* P, int32_t nb, float alpha,
                          float* f_global, float* losses, float* loss_mean,
                          const float* micro_aux, float global_weight, float micro_weight,
                          float* hybrid, float* hybrid_mean, void* stream);

/* ------------------------------------------------------------------ balanced assignment */

/* moe_balance_duals — balanced optimal assignment ([MoE tour 6] "선형계획" eq. (3)/(4):
 * every token takes k experts, every expert exactly q = m·k/n tokens).
 *   QB step ("교대 반복"): α_i ← (k+1)-th largest of fl32(s_i − β);
 *   β_j ← (q+1)-th largest of fl32(s_·j − α) — exact order statistics of fp32
 *   differences, bit-reproducible.
 *   mode SOLVE: start from the given beta, run `iters` QB steps, then
 *     idx = top-k of fl32(s_i − β) (ties: lower index).
 *   mode ONLINE ("함정에 주의"): idx = top-k of fl32(s_i − β_old) FIRST, then one
 *     QB step updates beta (iters must be 1, exact must be 0).
 *   | MOE_QB_QUANTILE: α_i and β_j are the 1 − k/n quantiles of fl32(s_i − β) and
 *     fl32(s_·j − α), interpolated linearly between the two neighbouring order
 *     statistics (fp32 arithmetic, numpy's rule; bit-reproducible).
 *   | MOE_QB_BIP: α and β clipped at 0 after each step.
 *   exact = 1 (SOLVE only): finish with successive shortest paths (min-cost
 *     flow on the expert graph, fp64) from x = top-k(s − β) until every expert
 *     holds exactly q tokens; idx is then the LP optimum (eq. (4), which has an
 *     integral optimum, "극대-극소") and beta the final potentials, an optimal
 *     dual of eq. (8) rounded to fp32.  Requires n <= 64, or n <= 128 with
 *     m <= 65535 and m·(16 + 2k) <= 129024 (MOE_ERR_UNSUPPORTED otherwise).
 * s [m, n] fp32; beta [n] fp32 in/out; idx [m, k] int32 out; counts [n] int32 out;
 * alpha [m] fp32 out or NULL (the last α computed); info [4] int32 out or NULL:
 * {QB steps run, augmentations, 1 if every count == q else 0, 0}.
 * Requires (m·k) % n == 0 and 1 <= k < n. */
moe_status moe_balance_duals(int64_t m, int32_t n, int32_t k, const float* s, float* beta,
                             int32_t iters, int32_t mode, int32_t exact,
                             int32_t* idx, int32_t* counts, float* alpha, int32_t* info,
                             void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for moe_balance_duals_minibatch; 0 for invalid sizes. */
size_t moe_balance_minibatch_workspace_size(int64_t m, int32_t n, int32_t k, int64_t batch_rows);

/* moe_balance_duals_minibatch — β from mini-batches ([MoE tour 6] "함정에 주의",
 * last paragraph: one column selection over all m tokens is too expensive, so the
 * tokens are split into mini-batches, β is computed on each by the same rule and
 * the results are averaged).  The mini-batches are the m / batch_rows blocks of
 * batch_rows consecutive tokens; block b has quota q_b = batch_rows·k/n and its
 * own β, and all blocks run in the same kernel launches.
 *   mode SOLVE: every block starts from the given beta and runs `iters` QB
 *     steps (as moe_balance_duals, on its own tokens); beta ← the mean of the
 *     blocks' β (sum in fp64 in block order, divided by the block count,
 *     rounded once to fp32); then idx = top-k of fl32(s_i − β).
 *   mode ONLINE: idx = top-k of fl32(s_i − β_old) first, then one QB step per
 *     block from β_old and beta ← their mean (iters must be 1).
 *   MOE_QB_QUANTILE / MOE_QB_BIP as for moe_balance_duals (each block's column
 *   quantile is taken over its batch_rows keys).  No exact completion.
 * s [m, n] fp32; beta [n] fp32 in/out; idx [m, k], counts [n] int32 out (the
 * top-k above and its histogram); alpha [m] fp32 out or NULL (the last α, each
 * row's from its own block's β); info [4] int32 out or NULL: {QB steps, 0,
 * 1 if every count == m·k/n else 0, 0}.
 * Requires m % batch_rows == 0, (batch_rows·k) % n == 0, 1 <= k < n; at most
 * 65535 blocks (else MOE_ERR_UNSUPPORTED). */
moe_status moe_balance_duals_minibatch(int64_t m, int32_t n, int32_t k, const float* s, float* beta,
                                       int32_t iters, int32_t mode, int64_t batch_rows,
                                       int32_t* idx, int32_t* counts, float* alpha, int32_t* info,
                                       void* ws, size_t ws_bytes, void* stream);

/* moe_balance_signsgd — sign-gradient steps on the balancing duals ([MoE tour 6]
 * "경사하강" eq. (15)-(17)): the dual's slope in β_j is q − c_j, so each step
 * takes c_j = the number of tokens whose top-k of fl32(s_i − β) holds expert j
 * (ties: lower index) and sets β_j ← fl32(β_j + γ·sign(c_j − q)).  After
 * `iters` steps, idx = top-k of fl32(s_i − β) and counts its histogram.
 * (c_j is the page's count of s_ij − α_i − β_j > 0 whenever a row's k-th and
 * (k+1)-th values differ.)
 * s [m, n] fp32; beta [n] fp32 in/out; gamma >= 0 finite; idx [m, k] int32
 * out; counts [n] int32 out; ws: moe_balance_workspace_size(m, n, k, 0) bytes.
 * Requires (m·k) % n == 0, 1 <= k < n, n <= 256 (else MOE_ERR_UNSUPPORTED). */
moe_status moe_balance_signsgd(int64_t m, int32_t n, int32_t k, const float* s, float* beta, float gamma,
                               int32_t iters, int32_t* idx, int32_t* counts, void* ws, size_t ws_bytes,
                               void* stream);

/* ------------------------------------------------------------------ capacity + dispatch */

/* moe_dispatch — capacity slots in token order and permute-dispatch.
 *   slot(t, r) = number of earlier pairs (t', r') < (t, r) in token-major order
 *   with the same expert; kept ⇔ slot < capacity ([Switch review] "Expert
 *   Capacity와 토큰 드롭": overflow tokens skip the expert and reach the next
 *   layer through the residual).  Kept pairs are gathered expert-major, in
 *   token order inside each expert ([Switch impl] "forward pass에서는 토큰
 *   순서를 두 번 변경한다").
 * Buffer layout (rows of `dispatched`, `row_to_token`):
 *   capacity >= 0: capacity-padded, the per-expert capacity buffer — expert j
 *     owns rows [j·C, (j+1)·C) and fills the first expert_rows[j] of them;
 *     n·C rows in all, unfilled rows untouched;
 *   capacity = -1 (unlimited): compact — expert j's rows follow expert j-1's;
 *     m·k rows at most.
 * capacity: -1 = unlimited, else >= 0.
 * x [m, d] (x_dtype) or NULL when dispatched is NULL; idx [m, k] int32 in;
 * token_to_row [m, k] int32 out (-1 = dropped); drop_mask [m, k] uint8 out or NULL;
 * expert_offsets [n + 1] int32 out: expert j's rows start at expert_offsets[j]
 *   (padded: j·C; compact: the prefix sums, [n] = rows in use);
 * expert_rows [n] int32 out or NULL: rows of expert j (= min(count_j, C));
 * row_to_token [rows] int32 out or NULL (unfilled rows untouched);
 * dispatched [rows, d] (x_dtype) out or NULL: row r = x[row_to_token[r]], bit copy. */
moe_status moe_dispatch(const moe_shape* shape, int32_t capacity, const void* x, const int32_t* idx,
                        int32_t* token_to_row, uint8_t* drop_mask, int32_t* expert_offsets,
                        int32_t* expert_rows, int32_t* row_to_token, void* dispatched,
                        void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ expert FFN */

/* moe_expert_ffn — per-expert ReLU FFN on the dispatched rows ([Switch review]
 * "Switch Layer의 구조": FFN(x) = max(0, x·W1)·W2, one weight set per expert;
 * no biases).  bf16 operands, fp32 accumulation, the hidden activation and
 * the output rounded to bf16 (nearest even).
 * rows_max: a host-known bound on any expert's row count (e.g. the capacity);
 *   the buffers hold n·rows_max rows.
 * expert_offsets [n + 1], expert_rows [n] or NULL, int32 (device, from
 *   moe_dispatch): expert j's rows are [offsets[j], offsets[j] + rows[j]), or
 *   [offsets[j], offsets[j+1]) when expert_rows is NULL (compact layout);
 * dispatched [rows, d] bf16; w1 [n, d_ff, d] bf16 (row f feeds hidden unit f);
 * w2 [n, d, d_ff] bf16 (row c feeds output channel c); y [rows, d] bf16 out
 *   (rows outside every expert's range untouched).
 * Limits: d and d_ff multiples of 32. */
moe_status moe_expert_ffn(int32_t n, int32_t d, int32_t d_ff, int32_t rows_max,
                          const int32_t* expert_offsets, const int32_t* expert_rows, const void* dispatched,
                          const void* w1, const void* w2, void* y,
                          void* ws, size_t ws_bytes, void* stream);

/* moe_expert_weights_pack — for callers that keep the expert weights fixed across many
 * layer calls (inference, or the micro-batches between two weight updates): rewrites
 * an [n][rows][cols] bf16 weight tensor in the Linear layout (w1: rows = d_ff,
 * cols = d; w2: rows = d, cols = d_ff) into the order in which the FFN's
 * weight-stream kernel consumes it as matrix-core operands, so that each wave reads
 * its weights as one contiguous run.  Same values and size (n * rows * cols bf16);
 * the FFN computes bit-identical outputs from either layout.  w and w_packed are
 * distinct caller buffers, 16-byte aligned.  rows % 32 == 0 and cols % 64 == 0, else
 * MOE_ERR_UNSUPPORTED. */
moe_status moe_expert_weights_pack(int32_t n, int32_t rows, int32_t cols, const void* w, void* w_packed,
                                   void* stream);

/* ------------------------------------------------------------------ combine */

/* moe_combine — inverse permute, gate scaling and residual:
 *   out[t] = residual[t] + Σ_{r kept} gate[t, r] · y[token_to_row[t, r]]
 *   in fp32, r in increasing order, rounded once to the output dtype
 *   ([Switch review] Step 3; [Switch impl] pipeline list: restore token order,
 *   multiply by the gate, join the residual path).  A token with no kept pair
 *   gets out[t] = residual[t] bit-exactly.  residual = NULL gives the expert
 *   branch alone.
 * y [rows, d] (y_dtype); gate [m, k] fp32; token_to_row [m, k] int32;
 * residual [m, d] (x_dtype) or NULL; out [m, d] (x_dtype). */
moe_status moe_combine(const moe_shape* shape, const void* y, int32_t y_dtype, const float* gate,
                       const int32_t* token_to_row, const void* residual, void* out, void* stream);

/* ------------------------------------------------------------------ whole layer */

typedef struct {
  int32_t capacity;      /* per-expert capacity, -1 = unlimited */
  int32_t expert_kind;   /* moe_expert_kind */
  int32_t d_ff;          /* FFN hidden width (relu_ffn) */
  float alpha;           /* aux-loss weight */
  /* NULL, or 6 hipEvent_t recorded on the stream at the stage boundaries:
   * [0] start, [1] router weight prepared, [2] routed (with statistics and
   * capacity prefix sums), [3] dispatched, [4] expert done, [5] combined.
   * Any entry may be NULL. */
  void* const* stage_events;
  /* Loss-Free ([MoE tour 6] eqs. (1)-(2)): NULL, or the layer's `bias` argument
   * itself, which the layer then updates in place once this batch is routed,
   * b_j <- b_j - gamma * sign(c_j * n - m * k), as moe_stats would after it. */
  float* update_bias;
  float gamma;
  /* NULL, or [n] / [1] int64 in/out: the global-batch counts and tokens
   * ([Qwen global] "글로벌-배치 로드 밸런스 구현"), both or neither. */
  int64_t* global_counts;
  int64_t* global_tokens;
  /* Nonzero: w1 and w2 are in moe_expert_weights_pack's layout (relu_ffn only; the
   * layer returns MOE_ERR_UNSUPPORTED where its FFN cannot read that layout:
   * d % 256, d_ff % 256 or the rows bound).  The backward takes the plain layout. */
  int32_t weights_packed;
} moe_layer_params;

/* Device output pointers of moe_switch_layer.  `out` is required; every other
 * field may be NULL (then the workspace holds it). */
typedef struct {
  int32_t* idx;            /* [m, k] */
  float* gate;             /* [m, k] */
  int32_t* counts;         /* [n] */
  float* prob_sum;         /* [n] */
  float* f;                /* [n] */
  float* P;                /* [n] */
  float* aux;              /* [1] */
  int32_t* token_to_row;   /* [m, k] */
  uint8_t* drop_mask;      /* [m, k] */
  int32_t* expert_offsets; /* [n + 1] */
  int32_t* expert_rows;    /* [n] */
  int32_t* row_to_token;   /* [rows] (rows as for moe_dispatch: n·C, or m·k without capacity) */
  void* dispatched;        /* [rows, d] x_dtype */
  void* y;                 /* [rows, d] bf16 expert outputs (relu_ffn; ignored for
                              the identity expert, whose output is `dispatched`) */
  void* out;               /* [m, d] x_dtype */
  void* hidden;            /* [rows, d_ff] bf16 hidden activation max(0, D·W1) of the
                              relu_ffn expert (kept for the backward), or NULL */
} moe_layer_outputs;

/* moe_switch_layer — route → stats → capacity + dispatch → expert → combine on one
 * stream, the Switch layer of [Switch impl] (pipeline list) and [Switch review]
 * ("Switch Layer의 구조", "Switch Routing 메커니즘", "Expert Capacity와 토큰
 * 드롭", "로드 밸런싱 손실").  Results equal those of the individual calls.
 * relu_ffn needs bf16 x; identity accepts fp32 or bf16. */
moe_status moe_switch_layer(const moe_shape* shape, const moe_layer_params* params,
                            const void* x, const float* w_r, const void* w1, const void* w2,
                            const float* bias, const moe_layer_outputs* outputs,
                            void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ backward */

/* Saved values of one moe_switch_layer forward (its outputs), read by the backward. */
typedef struct {
  const int32_t* idx;            /* [m, k] chosen experts */
  const float* gate;             /* [m, k] gates */
  const int32_t* counts;         /* [n] selections per expert (f_j = counts_j / m) */
  const int32_t* token_to_row;   /* [m, k], -1 = dropped */
  const int32_t* expert_offsets; /* [n + 1] */
  const int32_t* expert_rows;    /* [n] (capacity layout), or NULL (compact offsets) */
  const void* dispatched;        /* [rows, d] bf16 */
  const void* hidden;            /* [rows, d_ff] bf16 */
  const void* y;                 /* [rows, d] bf16 */
} moe_layer_saved;

/* Gradient outputs (device, fp32, every one required). */
typedef struct {
  float* dx;     /* [m, d] */
  float* dw_r;   /* [d, n] */
  float* dw1;    /* [n, d_ff, d] (zero for experts with no rows) */
  float* dw2;    /* [n, d, d_ff] */
} moe_layer_grads;

/* Workspace bytes for moe_switch_layer_backward; 0 for an invalid shape. */
size_t moe_switch_layer_backward_workspace_size(const moe_shape* shape, int32_t capacity, int32_t d_ff);

/* moe_switch_layer_backward — gradients of L = Σ out ⊙ dout + aux with respect to x, W_r, W1
 * and W2 for one moe_switch_layer forward with softmax scores, gate = the chosen expert's
 * probability and the relu_ffn expert ([Switch review] "Switch Routing 메커니즘" Step 3: the
 * gate multiplies the output, so W_r receives a gradient; [Switch impl] "argmax가 있어도
 * Router를 학습할 수 있는 이유": the chosen id itself gets none; [Switch review] "로드 밸런싱
 * 손실": f_i is constant, P_i carries the balancing loss's gradient).  At the forward's saved
 * values: dY = g·dout (combine transpose, rounded to bf16), dg = <dout, Y>; the expert data and
 * weight gradients on bf16 matrix cores (fp32 accumulation; the ReLU mask is H > 0); the
 * router's logits recomputed in fp32, dh = Σ_r dg_r g_r (e_{i_r} − p) + p ⊙ (c − <p, c>) with
 * c_j = α·n·counts_j/m², then dW_r = xᵀ·dh and dx = dout + (dispatch transpose of dD) + dh·W_rᵀ,
 * all fp32 (the router's products on fp32 matrix cores).  Every reduction has a fixed order.
 * params: capacity, d_ff and alpha as in the forward (expert_kind must be relu_ffn);
 * x [m, d] bf16; w_r [d, n] fp32; w1 [n, d_ff, d], w2 [n, d, d_ff] bf16; dout [m, d] fp32.
 * Requires softmax scores, the prob gate, bf16 x, d and d_ff multiples of 32
 * (else MOE_ERR_UNSUPPORTED / MOE_ERR_INVALID_ARG). */
moe_status moe_switch_layer_backward(const moe_shape* shape, const moe_layer_params* params,
                                     const void* x, const float* w_r, const void* w1, const void* w2,
                                     const moe_layer_saved* saved, const float* dout,
                                     const moe_layer_grads* grads, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
