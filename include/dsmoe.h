/*
 * dsmoe.h - C ABI of the DeepSeekMoE feed-forward layer for one MI355X (gfx950).
 *
 * The layer (sources are cited by page title and section):
 *   - affinity s = sigmoid(x . Wr^T) per token and routed expert
 *     (kaiyunto.com DeepSeek-V3 walkthrough, DeepSeekMoE paragraph);
 *   - a per-expert bias b is added to s for SELECTION ONLY, never to the gate
 *     values (gkm0120.cn DeepSeek-V3 notes, Q3; mhpq.cn "DeepSeek-V3 高效训练
 *     关键技术全景解析" §1.2);
 *   - optional group limit: experts form G groups (one per EP node), a token
 *     may use only its best M groups (same article, §3.1: at most 4 nodes);
 *   - top-K of (s + b) among eligible experts; gates = the selected s divided
 *     by their sum (kaiyunto.com walkthrough);
 *   - y = FFN_shared(x) + sum_k gate_k * FFN_{idx_k}(x), one always-on shared
 *     expert plus K routed experts (mhpq.cn article §1.1); experts are SwiGLU
 *     FFNs without biases;
 *   - after each step, b[e] -= gamma for overloaded experts and += gamma for
 *     underloaded ones (kaiyunto.com walkthrough; mhpq.cn §1.2);
 *   - FP8 variant: E4M3 codes with max-abs scales per 1x128 activation tile
 *     and per 128x128 weight block, fp32 accumulation (gkm0120.cn Q8;
 *     mhpq.cn §4.1).
 *
 * Conventions for every entry point:
 *   - Every pointer argument except `desc`, `w` and `bytes` is a DEVICE
 *     pointer. The caller owns every buffer. The library never allocates,
 *     frees or synchronizes, and keeps no pointer after it returns.
 *   - All work is enqueued on `stream` (NULL = the default stream) and runs
 *     asynchronously. Outputs are fully overwritten, never accumulated into.
 *   - Arguments are validated on the host BEFORE anything is enqueued; on an
 *     error nothing is launched, outputs are untouched and a status other
 *     than MOE_OK is returned; moe_last_error() then holds a message
 *     (thread-local). No C++ exception crosses this boundary. Faults inside
 *     kernels surface at the caller's next synchronization.
 *   - Row-major layouts throughout; base pointers 16-byte aligned.
 *   - Entry points are reentrant; calls that share output or workspace
 *     buffers must not overlap in time.
 */
#ifndef DSMOE_H
#define DSMOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSMOE_ABI_VERSION 2

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size or relation      */
  MOE_ERR_UNSUPPORTED = 2,        /* valid but outside what the kernels do   */
  MOE_ERR_MISALIGNED = 3,         /* a pointer is not 16-byte aligned        */
  MOE_ERR_WORKSPACE_TOO_SMALL = 4,
  MOE_ERR_HIP = 5                 /* a HIP launch or query failed            */
} moe_status;

typedef enum moe_dtype {
  MOE_DT_F32 = 0,
  MOE_DT_BF16 = 1,
  MOE_DT_FP8_E4M3 = 2             /* OCP E4M3FN: bias 7, max 448, no inf     */
} moe_dtype;

/* Shape and precision of one layer call.
 *   T            tokens in the call (>= 0; 0 is a no-op)
 *   d            hidden size
 *   n_experts    E routed experts, 1..512
 *   top_k        K routed experts per token, 1..min(E, 64)
 *   n_groups     G expert groups (1 = no group limit); E % G == 0, G <= 64
 *   topk_groups  M groups a token may use, 1..G; M*E/G >= K
 *   group_topn   a group's score is the sum of its group_topn best biased
 *                scores, 1..min(E/G, 8) (ignored when G == 1)
 *   inter        I, intermediate size of every routed expert
 *   shared_inter Is, intermediate size of the shared expert (0 = none)
 *   act_dtype    dtype of x and y: MOE_DT_F32 or MOE_DT_BF16
 *   w_dtype      expert weights: MOE_DT_F32 (with act F32), MOE_DT_BF16 or
 *                MOE_DT_FP8_E4M3 (both with act BF16)
 *   near_tie_eps a token counts as a near tie when the K-th and (K+1)-th
 *                biased scores of eligible experts differ by <= eps, or the
 *                M-th and (M+1)-th group scores do (fp32 difference).
 *   out_dtype    dtype of the layer output y: MOE_DT_F32 or MOE_DT_BF16 (the
 *                combine's fp32 sum, stored as is or rounded to bf16 once);
 *                y_perm and y_shared keep the activations' dtype. K <= 64
 *                (one lane per selected expert in the routing wave).
 * Divisibility: d, I, Is multiples of 64 for BF16/F32 weights and of 128 for
 * FP8 weights (the GEMMs step through the contraction 64 elements at a time,
 * and an FP8 scale covers 128 of them). The router weights and bias are
 * always fp32. Size limits (the kernels address gathered rows and one expert's
 * weights with 32-bit byte offsets; H and the routed rows are addressed per
 * tile from a 64-bit base): T*d*sizeof(x), one expert's weights, 6*E*d, T*K*4
 * (the int32 selections) and, with FP8 weights, T*(K+1)*max(I,Is)/128*4 (H's
 * scales) must each stay below 2^31 bytes; larger calls return
 * MOE_ERR_UNSUPPORTED. Training (moe_forward_train, moe_backward,
 * moe_backward_fp8) also needs T*max(d, 2*max(I,Is))*2 and
 * 2*max(I,Is)*d*4 below 2^31 bytes. */
typedef struct moe_layer_desc {
  int64_t T;
  int32_t d;
  int32_t n_experts;
  int32_t top_k;
  int32_t n_groups;
  int32_t topk_groups;
  int32_t group_topn;
  int32_t inter;
  int32_t shared_inter;
  int32_t act_dtype;
  int32_t w_dtype;
  float near_tie_eps;
  int32_t out_dtype;
} moe_layer_desc;

/* Expert weights (device pointers, w_dtype elements, row-major):
 *   w13  [E, 2I, d]  rows 0..I-1 gate projection W1, rows I..2I-1 up W3
 *   w2   [E, d, I]   down projection
 *   ws13 [2Is, d], ws2 [d, Is]  shared expert (NULL when Is == 0)
 * FP8 only, fp32 scales of the 128x128 blocks (128 output rows x 128 input
 * columns), as written by moe_quantize_fp8_blocks:
 *   w13_scale [E, 2I/128, d/128], w2_scale [E, d/128, I/128],
 *   ws13_scale [2Is/128, d/128], ws2_scale [d/128, Is/128]. */
typedef struct moe_weights {
  const void* w13;
  const void* w2;
  const void* ws13;
  const void* ws2;
  const float* w13_scale;
  const float* w2_scale;
  const float* ws13_scale;
  const float* ws2_scale;
} moe_weights;

/* Bytes of workspace that deepseek_moe_forward needs for `desc`; this also
 * covers moe_gate, moe_route_from_logits and moe_expert_ffn. Host only. */
moe_status moe_workspace_size(const moe_layer_desc* desc, size_t* bytes);

/* Router and routing, steps affinity -> bias -> group limit -> top-K -> gates
 * -> per-expert counts (sources above).
 *   x          [T, d] act_dtype
 *   w_router   [E, d] fp32;  bias [E] fp32
 *   logits     [T, E] fp32 OUT, optional (NULL = kept in the workspace). The
 *              router product is exact-input fp32 accumulation; the routing
 *              that follows is a fixed sequence of IEEE fp32 operations, so
 *              it is reproducible bit for bit from these logits.
 *   topk_idx   [T, K] int32 OUT, slot order = biased score descending, ties
 *              to the lower expert id
 *   topk_gate  [T, K] fp32 OUT, gates in slot order (sum to 1)
 *   counts     [E] int32 OUT, tokens routed to each expert
 *   near_tie   [1] int32 OUT, optional: number of near-tie tokens
 *   ws         workspace of >= moe_workspace_size bytes */
moe_status moe_gate(const moe_layer_desc* desc, const void* x, const float* w_router,
                    const float* bias, float* logits, int32_t* topk_idx, float* topk_gate,
                    int32_t* counts, int32_t* near_tie, void* ws, size_t ws_bytes,
                    hipStream_t stream);

/* The routing half of moe_gate on caller-supplied fp32 logits [T, E]. */
moe_status moe_route_from_logits(const moe_layer_desc* desc, const float* logits,
                                 const float* bias, int32_t* topk_idx, float* topk_gate,
                                 int32_t* counts, int32_t* near_tie, hipStream_t stream);

/* Per-expert token segments sized to the routed data (mhpq.cn §3.1: memory
 * opened for the data actually sent), by a stable counting sort.
 *   topk_idx [T, K], counts [E] IN (from moe_gate)
 *   offsets  [E+1] int32 OUT, exclusive prefix sum of counts
 *   perm     [T*K] int32 OUT, token ids, expert-major, ascending token order
 *            inside each expert
 *   inv      [T, K] int32 OUT, position of pair (t, k) in perm
 *   x        [T, d] act_dtype IN, only read when x_perm != NULL
 *   x_perm   [T*K, d] OUT, optional: gathered rows x[perm]; with FP8 weights
 *            these are E4M3 codes of 1x128 tiles and x_perm_scale [T*K, d/128]
 *            fp32 receives their scales. */
moe_status moe_permute(const moe_layer_desc* desc, const int32_t* topk_idx,
                       const int32_t* counts, const void* x, int32_t* offsets, int32_t* perm,
                       int32_t* inv, void* x_perm, float* x_perm_scale, hipStream_t stream);

/* Grouped expert FFNs (SwiGLU experts, fine-grained routed experts plus one
 * shared expert: mhpq.cn §1.1; FP8 GEMMs with 1x128 / 128x128 scaling:
 * mhpq.cn §4.1, gkm0120.cn Q8): for every expert e, rows offsets[e] ..
 * offsets[e+1]-1
 *   y_perm[r] = W2_e (silu(W1_e a_r) * (W3_e a_r)),
 * with a_r = x_perm[r] when x_perm != NULL, else x[perm[r]]; and for every
 * token y_shared[t] = the shared expert applied to x[t].
 *   y_perm [T*K, d], y_shared [T, d] OUT: fp32 with F32 weights, else bf16.
 *   With FP8 weights, x is quantized in 1x128 tiles, H in 1x128 tiles of the
 *   intermediate axis; fp32 accumulation with the block scales applied per
 *   128-wide slice of the contraction. */
moe_status moe_expert_ffn(const moe_layer_desc* desc, const moe_weights* w, const void* x,
                          const int32_t* perm, const void* x_perm, const float* x_perm_scale,
                          const int32_t* offsets, void* y_perm, void* y_shared, void* ws,
                          size_t ws_bytes, hipStream_t stream);

/* Gated combine: y[t] = y_shared[t] + sum_k topk_gate[t,k] * y_perm[inv[t,k]],
 * fp32 accumulation in slot order, y in out_dtype; y_perm and y_shared in
 * the activations' dtype. The shared expert is ungated and every token's K
 * routed outputs are weighted by its gates (mhpq.cn "DeepSeek-V3 高效训练关键
 * 技术全景解析" §1.1; kaiyunto.com walkthrough, DeepSeekMoE paragraph).
 * y_shared may be NULL (no shared expert). */
moe_status moe_combine(const moe_layer_desc* desc, const void* y_perm, const int32_t* inv,
                       const float* topk_gate, const void* y_shared, void* y,
                       hipStream_t stream);

/* Bias update from this step's loads (in place): with balanced load T*K/E,
 * b[e] -= gamma if counts[e]*E > T*K, b[e] += gamma if counts[e]*E < T*K,
 * unchanged otherwise; fp32 arithmetic (kaiyunto.com walkthrough, DeepSeekMoE
 * paragraph: bias update speed gamma; mhpq.cn §1.2: applied every step). The
 * only call that mutates an input. */
moe_status moe_bias_update(const moe_layer_desc* desc, const int32_t* counts, float gamma,
                           float* bias, hipStream_t stream);

/* The whole layer (the DeepSeekMoE feed-forward layer of the preamble's
 * sources: kaiyunto.com walkthrough, DeepSeekMoE paragraph; mhpq.cn §1.1,
 * §1.2, §3.1, §4.1): moe_gate, the counting sort, moe_expert_ffn (rows
 * gathered from x inside the GEMM) and moe_combine, enqueued back to back. It
 * does NOT update the bias: call moe_bias_update with `counts` afterwards.
 *   y [T, d] out_dtype OUT; topk_idx, topk_gate, counts OUT as in moe_gate;
 *   near_tie and logits optional OUT. */
moe_status deepseek_moe_forward(const moe_layer_desc* desc, const void* x,
                                const float* w_router, const float* bias, const moe_weights* w,
                                void* y, int32_t* topk_idx, float* topk_gate, int32_t* counts,
                                int32_t* near_tie, float* logits, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/* For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. deepseek_moe_forward with the same arguments and results, except
 * that its workspace is a fixed array of MOE_NOALLOC_SCRATCH_BYTES inside the
 * library instead of a caller buffer; the call allocates and frees nothing.
 *   - Each GPU the library runs on holds its own copy of that array from the
 *     first call on it until the process ends; the first call on a device
 *     looks its address up (hipGetSymbolAddress), with that device current.
 *   - A call whose workspace (moe_workspace_size) exceeds the array returns
 *     MOE_ERR_WORKSPACE_TOO_SMALL before anything is enqueued (at the V3 shape,
 *     d = 7168 and 256 experts of 2048 plus a shared one, calls of up to 532
 *     tokens fit with bf16 weights and up to 552 with FP8 weights).
 *   - Every call on one GPU uses the same array: calls on one GPU that
 *     overlap in time (e.g. on different streams without ordering between
 *     them) race and must be serialized by the caller. Nothing in the array
 *     needs to start zeroed: every buffer the forward keeps there is written
 *     before it is read, on every call. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
moe_status deepseek_moe_forward_noalloc(const moe_layer_desc* desc, const void* x,
                                        const float* w_router, const float* bias,
                                        const moe_weights* w, void* y, int32_t* topk_idx,
                                        float* topk_gate, int32_t* counts, int32_t* near_tie,
                                        float* logits, hipStream_t stream);

/* FP8 weight preparation, once per weight set: n_mats matrices [rows, cols]
 * of `src_dtype` (MOE_DT_F32 or MOE_DT_BF16) -> E4M3 codes q (same shape) and
 * fp32 scales [n_mats, rows/128, cols/128]. Per 128x128 block: amax = max|w|;
 * amax == 0 gives scale 1 and zero codes; else scale = amax/448 and
 * q = e4m3(w * (448/amax)), round to nearest even, saturating at 448
 * (gkm0120.cn Q8; mhpq.cn §4.1). rows, cols multiples of 128. */
moe_status moe_quantize_fp8_blocks(const void* src, int32_t src_dtype, int64_t n_mats,
                                   int32_t rows, int32_t cols, uint8_t* q, float* scale,
                                   hipStream_t stream);

/* The same rule on 1x128 tiles of each row: src [n, cols] -> q [n, cols],
 * scale [n, cols/128]. cols a multiple of 128. */
moe_status moe_quantize_fp8_rows(const void* src, int32_t src_dtype, int64_t n, int32_t cols,
                                 uint8_t* q, float* scale, hipStream_t stream);

/* ---- Training: forward that keeps tensors for the backward, and the backward
 *
 * bf16 activations with bf16 weights (moe_backward) or FP8 weights
 * (moe_backward_fp8); other dtypes: MOE_ERR_UNSUPPORTED.
 * The backward differentiates the layer for the selection its forward made
 * (top-K is piecewise constant in every parameter): with the gates
 * g = s / S over the selected sigmoid scores (kaiyunto.com walkthrough,
 * DeepSeekMoE paragraph), gradient flows to the selected router logits
 * through the normalisation and the sigmoid, and from there to x and the
 * router weights; the selection bias receives none, since it is adjusted by
 * the load rule instead (mhpq.cn §1.2). Weight gradients are fp32: the pages
 * keep weight gradients in high precision (mhpq.cn §4.1). Intermediates are
 * bf16 with fp32 accumulation, like the forward's. */

/* Tensors the training forward writes for the backward (device pointers,
 * caller-owned; TK = T*K, ldh = max(I, Is); rows 0..TK-1 are the routed
 * rows in permuted order, rows TK..TK+T-1 the shared expert's):
 *   logits [T, E] fp32, topk_idx [T, K] int32, topk_gate [T, K] fp32,
 *   counts [E] int32, offsets [E+1] int32, perm [TK] int32, inv [T, K] int32
 *     as in moe_gate / moe_permute;
 *   h      [TK + T, ldh] bf16, silu(a) * b, the down projection's input;
 *   gu     [TK + T, 2 ldh] bf16, the pre-activations a = x W1^T in columns
 *          [0, Ig) and b = x W3^T in [Ig, 2 Ig), Ig = I for routed rows and
 *          Is for shared rows;
 *   y_perm [TK, d] bf16, the routed experts' outputs before gating. */
typedef struct moe_saved {
  float* logits;
  int32_t* topk_idx;
  float* topk_gate;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv;
  void* h;
  void* gu;
  void* y_perm;
} moe_saved;

/* deepseek_moe_forward that also fills `saved` (every field required; h and
 * gu have TK + T rows when Is > 0, TK rows otherwise). Same workspace as
 * deepseek_moe_forward. With FP8 weights the forward is the FP8 one (its
 * down projection reads H in E4M3); saved.h then holds H in bf16 and
 * saved.gu the fp32-accumulated pre-activations in bf16. */
moe_status moe_forward_train(const moe_layer_desc* desc, const void* x, const float* w_router,
                             const float* bias, const moe_weights* w, void* y,
                             const moe_saved* saved, int32_t* near_tie, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/* Gradients of the layer (fp32, device pointers, fully overwritten):
 *   dw13 [E, 2I, d], dw2 [E, d, I], dws13 [2Is, d], dws2 [d, Is]
 *   (the shared ones NULL when Is == 0), dw_router [E, d]. An expert that
 *   received no token gets zero gradients. */
typedef struct moe_grads {
  float* dw13;
  float* dw2;
  float* dws13;
  float* dws2;
  float* dw_router;
} moe_grads;

/* Bytes of workspace moe_backward (bf16 weights) or moe_backward_fp8 (FP8
 * weights) needs for `desc`. Host only. */
moe_status moe_backward_workspace_size(const moe_layer_desc* desc, size_t* bytes);

/* Backward of the layer from the output gradient dy [T, d] bf16:
 *   dx [T, d] bf16 OUT, the input gradient (experts, shared expert and router);
 *   g  OUT, the weight gradients;
 * x, w_router, w: the forward's inputs (the weights in their forward layout);
 * saved: what moe_forward_train wrote. */
moe_status moe_backward(const moe_layer_desc* desc, const void* x, const float* w_router,
                        const moe_weights* w, const moe_saved* saved, const void* dy, void* dx,
                        const moe_grads* g, void* ws, size_t ws_bytes, hipStream_t stream);

/* Transposed copies of block-quantized FP8 weights, for the FP8 backward:
 * q [n_mats, rows, cols] E4M3 codes with scales [n_mats, rows/128,
 * cols/128] (as moe_quantize_fp8_blocks writes them) -> qt [n_mats, cols,
 * rows] and scale_t [n_mats, cols/128, rows/128]. A 128x128 block of W is a
 * block of W^T with the same scale, so this is exactly the block
 * quantization of the transposed matrices (mhpq.cn "DeepSeek-V3 高效训练
 * 关键技术全景解析" §4.1: 128x128 weight blocks). rows, cols multiples of
 * 128. Weight preparation: once per weight set. Caller-owned device buffers;
 * errors: MOE_ERR_INVALID_ARGUMENT (sizes, NULL), MOE_ERR_MISALIGNED,
 * MOE_ERR_UNSUPPORTED (more than 2^31 64x64 tiles); nothing is enqueued
 * on error. */
moe_status moe_transpose_fp8_blocks(const uint8_t* q, const float* scale, int64_t n_mats,
                                    int32_t rows, int32_t cols, uint8_t* qt, float* scale_t,
                                    hipStream_t stream);

/* Backward of the FP8 layer (bf16 activations, E4M3 weights): the forward
 * computes in E4M3, the backward in E5M2 (10100.com DeepSeek-V3 technical
 * report article, FP8 paragraph), with 1x128 tiles for activations and
 * gradients and the 128x128 weight blocks (mhpq.cn §4.1), fp32 accumulation.
 * Every GEMM of the backward contracts FP8 operands quantized along its own
 * contraction axis:
 *   - input gradients: the gradient rows (gated output gradients, then
 *     [da | db]) in E5M2 1x128 tiles, times the forward's E4M3 weights read
 *     through the transposed copies `wt` (w13 [E, d, 2I] = [W1; W3]^T, w2
 *     [E, I, d] = W2^T, ws13 [d, 2Is], ws2 [Is, d] and their scales, from
 *     moe_transpose_fp8_blocks);
 *   - weight gradients: contraction over each expert's tokens, both
 *     operands in 128x1 tiles (128 consecutive tokens of the segment per
 *     channel): dY and [da | db] in E5M2, H and x in E4M3.
 * The gates, the router and the combine stay in high precision, as in
 * moe_backward. x, w_router, w, saved, dy, dx, g as in moe_backward (saved
 * from moe_forward_train with the same FP8 weights). ws: ws_bytes >=
 * moe_backward_workspace_size(desc). Errors (nothing is enqueued):
 * MOE_ERR_UNSUPPORTED for weights other than E4M3 or sizes past the
 * training limits, MOE_ERR_INVALID_ARGUMENT for NULL buffers,
 * MOE_ERR_MISALIGNED, MOE_ERR_WORKSPACE_TOO_SMALL. */
moe_status moe_backward_fp8(const moe_layer_desc* desc, const void* x, const float* w_router,
                            const moe_weights* w, const moe_weights* wt, const moe_saved* saved,
                            const void* dy, void* dx, const moe_grads* g, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/* ---- Sequence-level balance loss of the router
 *
 * The training-techniques article (mhpq.cn "DeepSeek-V3 高效训练关键技术全景
 * 解析" §1.2) adds a per-sequence balance loss so that the tokens of one
 * sequence do not concentrate on a few experts, and gives no formula. For
 * each sequence of seq_len = L consecutive tokens (T = n_seq * L), with the
 * layer's fp32 logits u and its selection topk_idx:
 *   s = sigmoid(u) over all E experts, s'_ti = s_ti / sum_j s_tj (1/E for a
 *   token whose fp32 scores are all zero: it then gets no gradient);
 *   P_i = mean over the sequence of s'_ti;
 *   f_i = E / (K L) * (routed slots of expert i in the sequence), which is 1
 *   at perfect balance; loss = alpha * sum_i f_i P_i.
 * f is piecewise constant, so the gradient flows through P to u, and from
 * u = x W_r^T to x and W_r. The gradients are those of the sum of the
 * sequences' losses. bf16 activations only (MOE_ERR_UNSUPPORTED otherwise);
 * the two products du^T x and du W_r run on bf16 copies of du and W_r with
 * fp32 accumulation. */

/* Bytes of workspace moe_seq_balance_loss needs for `desc` and seq_len.
 * Host only. */
moe_status moe_seq_balance_workspace_size(const moe_layer_desc* desc, int32_t seq_len,
                                          size_t* bytes);

/* seq_len >= 1 dividing T; alpha finite. In (device pointers):
 *   x [T, d] bf16, w_router [E, d] fp32, logits [T, E] fp32 and topk_idx
 *   [T, K] int32 (entries in [0, E)) as the forward wrote them.
 * Out (fully overwritten):
 *   loss [T / seq_len] fp32, one value per sequence;
 *   dlogits [T, E] fp32, dloss/du (optional, NULL to skip);
 *   dx [T, d] fp32, dloss/dx;  dw_router [E, d] fp32, dloss/dW_r.
 * T == 0: only dw_router is written (zeros); the T-sized pointers may be
 * NULL. */
moe_status moe_seq_balance_loss(const moe_layer_desc* desc, int32_t seq_len, float alpha,
                                const void* x, const float* w_router, const float* logits,
                                const int32_t* topk_idx, float* loss, float* dlogits, float* dx,
                                float* dw_router, void* ws, size_t ws_bytes, hipStream_t stream);

/* Timing hook for benchmarks (thread-local setting). With n_events >= 6,
 * deepseek_moe_forward records events[0..5] on its stream: before the router,
 * after routing, right before the gate/up GEMM, after it, after the down GEMM
 * and after the combine. events == NULL or n_events == 0 turns it off. The
 * events stay owned by the caller. */
moe_status moe_profile_events(const hipEvent_t* events, int32_t n_events);

const char* moe_status_string(moe_status s);
const char* moe_last_error(void);
int moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSMOE_H */
