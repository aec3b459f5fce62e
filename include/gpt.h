/*
 * gpt.h - C ABI of the MI355X (gfx950) GPT-2 training-step library, libgpt.so.
 *
 * One training step, as the pages state the problem:
 *   zero grads -> forward + loss -> backward -> (clip) -> AdamW
 * ("Andrej Karpathy: reproducing GPT-2 from scratch", optimisation loop;
 *  "Implementing an LLM from scratch (CS336) - pretraining", section 3, full loop;
 *  "GPT training" (Zero), training loop).
 *
 * The model is GPT-2: token + learned position embedding, L pre-LN blocks
 * (LayerNorm, causal multi-head attention, residual; LayerNorm, tanh-GELU
 * 4C MLP, residual), final LayerNorm, LM head tied to the token embedding,
 * mean next-token cross-entropy over the B*T positions
 * (lecture, architecture section; Zero page, model, Embedding, Attention,
 *  Transformer Block and output-layer sections).
 *
 * Conventions for every call:
 *   - return 0 on success, a negative GPT_E* code otherwise; the text of the
 *     last error of the calling thread is in gpt_last_error();
 *   - "device" pointers are HIP device addresses, "host" pointers are
 *     ordinary process memory borrowed for the duration of the call only;
 *   - all GPU work is enqueued on the context's HIP stream (hipStream_t
 *     passed as void*; NULL means the default stream), except the weight-
 *     gradient products of the backward and of the tied head, the token sort
 *     of the embedding gradient, the position-embedding gradient, the final
 *     reduction of the bias and LayerNorm gradients, and the AdamW update
 *     itself, which run on a second stream the context owns.  That stream starts from events on the
 *     context stream and is joined back into it (the context stream waits
 *     for it) before gpt_backward's embedding step and at the start of
 *     gpt_make_batch, gpt_forward_loss, gpt_adamw_step, gpt_get_tensor and
 *     gpt_set_tensor; after gpt_adamw_step the next gpt_forward_loss waits
 *     for the update piece by piece (vectors, wte and wpe, then each layer's
 *     matrices) before it first reads them, and gpt_make_batch does not wait
 *     for it.  Work the caller enqueues on the context stream sees every
 *     gradient and updated parameter only after one of these joins (or
 *     gpt_get_tensor).  Only calls that are given a non-NULL host result
 *     pointer synchronise the context stream.
 *   - the library never allocates device memory: the caller owns the
 *     arena and every buffer passed in (gpt_init allocates only host memory,
 *     including two small pinned buffers for the batch windows).
 */
#ifndef GPT_MI355X_H
#define GPT_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* error codes */
#define GPT_OK           0
#define GPT_EINVAL      (-1) /* bad configuration or argument */
#define GPT_ERANGE      (-2) /* token id outside [0, vocab) or window past the stream end */
#define GPT_ENOMEM      (-3) /* arena or workspace too small */
#define GPT_EHIP        (-4) /* a HIP runtime call failed */
#define GPT_ENONFINITE  (-5) /* non-finite loss or gradient norm; AdamW not applied */

/* compute precision of a context (master weights and optimiser state are always fp32) */
#define GPT_F32   0 /* fp32 everywhere (fp32 MFMA) */
#define GPT_BF16  1 /* bf16 GEMM / attention operands, fp32 accumulation, fp32 statistics */

/* tensor kinds for gpt_get_tensor / gpt_set_tensor */
#define GPT_PARAM   0
#define GPT_GRAD    1
#define GPT_ADAM_M  2
#define GPT_ADAM_V  3

typedef struct gpt_ctx gpt_ctx; /* opaque, library-owned host object */

/*
 * Model and batch shape.
 *   n_layer L >= 1, n_embd C, n_head H with C % H == 0; head size D = C/H must be
 *   64 (bf16) or 16, 32, 64 (fp32); C must be a multiple of 64.
 *   vocab V: valid token ids are [0, V).  padded_vocab V_pad >= V rows of the
 *   tied embedding; the extra rows are ordinary softmax classes (lecture,
 *   vocabulary padding: padded rows stay in the output distribution) that
 *   never occur as input or target.
 *   max_seq T_max rows of the position table; seq T <= T_max; batch B.
 *   B*T at most 262144 (the token sort of the embedding gradient takes
 *   16384-token chunks, one workgroup each, and merges them), and
 *   padded_vocab * 2^ceil(log2(B*T)) below 2^32.  GEMM operands are read
 *   with 32-bit byte offsets: B*T * 4C (variant block: B*T * max(3C, 2 d_ff))
 *   and padded_vocab * C, times the element size (4 fp32, 2 bf16), below 2^32.
 */
typedef struct {
  int32_t n_layer, n_embd, n_head;
  int32_t vocab, padded_vocab;
  int32_t max_seq, batch, seq;
  int32_t dtype; /* GPT_F32 or GPT_BF16 */
  int32_t block; /* GPT_BLOCK_GPT2 (0) or GPT_BLOCK_RMS_ROPE_SWIGLU */
  int32_t d_ff;  /* GPT_BLOCK_RMS_ROPE_SWIGLU: SwiGLU hidden width, a multiple of 64 */
  float rope_theta; /* GPT_BLOCK_RMS_ROPE_SWIGLU: RoPE base (CS336 page: 10000), > 0 */
} gpt_config;

/*
 * Block types (CS336 pretraining page, sections 4 and 6, for the second).
 *   GPT_BLOCK_GPT2: pre-LayerNorm blocks with biases, tanh-GELU MLP of width
 *     4C, learned position table, LM head tied to the token embedding.
 *   GPT_BLOCK_RMS_ROPE_SWIGLU: pre-RMSNorm blocks without biases, RoPE on Q
 *     and K (channel pairs (2i, 2i+1) rotated by t * rope_theta^(-2i/D) at
 *     position t), SwiGLU feed-forward (W2 (silu(W1 x) * W3 x)) of width
 *     d_ff, no position table, final RMSNorm and an LM head of its own
 *     ("lm_head", [padded_vocab, C]).  Tensors, in order: wte; per block
 *     h{l}.rms1.g, h{l}.attn.w [3C, C], h{l}.proj.w [C, C], h{l}.rms2.g,
 *     h{l}.w1 [d_ff, C], h{l}.w3 [d_ff, C], h{l}.w2 [C, d_ff]; rmsf.g, lm_head.
 *     RMSNorm epsilon 1e-5.  max_seq bounds the positions RoPE is set up for.
 */
#define GPT_BLOCK_GPT2 0
#define GPT_BLOCK_RMS_ROPE_SWIGLU 1

/* Bytes of device memory gpt_init needs for this configuration (0 if invalid). */
size_t gpt_arena_bytes(const gpt_config* cfg);

/*
 * Validate cfg, carve `arena` (device, at least gpt_arena_bytes(cfg) bytes,
 * 256-byte aligned, owned by the caller and kept alive until gpt_destroy) into
 * parameters, gradients, AdamW moments, bf16 shadow weights, activations and
 * workspaces, and initialise the weights on the device from `seed`
 * (lecture, initialisation: N(0, 0.02) matrices and embeddings, the two
 * residual-output projections of each block N(0, 0.02/sqrt(2L)), biases and
 * LayerNorm beta 0, gamma 1; normals from Philox4x32-10 counters and
 * Box-Muller).  Gradients and moments start at zero, the step counter at 0.
 * Errors: EINVAL (cfg), ENOMEM (arena_bytes too small), EHIP.
 */
int gpt_init(const gpt_config* cfg, void* arena, size_t arena_bytes, void* hip_stream,
             uint64_t seed, gpt_ctx** out);

/* Release the host context (the arena stays the caller's). */
int gpt_destroy(gpt_ctx* ctx);

/*
 * Load one batch ("Chapter 28 Data, evaluation and resume", 28.3: B*T+1
 * contiguous tokens give x = window[:-1] and y = window[1:] viewed as [B, T],
 * each row its own causal window).  host_tokens: the token stream (host,
 * n_tokens int32).  The window starts at `start`.
 * Errors: ERANGE if start < 0, start + B*T + 1 > n_tokens, or any token of the
 * window is outside [0, vocab) (checked on the host before any copy).
 * The call copies the window out of host_tokens before it returns (the
 * caller may reuse that memory at once) and does not wait for the GPU: the
 * window goes through one of two pinned host buffers the context owns
 * (2 * (B*T+1) int32, allocated by gpt_init), and the host-to-device copy is
 * queued on the context stream after the work already there.
 */
int gpt_make_batch(gpt_ctx* ctx, const int32_t* host_tokens, int64_t n_tokens, int64_t start);

/*
 * Cursor rule of the data loader (lecture, data loader and DDP sections;
 * "Chapter 28", 28.3): rank r starts at B*T*r and advances B*T*world per
 * batch; when the next window would run past n_tokens it returns to B*T*r.
 * Pure host arithmetic; returns the next start or a negative code.
 */
int64_t gpt_next_start(int64_t pos, int64_t n_tokens, int32_t B, int32_t T, int32_t rank,
                       int32_t world);

/*
 * Forward pass over the current batch and the mean cross-entropy
 * loss = -(1/BT) sum log P(y | x_<=t) (Zero page, autoregressive objective;
 * CS336 page, section 1).  With loss_scale > 0 it also runs the backward of
 * the fused head + cross-entropy, so that gradients of loss_scale * loss
 * start to accumulate (use 1/steps for gradient accumulation, lecture,
 * gradient accumulation).  loss_scale == 0 runs the forward only.
 * loss_host (nullable): if given, the stream is synchronised and the
 * micro-batch's unscaled mean loss is written there; ENONFINITE if it is not
 * finite.  Every call also appends the loss to a device ring read by
 * gpt_read_losses, without synchronising.
 */
int gpt_forward_loss(gpt_ctx* ctx, float loss_scale, float* loss_host);

/*
 * Backward pass of the last gpt_forward_loss (which must have had
 * loss_scale > 0).  Adds the gradients of loss_scale * loss to the gradient
 * buffers (which are zero after gpt_init and after each gpt_adamw_step);
 * the tied embedding receives the head's and the input embedding's parts.
 */
int gpt_backward(gpt_ctx* ctx);

/*
 * AdamW with decoupled weight decay on every parameter (CS336 page,
 * section 2 AdamW): t <- t + 1; m <- b1 m + (1-b1) g; v <- b2 v + (1-b2) g^2;
 * a = lr sqrt(1-b2^t)/(1-b1^t); p <- p (1 - lr wd); p <- p - a m/(sqrt(v)+eps).
 * Weight decay applies to the 2-D tensors only (lecture, parameter groups).
 * The global gradient L2 norm is always computed; when grad_clip > 0 the
 * gradients are first scaled by min(1, grad_clip/(norm + 1e-6)) (lecture,
 * gradient clipping; CS336 page, section 2 clipping).  Then the bf16 shadow
 * weights are refreshed and the gradients are cleared.
 * grad_norm_host (nullable): if given, synchronise and return the pre-clip
 * norm.  A non-finite norm skips the update on the device (parameters,
 * moments and step counter unchanged, gradients kept for inspection); the
 * call returns ENONFINITE when it synchronises, otherwise the next
 * synchronising call (or gpt_read_losses) reports it.
 */
int gpt_adamw_step(gpt_ctx* ctx, float lr, float beta1, float beta2, float eps,
                   float weight_decay, float grad_clip, float* grad_norm_host);

/*
 * LM head + cross-entropy on caller buffers, no model context (Zero page,
 * output layer: the projection and the cross-entropy as one operator).
 *   X  device [N, C] rows (dtype: fp32 or bf16 bits), W device [V, C],
 *   y  device int32 [N], target ids in [0, V).
 *   loss_dev  device fp32 [1]: mean over N of logsumexp(X W^T)_n - (X W^T)_n,y_n.
 *   dX  device fp32 [N, C] (nullable): gradient of the mean loss w.r.t. X.
 *   dW  device fp32 [V, C] (nullable): gradient w.r.t. W (overwritten).
 *   ws  device workspace of at least gpt_lmhead_ce_ws_bytes(N, V, C, dtype)
 *       bytes (0 for an invalid shape), 256-byte aligned.  It holds the
 *       per-row losses and log-sum-exps, the out-of-range flag and (bf16)
 *       the partial dW sums of the last, split round of the dW kernel.  The loss,
 *       the log-sum-exps and dX come from one pass that streams W through each
 *       workgroup and never stores a logit; dW comes from a second kernel that
 *       streams the rows of X past each block of W rows, recomputing the
 *       logits from the log-sum-exps.  [N, V] is never held.  With the
 *       environment variable GPT_HEAD_DW=gemm (set when both the size and the
 *       call are made) dW instead comes from GEMMs over blocks of vocabulary
 *       columns, and the workspace also holds one block's logit gradient
 *       ([N, cols] in dtype, cols about 128 MB / (N * element size), a
 *       multiple of 256) and a split-K workspace.
 * C must be a multiple of 64 and at most 1792 (bf16) or 1024 (fp32); N and V
 * below 2^31 (bf16: (N + 32) C and (V + 32) C below 2^31).
 * The call synchronises the stream at its end.  A target id outside [0, V)
 * is clamped on the device (never read out of bounds) and the call returns
 * ERANGE; loss and gradients are then not meaningful.
 * Errors: EINVAL (shape, null pointer), ENOMEM (ws too small), ERANGE, EHIP.
 */
size_t gpt_lmhead_ce_ws_bytes(int64_t N, int64_t V, int64_t C, int32_t dtype);
int gpt_lmhead_ce(const void* X, const void* W, const int32_t* y, int64_t N, int64_t V,
                  int64_t C, int32_t dtype, float* loss_dev, float* dX, float* dW, void* ws,
                  size_t ws_bytes, void* hip_stream);

/*
 * gpt_lmhead_ce without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Arguments, results, synchronisation and errors as
 * gpt_lmhead_ce; dW, when asked for, comes from the single-kernel recompute
 * (each workgroup streams all N rows for its vocabulary rows), which needs
 * only the per-row log-sum-exps.  Its per-row losses, log-sum-exps and
 * out-of-range flag live in a static device array of 512 KB + 256 B inside
 * the library (one copy per GPU, held until the process ends), so N is at
 * most 65536; larger N returns EINVAL.  Every call on a GPU shares that
 * GPU's copy and it keeps the last call's contents: calls that overlap on one
 * GPU (other streams, other threads) race, and must be serialised by the
 * caller.  No allocation of any kind is made.
 */
int gpt_lmhead_ce_noalloc(const void* X, const void* W, const int32_t* y, int64_t N,
                          int64_t V, int64_t C, int32_t dtype, float* loss_dev, float* dX,
                          float* dW, void* hip_stream);

/* ---- harness and parity helpers ---- */

/* Number of parameter tensors (2 + 12 L + 2), in the order
 * wte, wpe, per block: ln1.g, ln1.b, attn.w [3C,C] (rows q|k|v), attn.b,
 * proj.w [C,C], proj.b, ln2.g, ln2.b, fc.w [4C,C], fc.b, mlp_proj.w [C,4C],
 * mlp_proj.b; then lnf.g, lnf.b.  Matrices are row-major [out, in]. */
int gpt_num_tensors(const gpt_ctx* ctx);

/* Name (static storage), shape (shape[1] = 0 for vectors) and decay flag of tensor id. */
int gpt_tensor_info(const gpt_ctx* ctx, int id, const char** name, int64_t shape[2],
                    int* decays);

/* Copy tensor `id` of `kind` to / from host fp32 (n must equal its element
 * count).  gpt_set_tensor of a PARAM also refreshes its bf16 shadow.  Both
 * synchronise the stream. */
int gpt_get_tensor(gpt_ctx* ctx, int kind, int id, float* host, int64_t n);
int gpt_set_tensor(gpt_ctx* ctx, int kind, int id, const float* host, int64_t n);

/* The current batch as the device holds it: x, y int32 [B, T] each, to host
 * (synchronises); n must be B*T. */
int gpt_get_batch(gpt_ctx* ctx, int32_t* x_host, int32_t* y_host, int64_t n);

/* Per-position losses of the last forward, [B, T] fp32, to host (synchronises). */
int gpt_get_token_losses(gpt_ctx* ctx, float* host, int64_t n);

/* Losses of the forward calls since the last read (at most `max`, oldest
 * first) to host; returns how many were written (synchronises). */
int gpt_read_losses(gpt_ctx* ctx, float* host, int max);

/* AdamW step counter t (number of applied updates). */
int64_t gpt_step_count(const gpt_ctx* ctx);

/*
 * Set the AdamW step counter t, so that a context restored from a checkpoint
 * (parameters, m and v through gpt_set_tensor) applies the bias corrections
 * of the next update exactly as the uninterrupted run would ("Chapter 28
 * Data, evaluation and resume", 28.6: exact resume needs the optimiser's
 * internal state and the index of the next update; CS336 page, section 3,
 * Checkpoint).  t in [0, 2^31).  Synchronises the stream.
 * Errors: EINVAL, EHIP.
 */
int gpt_set_step_count(gpt_ctx* ctx, int64_t t);

/*
 * Kernel timing for measurement.  gpt_profile_begin(ctx, cls) starts
 * recording HIP events around every launch of kernel class `cls` on the
 * context stream (classes: "gemm_fc_fwd", "attn_fwd", "attn_bwd",
 * "layernorm_fwd", "adamw", "head_gemm", "any"); gpt_profile_end synchronises
 * and returns the summed device time, the launch count, and the algorithmic
 * FLOPs and bytes those launches account for.
 */
int gpt_profile_begin(gpt_ctx* ctx, const char* cls);
int gpt_profile_end(gpt_ctx* ctx, double* total_ms, int64_t* launches, double* flops,
                    double* bytes);

/* Thread-local text of the last error (never NULL). */
const char* gpt_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* GPT_MI355X_H */
