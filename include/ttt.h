/*
 * ttt.h -- C ABI of the MI355X (gfx950) TTT-E2E inner loop.
 *
 * The method (page "TTT-E2E 如何让大模型边用边学", §4.2 and the §4.4
 * pseudo-code): a sliding-window-attention transformer reads a long text in
 * non-overlapping chunks of b tokens.  For each chunk it runs the forward
 * pass with window k, takes the mean next-token cross-entropy of the chunk,
 * back-propagates it into the MLP weights of the last quarter of the blocks
 * only, and applies one gradient step to those weights before the next chunk.
 * Keys/values of earlier chunks are constants (same page, §8 Q1); k >= b
 * (same page, §8 Q4).  One gradient step per update on mlp_layers[-L/4:]
 * (page "突破大语言模型上下文限制的新范式", §2.1); the step is
 * theta <- theta - eta * grad (page "测试时训练：长上下文的持续学习", §2.1.2).
 *
 * Conventions
 *  - Matrices are row-major [out, in]: y = x W^T.
 *  - Batch rows are independent sequences: each has its own fast weights,
 *    key/value window and position.  Token arrays are [batch, n] row-major.
 *  - Every function returns TTT_OK (0) or a negative TTT_E* code and never
 *    throws.  Argument errors are detected before any device work and leave
 *    the context unchanged.  A device error or a non-finite loss poisons the
 *    context: later calls return TTT_ESTATE until ttt_reset().
 *  - A context is not thread-safe; distinct contexts are independent.
 *  - All device memory is owned by the context (allocated through the hook
 *    of ttt_set_allocator when one is installed, else hipMalloc) and is
 *    released by ttt_destroy().  The caller owns every host buffer.
 *  - The library only runs on a gfx950 GPU; without one ttt_create returns
 *    TTT_ENODEV.  There is no CPU fallback.
 */
#ifndef TTT_H
#define TTT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  TTT_OK = 0,
  TTT_EINVAL = -1,     /* bad argument (ids out of range, k < b, n > b, NULL, size mismatch) */
  TTT_ENOMEM = -2,     /* device allocation failed */
  TTT_EDEVICE = -3,    /* HIP runtime error */
  TTT_ESTATE = -4,     /* context poisoned by an earlier device or non-finite error */
  TTT_ENONFINITE = -5, /* a chunk loss was not finite */
  TTT_ENODEV = -6      /* no gfx950 device */
};

enum { TTT_F32 = 0, TTT_BF16 = 1 };

typedef struct ttt_ctx ttt_ctx;

typedef struct {
  int32_t n_layers;   /* L */
  int32_t d_model;    /* d = n_heads * head_dim, head_dim even */
  int32_t n_heads;    /* H (multi-head attention, no grouping) */
  int32_t d_ff;       /* f, SwiGLU hidden width */
  int32_t vocab;      /* V */
  int32_t window;     /* k: a query at position t sees keys t-k < s <= t; requires k >= chunk */
  int32_t chunk;      /* b: tokens per inner-loop step */
  int32_t n_fast;     /* blocks whose MLP is updated: the last n_fast blocks (0 = L/4, at least 1) */
  int32_t batch;      /* B independent rows */
  int32_t dtype;      /* TTT_F32: fp32 everywhere; TTT_BF16: bf16 weights/activations, fp32 accumulate,
                         fp32 residual stream and fp32 master copy of the fast weights */
  int32_t lookahead;  /* chunks whose frozen lower blocks run as one batch (0 = default: 32, at most
                         ceil(max_positions / chunk)); costs (window + lookahead * chunk) ring slots */
  int32_t n_steps;    /* SGD steps per chunk (0 = 1): each chunk is processed n_steps times in a row at the
                         weights the previous step left -- forward, loss, gradient, SGD -- and the loss of
                         the first is reported (page "从KV Cache到权重压缩：大模型持续学习的新范式",
                         §2.2: one to three gradient steps before the next prediction) */
  int64_t max_positions; /* largest absolute position + 1 that will be processed (RoPE table size) */
  double rope_theta;  /* RoPE base; rotate-half pairing (i, i + head_dim/2) */
  double rms_eps;     /* RMSNorm epsilon: g * x / sqrt(mean(x^2) + eps) */
  float lr;           /* SGD step size of the inner loop */
  int32_t dual_mlp;   /* 0: the updated blocks' own MLPs are the fast weights.  1: each updated block keeps
                         its MLP frozen (static) and adds a dynamic SwiGLU MLP of the same width, whose
                         weights (ttt_weights.dyn_*) are the fast weights; both read the block's MLP
                         RMSNorm output and their outputs add (page "从KV Cache到权重压缩：大模型持续学习的新范式",
                         §2.2: a static MLP keeps pretrained knowledge, a dynamic MLP adapts) */
} ttt_config;

/* Host fp32 weight arrays (copied by ttt_create; bf16 contexts round them to
 * nearest-even bf16).  Per-layer fields are arrays of L pointers; the dyn_*
 * fields (read only when cfg.dual_mlp = 1, may be NULL otherwise) are arrays of
 * n_fast pointers, entry j for block L - n_fast + j. */
typedef struct {
  const float* embed;      /* [V, d] */
  const float* final_norm; /* [d] */
  const float* lm_head;    /* [V, d] (untied) */
  const float* const* attn_norm; /* [d] */
  const float* const* wq;        /* [d, d] */
  const float* const* wk;        /* [d, d] */
  const float* const* wv;        /* [d, d] */
  const float* const* wo;        /* [d, d] */
  const float* const* mlp_norm;  /* [d] */
  const float* const* w_gate;    /* [f, d] */
  const float* const* w_up;      /* [f, d] */
  const float* const* w_down;    /* [d, f] */
  const float* const* dyn_gate;  /* [f, d] initial dynamic MLP of each updated block (dual_mlp) */
  const float* const* dyn_up;    /* [f, d] */
  const float* const* dyn_down;  /* [d, f] */
} ttt_weights;

/* Optional device allocator (e.g. PyTorch's caching allocator).  Install it
 * before ttt_create; passing NULLs restores hipMalloc/hipFree.  The hook is
 * process-wide; a context frees with the hook it allocated with. */
typedef void* (*ttt_alloc_fn)(size_t bytes, void* user);
typedef void (*ttt_free_fn)(void* ptr, void* user);
int ttt_set_allocator(ttt_alloc_fn alloc, ttt_free_fn free_fn, void* user);

/* Create a context on the current HIP device (page "TTT-E2E 如何让大模型边用
 * 边学", §9: a model is made from a checkpoint together with the window size
 * and the inner batch b; here the checkpoint is the host weight arrays `w`
 * and window / chunk are fields of `cfg`).  `hip_stream` (hipStream_t, may be
 * NULL for the null stream) is the stream every call enqueues on.  Fast
 * weights start as copies of the given MLP weights of the last n_fast blocks;
 * the key/value window is empty and the position is 0.
 * Errors: TTT_EINVAL for a NULL argument or an invalid configuration (k < b,
 * d % H, head_dim odd or > 128, n_fast out of range, non-finite lr, dual_mlp
 * without its dyn_* arrays ...),
 * TTT_ENODEV without a gfx950 device, TTT_ENOMEM when the allocator (or the
 * installed hook) returns NULL, TTT_EDEVICE for other HIP failures.  On error
 * *out is NULL, nothing stays allocated and ttt_last_error(NULL) says why. */
int ttt_create(const ttt_config* cfg, const ttt_weights* w, void* hip_stream, ttt_ctx** out);

/* One inner-loop step for every row on n (1..chunk) new tokens (page "TTT-E2E
 * 如何让大模型边用边学", §4.4): forward over positions [pos, pos+n) with the
 * window, loss_out[r] = mean over valid targets of -log p(target | prefix)
 * (targets equal to -1 are ignored; a chunk with none has loss 0 and no
 * update), gradient into the fast weights with earlier keys/values constant,
 * one SGD step, pos += n.  tokens, targets: host [batch, n]; ids in [0, V)
 * (targets may be -1).  loss_out: host [batch] or NULL.  The reported loss is
 * the one before the step.  Returns after the step has completed. */
int ttt_prefill_chunk(ttt_ctx* ctx, const int32_t* tokens, const int32_t* targets, int32_t n, float* loss_out);

/* The chunk loop over n_tokens tokens per row: chunks of `chunk` tokens (the
 * last one may be shorter), exactly as repeated ttt_prefill_chunk calls.
 * tokens, targets: host [batch, n_tokens].  losses: host [batch, n_chunks]
 * with n_chunks = ceil(n_tokens / chunk), or NULL.  Synchronous. */
int ttt_prefill(ttt_ctx* ctx, const int32_t* tokens, const int32_t* targets, int64_t n_tokens, float* losses);

/* Same as ttt_prefill with DEVICE arrays: d_tokens, d_targets [batch,
 * n_tokens] int32, d_losses [n_chunks, batch] fp32 (chunk-major) or NULL.
 * Asynchronous on the context's stream; ids are range-checked on the device
 * and a bad id is reported (TTT_EINVAL, context poisoned) by the next
 * ttt_sync.  Inputs must stay valid until the stream reaches this work. */
int ttt_prefill_device(ttt_ctx* ctx, const int32_t* d_tokens, const int32_t* d_targets, int64_t n_tokens,
                       float* d_losses);

/* Wait for the context's stream; report device-side errors (bad ids,
 * non-finite losses of ttt_prefill_device / ttt_score_device work). */
int ttt_sync(ttt_ctx* ctx);

/* Forward and loss only: the chunk losses that ttt_prefill would report for
 * the same tokens, without the backward pass and without any update (the fast
 * weights stay as they are), so the chunks are independent and every block
 * runs as one batch over up to `lookahead` chunks.  The window's keys/values
 * are written and pos advances, exactly as in ttt_prefill.  With window >=
 * the number of positions this is the plain causal transformer, i.e. the
 * full-attention model that page "TTT-E2E 如何让大模型边用边学" §5.1 compares
 * TTT-E2E's latency with; it also scores a text under frozen weights.
 * ttt_score: host arrays and losses as ttt_prefill (synchronous).
 * ttt_score_device: device arrays as ttt_prefill_device (asynchronous; errors
 * and non-finite losses reported by ttt_sync).  Argument errors and poisoning
 * as for ttt_prefill. */
int ttt_score(ttt_ctx* ctx, const int32_t* tokens, const int32_t* targets, int64_t n_tokens, float* losses);
int ttt_score_device(ttt_ctx* ctx, const int32_t* d_tokens, const int32_t* d_targets, int64_t n_tokens,
                     float* d_losses);

/* Greedy generation with test-time training (page "突破大语言模型上下文限制
 * 的新范式", §2.2: an update after every block of generated tokens).  Step j
 * feeds the input (first_input[r], then the previous output) at the next
 * position and outputs the arg-max token (lowest id on ties).  After every
 * `update_every` (1..chunk) steps, those positions are processed again as
 * one inner-loop step whose inputs are what was fed and whose targets are
 * what was output: forward recomputed with earlier keys/values constant
 * (their own window entries overwritten), loss, gradient, SGD.
 * first_input: host [batch]; out_tokens: host [batch, n_new];
 * update_losses: host [batch, n_new / update_every] or NULL.  Synchronous. */
int ttt_generate(ttt_ctx* ctx, const int32_t* first_input, int32_t n_new, int32_t update_every,
                 int32_t* out_tokens, float* update_losses);

/* Copy the fp32 fast weights of row `row` to host `dst`: for each fast block
 * in ascending order, W_gate [f, d], W_up [f, d], W_down [d, f] (with dual_mlp,
 * those of the dynamic MLP).  n_floats
 * must equal 3 * d * f * n_fast.  These are the parameters the inner loop
 * changes (page "TTT-E2E 如何让大模型边用边学", §4.2: only the MLPs of the last
 * quarter of the blocks), i.e. the per-session parameter snapshot of page
 * "突破大语言模型上下文限制的新范式", §5.1.  Waits for the context's stream;
 * works on a poisoned context (it returns what the device holds).  TTT_EINVAL
 * for a bad row, a NULL dst or a size mismatch. */
int ttt_get_fast_weights(ttt_ctx* ctx, int32_t row, float* dst, int64_t n_floats);

/* Per-session snapshot and resume (page "突破大语言模型上下文限制的新范式": a
 * per-session parameter snapshot; resuming also needs the window and the position).
 *
 * ttt_set_fast_weights: host `src` (layout of ttt_get_fast_weights, n_floats = 3 * d
 * * f * n_fast) becomes the fp32 fast weights of row `row`; its bf16 copies are
 * refreshed.  Synchronous.  TTT_EINVAL on a bad row, size or NULL, TTT_ESTATE when
 * poisoned.
 *
 * ttt_state_size: bytes of a whole-context snapshot: a header of 17 int64 (magic,
 * version, batch, n_layers, n_heads, head dim, ring slots, element bytes, fast blocks,
 * d_ff, d_model, position, window, chunk, vocab, bit pattern of rope_theta, dual_mlp),
 * then the fp32 fast weights of every block
 * ([n_fast][batch][3 d f]), then per layer its key/value ring arrays as stored on the
 * device (K, V, V^T, and K^T where the layer keeps it).  -1 for a NULL context.
 * ttt_save_state writes it to host `dst` (nbytes >= ttt_state_size; synchronous;
 * TTT_ESTATE when poisoned; a device-side error of earlier ttt_prefill_device work is
 * reported as ttt_sync would, and poisons, before anything is written).  ttt_load_state reads one back into a context of the same
 * configuration (TTT_EINVAL when the header does not match or nbytes is short): fast
 * weights, window, position; bf16 weight copies refreshed, poisoning and pending device
 * work of ttt_prefill_device cleared.  The caller owns both buffers. */
int ttt_set_fast_weights(ttt_ctx* ctx, int32_t row, const float* src, int64_t n_floats);
int64_t ttt_state_size(const ttt_ctx* ctx);
int ttt_save_state(ttt_ctx* ctx, void* dst, int64_t nbytes);
int ttt_load_state(ttt_ctx* ctx, const void* src, int64_t nbytes);

/* Start a new text (page "TTT-E2E 如何让大模型边用边学", §4.2: every new text
 * starts from the trained initial weights): fast weights back to their initial
 * values, window emptied (pos = 0: no earlier key is visible to the new text; the
 * ring memory is zeroed only after a failure or an unchecked ttt_prefill_device, since
 * the new text reads only slots it writes itself), poisoning cleared.  Synchronous. */
int ttt_reset(ttt_ctx* ctx);

/* Current absolute position of every row (rows advance together). */
int64_t ttt_position(const ttt_ctx* ctx);

/* Kernel timing (tracing): while enabled, every launch of the selected classes
 * below is bracketed by HIP events on the stream it runs on.  ttt_profile_enable
 * takes a bit mask (bit i selects class i, -1 all of them, 0 turns timing off;
 * events cost a little time per launch, so time only what is needed) and clears
 * earlier records; ttt_profile_read synchronizes and returns, per
 * class, the summed device time (ms), the launch count and the algorithmic
 * FLOPs of those launches (matmul = 2 M N K; attention = 4 * head_dim per
 * visible query-key pair, plus 4 * head_dim per in-chunk pair in backward).
 * Classes: GEMMs without a K split by epilogue -- 0 fp32 output, 1 bf16 output,
 * 2 residual add, 3 SwiGLU (gate and up), 4 SwiGLU backward, 5 weight gradient
 * with the fused SGD step (one kernel each) -- 6 K-split GEMMs (kernel + ordered
 * sum), 7 sliding-window attention forward (one kernel), 8 the same with a split
 * key range (kernel + merge), 9 attention backward (all its kernels), 10 attention
 * of one query per head in generation (the kernel over blocks of window keys; their
 * merge is not timed), 11 the q|k|v product with RoPE and the key/value ring writes in its
 * epilogue, 12 the lm_head product with the vocabulary-tiled softmax statistics in its
 * epilogue (the per-row merge after it is not timed). */
enum {
  TTT_PROF_GEMM_F32 = 0, TTT_PROF_GEMM_BF16 = 1, TTT_PROF_GEMM_RESID = 2, TTT_PROF_GEMM_SWIGLU = 3,
  TTT_PROF_GEMM_SWIGLU_BWD = 4, TTT_PROF_GEMM_SGD = 5, TTT_PROF_GEMM_SPLITK = 6, TTT_PROF_SWA_FWD = 7,
  TTT_PROF_SWA_FWD_SPLIT = 8, TTT_PROF_SWA_BWD = 9, TTT_PROF_SWA_DECODE = 10, TTT_PROF_GEMM_QKV_ROPE = 11,
  TTT_PROF_GEMM_LM_CE = 12, TTT_PROF_CLASSES = 13
};
int ttt_profile_enable(ttt_ctx* ctx, int32_t on);
int ttt_profile_read(ttt_ctx* ctx, int32_t n_classes, double* ms, int64_t* counts, double* flops);

void ttt_destroy(ttt_ctx* ctx);

/* Message of the last error of `ctx`, or of the calling thread's last failed
 * ttt_create when ctx is NULL.  Valid until the next call on ctx. */
const char* ttt_last_error(const ttt_ctx* ctx);

#ifdef __cplusplus
}
#endif
#endif /* TTT_H */
