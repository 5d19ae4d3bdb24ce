/*
 * gptmi — one decoder-only GPT training step on an MI355X (gfx950) GPU.
 *
 * C ABI over hand-written HIP kernels.  The operations follow the pages that
 * define the model:
 *   [nanoGPT]  "nanoGPT — Karpathy's minimal GPT pretraining repo", sections
 *              "model.py — the GPT" (GPTConfig, Block, CausalSelfAttention,
 *              MLP, LayerNorm, weight tying) and "train.py — the loop"
 *              (shifted targets, mean loss, gradient accumulation).
 *   [nanochat] "Train your own ChatGPT", section 6.2, paragraph on
 *              loss_eval.py (bits per byte with a token_bytes table).
 *   [d20]      "nanochat-d20-chat — a chat model trained from scratch",
 *              Architecture row (RoPE + QK-norm, parameter-free norms).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers unless stated otherwise.  The
 *    caller allocates and owns every buffer (weights, activations, saved
 *    activations, workspace, gradients).  The library never allocates or
 *    frees device memory, never synchronises the stream, and keeps no state
 *    between calls apart from a thread-local error message, the opt-in
 *    trace hooks' event pool (gpt_trace_begin) and the fixed device scratch
 *    of gpt_adamw_step_noalloc (documented with it).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every kernel of a call is enqueued on it in order.
 *  - Activations are row-major [N, C] with N = B*T tokens, row n = b*T + t.
 *    Storage type is cfg->dtype (bf16 or fp32); arithmetic accumulates in
 *    fp32.  Parameter gradients are always fp32.
 *  - Linear weights use the nn.Linear layout [out, in]: y = x W^T + b.
 *    w_qkv is [3C, C] with row blocks q | k | v; head h owns rows
 *    [h*D, (h+1)*D) of each block (D = C / n_head).
 *  - Outputs must not alias inputs.  `accumulate` = 0 overwrites gradient
 *    outputs, 1 adds to them (gradient accumulation over micro-steps).
 *  - Every entry point validates its arguments before enqueuing any work;
 *    on error it returns a non-zero status, writes nothing, and leaves a
 *    message for gpt_last_error().
 *  - Row and column extents must be multiples of 8 elements for bf16
 *    storage (C, 3C, 4C) so rows stay 16-byte aligned; device pointers
 *    must be 16-byte aligned.
 */
#ifndef GPTMI_H
#define GPTMI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define GPT_OK              0
#define GPT_ERR_INVALID     1  /* null pointer, non-positive size, bad config  */
#define GPT_ERR_UNSUPPORTED 2  /* valid but not implemented (head_dim, dtype)  */
#define GPT_ERR_WORKSPACE   3  /* ws_bytes smaller than required               */
#define GPT_ERR_HIP         4  /* a HIP launch/runtime call failed             */

#define GPT_DTYPE_FP32 0
#define GPT_DTYPE_BF16 1
#define GPT_NORM_LAYERNORM 0
#define GPT_NORM_RMSNORM   1

/* Model configuration: nanoGPT's GPTConfig (block_size, vocab_size,
 * n_layer, n_head, n_embd, bias) plus the fields of the nanochat form. */
typedef struct gpt_config {
  int32_t n_layer;
  int32_t n_head;
  int32_t n_embd;
  int32_t block_size;  /* max T                                          */
  int32_t vocab_size;
  int32_t bias;        /* 1: Linear biases and LayerNorm bias            */
  int32_t norm;        /* GPT_NORM_LAYERNORM (gain [+bias]) or RMSNORM    */
  int32_t rope;        /* 0: learned positions (wpe, added in embed)
                          1: rotary embedding on q, k: pairs (i, i+D/2)
                             rotated by t * rope_base^(-2i/D)            */
  int32_t qk_norm;     /* 1: parameter-free RMSNorm of q and k over D     */
  float   rope_base;
  float   norm_eps;    /* eps of every norm (LayerNorm, RMSNorm, QK-norm) */
  int32_t dtype;       /* GPT_DTYPE_BF16 or GPT_DTYPE_FP32 storage        */
  int32_t attn_window; /* 0: causal attention over all earlier positions;
                          W > 0: position i attends to i-W+1 .. i only (the
                          sliding windows of the "SSSL" layer pattern,
                          [nanochat] 6.2; per-layer windows are per-call
                          configs).  W >= T is the full causal mask.      */
  int32_t fp8;         /* 1: the four Linear layers of gpt_block_fwd/bwd run
                          as FP8 GEMMs ([nanochat] 6.2, FP8 paragraph):
                          activations and weights E4M3, gradients E5M2, each
                          quantized from its bf16 value with a dynamic
                          per-tensor scale (fmt_max / amax), fp32
                          accumulation; both backward matmuls in FP8 too.
                          bf16 storage and n_embd % 16 == 0 required.  0:
                          bf16 GEMMs.                                      */
} gpt_config;

/* Block parameters (device pointers, storage dtype).  Absent ones are NULL:
 * LayerNorm gains are required for norm = LAYERNORM, biases iff bias = 1. */
typedef struct gpt_block_weights {
  const void *ln1_w, *ln1_b;   /* [C]                 */
  const void *w_qkv, *b_qkv;   /* [3C, C], [3C]       */
  const void *w_o, *b_o;       /* [C, C],  [C]        */
  const void *ln2_w, *ln2_b;   /* [C]                 */
  const void *w_fc, *b_fc;     /* [4C, C], [4C]       */
  const void *w_proj, *b_proj; /* [C, 4C], [C]        */
} gpt_block_weights;

/* Block parameter gradients, fp32, same shapes; NULL where the parameter is
 * absent. */
typedef struct gpt_block_grads {
  float *ln1_w, *ln1_b, *w_qkv, *b_qkv, *w_o, *b_o;
  float *ln2_w, *ln2_b, *w_fc, *b_fc, *w_proj, *b_proj;
} gpt_block_grads;

/* Bytes of the `saved` buffer that gpt_block_fwd fills and gpt_block_bwd
 * reads for a batch of B sequences of length T.  0 on invalid input. */
size_t gpt_block_saved_bytes(const gpt_config* cfg, int B, int T);

/* Workspace bytes that suffice for every entry point below at this config
 * and batch shape (lm_head_xent_fwd_bwd at N = B*T, vocab_size).  The
 * workspace holds temporaries only; its contents are undefined between
 * calls.  0 on invalid input. */
size_t gpt_workspace_bytes(const gpt_config* cfg, int B, int T);

/* One pre-norm transformer block forward ([nanoGPT] Block:
 *   x1 = x + attn(norm1(x)),  y = x1 + mlp(norm2(x1)),
 * attn = causal softmax(q k^T / sqrt(D)) v per head after the fused QKV
 * Linear, with RoPE then QK-norm on q and k when enabled ([d20]);
 * mlp = Linear(4C) -> exact-erf GELU -> Linear(C)).
 *   x     [B*T, C] input (dtype); the caller keeps it alive until the
 *         matching gpt_block_bwd.
 *   y     [B*T, C] output (dtype).
 *   saved gpt_block_saved_bytes() bytes, filled for the backward (with the
 *         RoPE table and, in bf16 without fp8, transposed copies of W_fc,
 *         W_o and W_qkv that it reads too); NULL runs inference only
 *         (intermediates then live in the workspace).
 *   ws    gpt_workspace_bytes() bytes of temporaries: the FP8 codes with
 *         cfg->fp8, the intermediates when saved is NULL.  Where neither
 *         applies the forward does not touch it and NULL is accepted.
 * Errors: INVALID (null pointer, B/T <= 0, T > block_size, n_embd % n_head,
 * odd head_dim with rope), UNSUPPORTED (head_dim not a multiple of 8 or
 * above 128, n_embd above 2048, or B*T*4*n_embd elements of 2 GiB or more:
 * the largest operand, refused before any launch), WORKSPACE, HIP.  In bf16,
 * head_dim 64 and 128 run the matrix-core attention kernels; other head
 * dims run a slower vector-ALU attention path (same function, its own
 * rounding). */
int gpt_block_fwd(const gpt_config* cfg, int B, int T, const void* x,
                  const gpt_block_weights* w, void* y, void* saved,
                  void* ws, size_t ws_bytes, void* stream);

/* Backward of gpt_block_fwd.  dy [B*T, C] upstream gradient (dtype);
 * dx [B*T, C] output gradient (dtype); parameter gradients into g (fp32,
 * overwritten or accumulated per `accumulate`).  `saved`, `x` and the
 * weights `w` must be those of the matching forward (the input gradients
 * read the forward's transposed weights from `saved`).  Same errors as gpt_block_fwd. */
int gpt_block_bwd(const gpt_config* cfg, int B, int T, const void* x,
                  const void* dy, const gpt_block_weights* w,
                  const void* saved, void* dx, const gpt_block_grads* g,
                  int accumulate, void* ws, size_t ws_bytes, void* stream);

/* LM head with softmax cross-entropy ([nanoGPT] model.py: final norm output
 * h times the (tied) head weight gives vocabulary logits; train.py: the loss
 * is the mean over tokens of -log softmax at the target).
 *   h        [N, C] final-norm output (dtype)
 *   W        [V, C] head weight (dtype; wte when tied), V = cfg->vocab_size
 *   targets  int32 [N], each in [0, V)
 *   loss_scale  multiplies the summed nats (1/N gives the mean)
 *   loss     device fp32 scalar, overwritten with loss_scale * sum(nats)
 *   nats     device fp32 [N] per-token nats (logsumexp - target logit), or NULL
 *   dh       [N, C] gradient wrt h (dtype), or NULL for forward only
 *   dW       [V, C] fp32 gradient wrt W (accumulate 0/1), or NULL
 * The logits are produced one vocabulary chunk at a time and the full
 * [N, V] matrix never exists in memory.  Errors: INVALID, UNSUPPORTED
 * (N * max(min(V, 8192), C) elements of 2 GiB or more), WORKSPACE, HIP. */
int lm_head_xent_fwd_bwd(const gpt_config* cfg, int N, const void* h,
                         const void* W, const int32_t* targets,
                         float loss_scale, float* loss, float* nats,
                         void* dh, float* dW, int accumulate,
                         void* ws, size_t ws_bytes, void* stream);

/* lm_head_xent_fwd_bwd with a weight per token ("Train your own ChatGPT",
 * section 6.3: the chat fine-tuning loss multiplies the per-token losses by
 * a 0/1 mask of the tokens to learn, sums, and divides by the mask's sum).
 * token_weight: device fp32 [N].  loss = loss_scale * sum_n w_n nats_n and
 * row n of the logit gradient carries loss_scale * w_n; a token with w_n = 0
 * is left out of the sum entirely (its nats are still written, NaN when its
 * target is out of range).  The masked mean is w = mask, loss_scale =
 * 1 / sum(mask).  Other arguments, layouts and errors as
 * lm_head_xent_fwd_bwd, which equals this call with every w_n = 1. */
int lm_head_xent_weighted_fwd_bwd(const gpt_config* cfg, int N, const void* h,
                                  const void* W, const int32_t* targets,
                                  const float* token_weight, float loss_scale,
                                  float* loss, float* nats, void* dh, float* dW,
                                  int accumulate, void* ws, size_t ws_bytes,
                                  void* stream);

/* Bits-per-byte reduction ([nanochat] 6.2, loss_eval.py paragraph): with
 * b_n = token_bytes[targets[n]], adds sum over b_n > 0 of nats[n] into
 * *sum_nats (fp64) and sum of b_n into *sum_bytes (int64).  Tokens with
 * zero byte length are excluded from both sums.  Both accumulators are
 * device scalars the caller zeroes once; many batches may be added before
 * the host forms bpb = sum_nats / (ln 2 * sum_bytes).  The reduction order
 * is fixed, so results are bitwise reproducible.  Errors: INVALID, HIP. */
int val_bpb_reduce(int N, const float* nats, const int32_t* targets,
                   const int32_t* token_bytes, int V, double* sum_nats,
                   int64_t* sum_bytes, void* stream);

/* ---- optimizer step ---- */

/* One tensor of a parameter set.  All device pointers, 16-byte aligned; the
 * tensors of one call must not overlap. */
typedef struct {
  float* param;        /* fp32 [n], updated in place                          */
  const float* grad;   /* fp32 [n], as the backward entry points write them  */
  float* m;            /* fp32 [n] first moment, in place (zeros at step 1)   */
  float* v;            /* fp32 [n] second moment, in place (zeros at step 1)  */
  void* param_bf16;    /* bf16 [n] copy of the updated param, or NULL         */
  int64_t n;           /* elements, > 0                                        */
  int32_t decay;       /* 1: weight decay applies (2-D tensors), 0: none      */
} gpt_adamw_tensor;

typedef struct {
  float lr, beta1, beta2, eps, weight_decay;
  int32_t step;        /* 1 for the first update                              */
  float max_norm;      /* clip of the global gradient norm; <= 0: no clip     */
} gpt_adamw_config;

/* AdamW step over `count` tensors ([nanoGPT] model.py section,
 * configure_optimizers: weight decay on every 2-D tensor, none on 1-D ones;
 * train.py section: the gradients are clipped to a global norm, 1.0 there,
 * before the step).  With ||g|| the L2 norm over all `grad` arrays and
 * s = max_norm / ||g|| when max_norm > 0 and ||g|| > max_norm (else 1), each
 * element takes, in fp32 (t = step; Loshchilov & Hutter, "Decoupled Weight
 * Decay Regularization", Algorithm 2, in PyTorch's AdamW order):
 *   g' = s g;  m = b1 m + (1 - b1) g';  v = b2 v + (1 - b2) g'^2;
 *   p = p (1 - lr wd)   [decay tensors only];
 *   p = p - lr / (1 - b1^t) * m / (sqrt(v) / sqrt(1 - b2^t) + eps);
 * and param_bf16 (when given) receives p rounded to bf16.  `tensors` is a
 * HOST array read during the call.  grad_norm: optional device fp32 scalar
 * that receives ||g|| (before clipping).  The norm is summed in fp64 in a
 * fixed order, so results are bitwise reproducible.  ws: device workspace of
 * gpt_adamw_workspace_bytes(tensors, count) bytes.  The hyperparameters are
 * inputs; the pages fix only the decay grouping and the clip.
 * Errors: INVALID, WORKSPACE, HIP. */
int gpt_adamw_step(const gpt_adamw_config* cfg, const gpt_adamw_tensor* tensors,
                   int count, float* grad_norm, void* ws, size_t ws_bytes,
                   void* stream);
size_t gpt_adamw_workspace_bytes(const gpt_adamw_tensor* tensors, int count);

/* gpt_adamw_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight training loops, harnesses that forbid
 * hipMalloc): the same update and results, with no workspace argument.  Its
 * scratch is a device array inside the library of GPT_ADAMW_NOALLOC_MAX_CHUNKS
 * fp64 partials plus 256 bytes (1 MiB), one copy per GPU, held until the
 * process ends; the call makes no hipMalloc, hipFree or other allocation.
 * Capacity: the sum over tensors of ceil(n / 8192) must not exceed
 * GPT_ADAMW_NOALLOC_MAX_CHUNKS (up to 2^30 parameters); larger sets return
 * UNSUPPORTED.  Every call on one GPU shares that GPU's scratch: calls that
 * overlap in time on one GPU (concurrent streams, threads) race and must be
 * serialized by the caller.  Errors: INVALID, UNSUPPORTED, HIP. */
#define GPT_ADAMW_NOALLOC_MAX_CHUNKS 131072
int gpt_adamw_step_noalloc(const gpt_adamw_config* cfg,
                           const gpt_adamw_tensor* tensors, int count,
                           float* grad_norm, void* stream);

/* ---- FP8 GEMMs ---- */

#define GPT_FP8_E4M3 0   /* OCP E4M3: bias 7, largest finite 448, no infinities */
#define GPT_FP8_E5M2 1   /* OCP E5M2: bias 15, largest finite 57344           */

/* Dynamic per-tensor FP8 quantization ([nanochat] 6.2, FP8 paragraph; [d20]
 * Pretraining row: the published run trained its matmuls in FP8).  x: bf16
 * [n].  scale: device fp32 [3] receiving s = fmt_max / amax (1 when amax is
 * 0), amax = max |x| and 1 / s.  q: [n] bytes receiving the code of
 * clamp(x * s, -fmt_max, fmt_max) (product in fp32) rounded to nearest even.
 * ws: gpt_fp8_workspace_bytes(n) bytes.  Deterministic.  Errors: INVALID,
 * WORKSPACE, HIP. */
int gpt_fp8_quantize(int64_t n, const void* x, int fmt, void* q, float* scale,
                     void* ws, size_t ws_bytes, void* stream);
size_t gpt_fp8_workspace_bytes(int64_t n);

/* out[m][n] = sum_k qa[m][k] qb[n][k] * inv_a * inv_b (inv = element 2 of
 * the quantizer's scale array), bf16 [M][ldc] output, fp32 accumulation on
 * the 8-bit MFMA.  qa [M][lda], qb [N][ldb] are codes of formats fmt_a,
 * fmt_b with k contiguous (a Linear forward: activations times the weight
 * [out, in]; an input gradient with a transposed weight).  K, lda and ldb
 * multiples of 16; N and ldc multiples of 8; pointers 16-byte aligned; each
 * operand under 2 GiB.  Errors: INVALID, HIP. */
int gpt_fp8_gemm(int M, int N, int K, const void* qa, int64_t lda, int fmt_a,
                 const float* scale_a, const void* qb, int64_t ldb, int fmt_b,
                 const float* scale_b, void* out, int64_t ldc, void* stream);

/* ---- helpers used to assemble a full model step (same conventions) ---- */

/* Token embedding ([nanoGPT] model.py section: the token embedding wte,
 * plus the learned absolute position embedding wpe in the nanoGPT form; the
 * nanochat form uses RoPE in the attention instead, [d20] Architecture row):
 * x0[n] = wte[ids[n]] (+ wpe[t] with learned positions, cfg->rope == 0).
 * ids int32 [B*T] (an id outside [0, V) gives a zero token row); wte [V, C];
 * wpe [block_size, C] or NULL when rope; x0 [B*T, C] (dtype).  Errors:
 * INVALID, UNSUPPORTED (as gpt_block_fwd), HIP. */
int gpt_embed_fwd(const gpt_config* cfg, int B, int T, const int32_t* ids,
                  const void* wte, const void* wpe, void* x0, void* stream);

/* Backward of gpt_embed_fwd ([nanoGPT] model.py section; with weight tying
 * the head's gradient is added into the same dwte, accumulate = 1):
 * dwte[v] (+)= sum of dx0 rows with id v (fixed summation order: by
 * position), dwpe[t] (+)= sum over the batch of dx0[b, t]; fp32 outputs.
 * dwpe may be NULL.  Rows of dwte that no id touches are zeroed when
 * accumulate = 0 and left alone otherwise.  ws: gpt_workspace_bytes bytes.
 * Errors: INVALID, UNSUPPORTED, WORKSPACE, HIP. */
int gpt_embed_bwd(const gpt_config* cfg, int B, int T, const int32_t* ids,
                  const void* dx0, float* dwte, float* dwpe, int accumulate,
                  void* ws, size_t ws_bytes, void* stream);

/* Row norm of the configuration ([nanoGPT] model.py section: LayerNorm
 * with a gain and an optional bias, the final norm before the head; [d20]
 * Architecture row: the parameter-free RMSNorm of the nanochat form):
 * y = norm(x) over the C entries of each of the N rows (dtype).  stats fp32
 * [2N] receives mean (0 for RMSNorm) and 1/sqrt(var + eps) per row, or
 * NULL.  Errors: INVALID, HIP. */
int gpt_norm_fwd(const gpt_config* cfg, int N, const void* x, const void* w,
                 const void* b, void* y, float* stats, void* stream);

/* Backward of gpt_norm_fwd (same passages): dx = dnorm(dy) (+ resid when
 * resid != NULL, the residual branch's gradient), dw, db fp32 [C]
 * (accumulate 0/1; NULL for RMSNorm or no bias).  ws: gpt_workspace_bytes
 * bytes (LayerNorm only).  Errors: INVALID, WORKSPACE, HIP. */
int gpt_norm_bwd(const gpt_config* cfg, int N, const void* x, const void* w,
                 const void* dy, const void* resid, void* dx, float* dw,
                 float* db, int accumulate, void* ws, size_t ws_bytes,
                 void* stream);

/* Kernel timing for diagnostics and benchmarks.  After gpt_trace_begin(n),
 * each kernel call site of the entry points above is bracketed by a pair of
 * hipEvents recorded on the call's stream (up to n call sites; the event
 * pool is created here and kept for the process).  gpt_trace_end waits for
 * the recorded events, writes one text line per call-site name,
 * "<name> <launches> <total microseconds>\n", into buf (len bytes, NUL
 * terminated), clears the records and stops timing.  Process-wide state;
 * not for concurrent use from several threads.  Errors: INVALID (capacity
 * <= 0, buf too small), HIP. */
int gpt_trace_begin(int capacity);
int gpt_trace_end(char* buf, size_t len);

/* Text of a status code; the last error message of this thread. */
const char* gpt_status_string(int status);
const char* gpt_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* GPTMI_H */
