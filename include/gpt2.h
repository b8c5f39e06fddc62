/*
 * gpt2.h -- C ABI of the MI355X (gfx950) GPT-2 decoder forward pass.
 *
 * The library maps token ids [B, T] to logits [B, T, n_vocab]: wte + wpe embedding gather-add,
 * n_layer Pre-LN blocks (LayerNorm, fused QKV projection, causal multi-head self-attention with
 * the mask applied before the softmax, output projection plus residual, LayerNorm, 4x GELU MLP
 * plus residual), the final LayerNorm ln_f and the lm_head tied to wte.
 *
 * Pages the operations are defined on (titles as printed on the pages):
 *   [手写] "从零手写GPT-2：PyTorch实现Transformer解码器核心模块"
 *   [实战] "GPT2模型开发实战：从原理到部署全解析"
 *   [解析] "GPT-2模型架构解析与实现指南"
 *   [复现] "复现GPT-2 124M"
 *   [指南] "从零实现 GPT-2：PyTorch 版大语言模型构建指南"
 *
 * Conventions shared by every entry point
 *   - Every pointer named *_dev is a device pointer on the current HIP device. The caller owns
 *     every buffer (tokens, logits, packed weights, workspace); the library never calls
 *     hipMalloc or hipFree. Its only device memory of its own is the fixed scratch array of
 *     gpt2_forward_noalloc (80 MiB per device, present from module load).
 *   - Every call that takes a hipStream_t only enqueues work on that stream (NULL = the null
 *     stream) and returns without synchronising, except gpt2_check, which synchronises it.
 *   - Arguments are validated on the host before anything is launched; on any error nothing is
 *     enqueued and the output buffers are left untouched.
 *   - Linear weights use the [out, in] layout of nn.Linear: y = x W^T + b.
 *   - A gpt2_model handle is host memory only. It is immutable once weights are loaded; several
 *     forwards may run concurrently on one handle provided each uses its own workspace.
 */
#ifndef GPT2_H
#define GPT2_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GPT2_OK = 0,
    GPT2_EINVAL = 1,      /* null pointer, bad enum value, inconsistent sizes */
    GPT2_ESHAPE = 2,      /* B < 1, T < 1, T > n_ctx, or a dimension the kernels do not support */
    GPT2_EWORKSPACE = 3,  /* workspace or destination buffer smaller than required */
    GPT2_ETOKEN = 4,      /* a token id outside [0, n_vocab) was seen by the last forward */
    GPT2_EHIP = 5,        /* a HIP runtime call or kernel launch failed */
    GPT2_ESTATE = 6       /* call made in the wrong state (e.g. forward before weights) */
} gpt2_status;

/* Compute mode. GPT2_F32: every operand and intermediate in fp32. GPT2_BF16: GEMM and attention
 * operands in bf16 with fp32 accumulation; the residual stream, LayerNorm and softmax statistics
 * and the logits stay fp32. */
typedef enum { GPT2_F32 = 0, GPT2_BF16 = 1 } gpt2_dtype;

/* GELU form used in the MLP: the tanh form is the one original GPT-2 uses ([复现] §2.4);
 * the erf form is the F.gelu default of [解析] §2.2. */
typedef enum { GPT2_GELU_TANH = 0, GPT2_GELU_ERF = 1 } gpt2_gelu;

/* Model hyper-parameters: the GPT2Config fields of [手写] §4.1 and the GPT_CONFIG_124M table of
 * [指南] (configuration section). Requirements: all sizes > 0, d_model % n_head == 0,
 * d_model / n_head == 64, d_model % 64 == 0, d_model <= 4096, d_mlp % 64 == 0,
 * n_ctx <= 65536. */
typedef struct {
    int32_t n_vocab;   /* 50257 */
    int32_t n_ctx;     /* 1024: the largest T accepted (longer inputs are an error, [手写] §3.3) */
    int32_t d_model;   /* 768 / 1024 / 1600 */
    int32_t n_head;    /* 12 / 16 / 25 */
    int32_t n_layer;   /* 12 / 24 / 48 */
    int32_t d_mlp;     /* 4 * d_model */
    float ln_eps;      /* 1e-5 ([手写] §3.2) */
    int32_t dtype;     /* gpt2_dtype */
    int32_t gelu;      /* gpt2_gelu */
} gpt2_config_t;

typedef struct gpt2_model gpt2_model;

/* Validate *cfg and create a host-side handle in *out. No HIP call is made. */
gpt2_status gpt2_config(const gpt2_config_t* cfg, gpt2_model** out);

/* Release a handle (NULL is ignored). Device buffers stay the caller's. */
void gpt2_destroy(gpt2_model* m);

/* Number of source tensors gpt2_load_weights expects: 2 + 12 * n_layer + 2. */
int32_t gpt2_n_tensors(const gpt2_model* m);

/* Shape of source tensor i in the fixed order below: rows/cols (cols = 0 for a vector).
 * Order: wte[n_vocab,d], wpe[n_ctx,d], then for each layer ln_1.w[d], ln_1.b[d],
 * attn.c_attn.w[3d,d], attn.c_attn.b[3d], attn.c_proj.w[d,d], attn.c_proj.b[d], ln_2.w[d],
 * ln_2.b[d], mlp.c_fc.w[d_mlp,d], mlp.c_fc.b[d_mlp], mlp.c_proj.w[d,d_mlp], mlp.c_proj.b[d],
 * then ln_f.w[d], ln_f.b[d]. There is no lm_head tensor: it is wte ([手写] §2.2 item 4). */
gpt2_status gpt2_tensor_shape(const gpt2_model* m, int32_t i, int64_t* rows, int64_t* cols);

/* Bytes of the packed device weight buffer gpt2_load_weights fills. Matrices are stored in the
 * compute dtype with their row count padded to a multiple of 256 (padding rows are zero);
 * vectors are fp32; every tensor starts on a 256-byte boundary. A bf16 model also holds, after the
 * source tensors, a k-blocked copy of wte and of the four projection matrices of every layer
 * ([cols/32][rows padded][32]: 32-column blocks of all rows one after another), which the tiled
 * projections of the forward read so that every slab of a K step is contiguous, and a transposed
 * copy of the same five matrices ([cols padded to 256][rows]; wte^T [d padded][n_vocab rounded up
 * to 64], zero padding) that gpt2_backward reads for the input gradients. */
size_t gpt2_weight_bytes(const gpt2_model* m);

/* Bytes of device workspace one forward of shape [B, T] needs (0 for invalid B, T). */
size_t gpt2_workspace_bytes(const gpt2_model* m, int32_t B, int32_t T);

/* Pack the caller's source tensors (n_src device pointers in the order of gpt2_tensor_shape,
 * each contiguous, element type src_dtype: GPT2_F32 = float, GPT2_BF16 = bf16) into dst_dev,
 * converting to the compute dtype (fp32 -> bf16 rounds to nearest even). dst_dev must hold
 * gpt2_weight_bytes(m) bytes and be 256-byte aligned; the handle keeps the pointer (borrowed)
 * and every later forward reads the weights from it. Asynchronous on stream: the sources must
 * stay valid until the stream reaches this point. */
gpt2_status gpt2_load_weights(gpt2_model* m, const void* const* src, int32_t n_src, int32_t src_dtype,
                              void* dst_dev, size_t dst_bytes, hipStream_t stream);

/* The forward pass ([手写] §4.1 forward; [复现] §2.1-§2.4).
 *   tokens_dev  int32 [B, T] row-major, ids in [0, n_vocab) (an id outside is clamped for the
 *               read and reported by gpt2_check as GPT2_ETOKEN).
 *   logits_dev  fp32 [B, T, n_vocab] contiguous (row stride n_vocab), written in full.
 *   argmax_dev  int32 [B, T] or NULL: index of the largest logit of each row, the first one on
 *               ties, computed from the fp32 logits this call writes.
 *   ws_dev      workspace of at least gpt2_workspace_bytes(m, B, T) bytes, 256-byte aligned,
 *               used by this call alone until the stream passes it.
 * Requires 1 <= B, 1 <= T <= n_ctx and loaded weights. */
gpt2_status gpt2_forward(const gpt2_model* m, const int32_t* tokens_dev, int32_t B, int32_t T,
                         float* logits_dev, int32_t* argmax_dev, void* ws_dev, size_t ws_bytes,
                         hipStream_t stream);

/* gpt2_forward for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same launches and results as gpt2_forward,
 * with the workspace taken from a fixed array inside the library instead of a caller's buffer.
 *   - The array holds 80 MiB per GPU the library runs on (GPT-2 small up to B*T = 4096 rows) and
 *     lives until the process ends; its address on each device is looked up once, on the first call
 *     for that device. The call itself allocates nothing and calls no allocating routine.
 *   - GPT2_EWORKSPACE when gpt2_workspace_bytes(m, B, T) exceeds 80 MiB; the other argument rules
 *     and errors are gpt2_forward's (logits_dev required, argmax_dev optional).
 *   - Every call on one GPU shares that GPU's array: calls that overlap on one GPU (other streams,
 *     other threads) race and must be serialised by the caller. Nothing in it needs clearing.
 *   - Out-of-range token ids are clamped as in gpt2_forward but cannot be reported: gpt2_check
 *     needs the caller's workspace. */
gpt2_status gpt2_forward_noalloc(const gpt2_model* m, const int32_t* tokens_dev, int32_t B, int32_t T,
                                 float* logits_dev, int32_t* argmax_dev, hipStream_t stream);

/* The forward pass followed by the shifted next-token cross-entropy of [手写] §4.1, without
 * writing the logits: the vocabulary projection reduces each row to its log-sum-exp and the
 * logit of its target inside the GEMM epilogue, so the [B, T, n_vocab] fp32 logits are never
 * stored.
 *   labels_dev  int32 [B, T] or NULL (NULL: the tokens themselves, the language-model case).
 *               Position t of row b is scored against labels[b, t+1]; the last position of each
 *               row has no target. A label of -100 (the loss's default ignore index) leaves its
 *               position out; any other label outside [0, n_vocab) is left out too and reported
 *               by gpt2_check as GPT2_ETOKEN.
 *   nll_dev     fp32 [B, T]: nll[b, t] = logsumexp(logits[b, t, :]) - logits[b, t, labels[b, t+1]],
 *               0 where the position has no counted target (t = T-1 or ignored).
 *   loss_dev    fp32 [1]: the mean of nll over the counted positions (NaN when none counts),
 *               summed in a fixed order (run to run identical).
 *   ws_dev      as for gpt2_forward (the same gpt2_workspace_bytes).
 * Requires 2 <= T <= n_ctx (GPT2_ESHAPE otherwise), 1 <= B and loaded weights. */
gpt2_status gpt2_forward_loss(const gpt2_model* m, const int32_t* tokens_dev, const int32_t* labels_dev,
                              int32_t B, int32_t T, float* nll_dev, float* loss_dev, void* ws_dev,
                              size_t ws_bytes, hipStream_t stream);

/* Cached incremental decoding ([手写] §6.3 greedy generation; [解析] §4.2 KV cache): the keys and values of
 * every layer are kept in a caller-owned cache so that each new token costs one position of the
 * forward. Layout: for each layer l, K then V, each [B][n_head][n_ctx][64] in the compute dtype
 * (bf16 or fp32). Positions are shared by the batch: every sequence has the same length.
 * Bytes of the cache for B sequences (0 for invalid B). */
size_t gpt2_kv_cache_bytes(const gpt2_model* m, int32_t B);

/* Run the forward over the prompt tokens_dev int32 [B, T] (1 <= T <= n_ctx), writing the keys and
 * values of positions 0 .. T-1 of every layer into cache_dev (cache_bytes >= gpt2_kv_cache_bytes,
 * 256-byte aligned); positions >= T are untouched. Then, for the last position of each sequence:
 *   logits_dev fp32 [B, n_vocab] or NULL: its logits (the same values gpt2_forward gives for row T-1);
 *   next_dev   int32 [B] or NULL: their argmax, the first index on ties (the greedy next token).
 * Workspace: gpt2_workspace_bytes(m, B, T). Asynchronous on stream. */
gpt2_status gpt2_prefill(const gpt2_model* m, const int32_t* tokens_dev, int32_t B, int32_t T, void* cache_dev,
                         size_t cache_bytes, float* logits_dev, int32_t* next_dev, void* ws_dev, size_t ws_bytes,
                         hipStream_t stream);

/* One decoding step: tokens_dev int32 [B] is the token at position pos (0 <= pos < n_ctx) of each
 * sequence, whose positions 0 .. pos-1 are already in cache_dev (from gpt2_prefill and earlier
 * steps with this cache). Appends the keys and values of position pos, attends over positions
 * 0 .. pos, and writes the next-token logits_dev fp32 [B, n_vocab] and/or next_dev int32 [B] as
 * gpt2_prefill does (by causality these are row pos of gpt2_forward over the whole sequence).
 * Workspace: gpt2_workspace_bytes(m, B, 1). GPT2_ESHAPE for pos outside [0, n_ctx). */
gpt2_status gpt2_decode_step(const gpt2_model* m, const int32_t* tokens_dev, int32_t B, int32_t pos,
                             void* cache_dev, size_t cache_bytes, float* logits_dev, int32_t* next_dev,
                             void* ws_dev, size_t ws_bytes, hipStream_t stream);

/* Residual stream after the embedding and the first n_layers blocks (0 = embedding only,
 * n_layer = all blocks, before ln_f), as fp32 [B, T, d] into resid_dev. Same workspace and
 * argument rules as gpt2_forward. Used for per-block alignment checks ([手写] §4.2). */
gpt2_status gpt2_forward_debug(const gpt2_model* m, const int32_t* tokens_dev, int32_t B, int32_t T,
                               int32_t n_layers, float* resid_dev, void* ws_dev, size_t ws_bytes,
                               hipStream_t stream);

/* Kinds of the kernel launches a forward enqueues, in order (gpt2_forward_launches). */
typedef enum {
    GPT2_K_EMBED = 0, GPT2_K_LN = 1, GPT2_K_QKV = 2, GPT2_K_ATTN = 3, GPT2_K_ATTN_PROJ = 4, GPT2_K_FC = 5,
    GPT2_K_MLP_PROJ = 6, GPT2_K_LN_F = 7, GPT2_K_LM_HEAD = 8, GPT2_K_ARGMAX = 9, GPT2_K_XENT = 10,
    GPT2_K_KV = 11
} gpt2_kernel_kind;

/* Number of kernel launches one gpt2_forward over B x T tokens enqueues (with_argmax: argmax_dev !=
 * NULL); when kinds != NULL, also writes the gpt2_kernel_kind of the first min(cap, count)
 * launches. The sequence depends on the shape (in bf16 with more than 16 rows the embedding launch
 * also computes the first block's ln_1). 0 for a NULL handle or B < 1, T < 1, T > n_ctx. Host only. */
int32_t gpt2_forward_launches(const gpt2_model* m, int32_t B, int32_t T, int32_t with_argmax, int32_t* kinds,
                              int32_t cap);

/* gpt2_forward that also records caller-created HIP events (hipEventCreate) on stream around its
 * launches: for launch i < n_slots, ev_before[i] (if not NULL) is recorded right before it and
 * ev_after[i] (if not NULL) right after it. ev_before / ev_after may themselves be NULL. Used to
 * time individual kernels on the stream they run on; everything else is as gpt2_forward. */
gpt2_status gpt2_forward_timed(const gpt2_model* m, const int32_t* tokens_dev, int32_t B, int32_t T,
                               float* logits_dev, int32_t* argmax_dev, void* ws_dev, size_t ws_bytes,
                               hipStream_t stream, hipEvent_t* ev_before, hipEvent_t* ev_after,
                               int32_t n_slots);

/* gpt2_forward with launch number `launch` (0-based, in the order of gpt2_forward_launches)
 * enqueued `repeats` times back to back, with the caller's events ev_before / ev_after (either may
 * be NULL) recorded around that group: for timing one kernel of the forward in the forward's own
 * data layout, with no event between its launches. A repeated launch that accumulates into its
 * output (the residual projections) leaves results that are not the forward's; GPT2_EINVAL for a
 * launch number outside the forward or repeats < 1. Otherwise as gpt2_forward. */
gpt2_status gpt2_forward_repeat(const gpt2_model* m, const int32_t* tokens_dev, int32_t B, int32_t T,
                                float* logits_dev, int32_t* argmax_dev, void* ws_dev, size_t ws_bytes,
                                hipStream_t stream, int32_t launch, int32_t repeats, hipEvent_t ev_before,
                                hipEvent_t ev_after);

/* Synchronise stream, then report GPT2_ETOKEN if the last forward that used ws_dev saw a token
 * id (or, for gpt2_forward_loss, a label other than -100) outside [0, n_vocab), else GPT2_OK.
 * B and T must be those of that forward. */
gpt2_status gpt2_check(const gpt2_model* m, const void* ws_dev, int32_t B, int32_t T, hipStream_t stream);

/* Causal multi-head attention on its own ([复现] §2.1-§2.2; [解析] §2.1):
 *   o[b,h,i,:] = sum_{j<=i} softmax_j(q[b,h,i,:] . k[b,h,j,:] / sqrt(dh)) v[b,h,j,:].
 * q, k, v, o are device tensors of element type dtype (GPT2_BF16: bf16, softmax in fp32;
 * GPT2_F32: fp32) addressed as base + b*s_b + h*s_h + t*s_t + c (strides in elements, the last
 * dimension contiguous; each of q/k/v/o has its own three strides given as {s_b, s_h, s_t}).
 * Requires dh == 64, B, H, T >= 1, every stride a multiple of 8 and every base 16-byte aligned. */
gpt2_status gpt2_attention(const void* q_dev, const int64_t* q_strides, const void* k_dev,
                           const int64_t* k_strides, const void* v_dev, const int64_t* v_strides,
                           void* o_dev, const int64_t* o_strides, int32_t B, int32_t H, int32_t T,
                           int32_t dh, int32_t dtype, hipStream_t stream);

/* LayerNorm of M rows of width n over fp32 x ([复现] §2.1 LayerNorm: biased variance):
 * y = (x - mean) / sqrt(var + eps) * gamma + beta, gamma/beta fp32 [n], y of element type
 * out_dtype (GPT2_BF16 rounds to nearest even), both row-major with row stride n.
 * Requires n % 4 == 0 and n <= 4096. */
gpt2_status gpt2_layernorm(const float* x_dev, const float* gamma_dev, const float* beta_dev, void* y_dev,
                           int32_t M, int32_t n, float eps, int32_t out_dtype, hipStream_t stream);

/* Epilogues of gpt2_linear (the fused forms the forward uses). */
typedef enum {
    GPT2_EPI_BIAS = 0,          /* C = A W^T + b                  (C in dtype)             */
    GPT2_EPI_BIAS_GELU = 1,     /* C = gelu(A W^T + b)            (C in dtype; gelu = cfg) */
    GPT2_EPI_BIAS_RESIDUAL = 2, /* C += A W^T + b                 (C fp32, read and written) */
    GPT2_EPI_LOGITS = 3         /* C = A W^T, no bias             (C fp32)                 */
} gpt2_epilogue;

/* C[M, N] = epi(A[M, K] W[N, K]^T + bias[N]) with A, W of element type dtype (row-major, K
 * contiguous) and bias fp32 (ignored for GPT2_EPI_LOGITS, may be NULL there). ldc is C's row
 * stride in elements. A must have round_up(M, 256) readable rows and W round_up(N, 256) readable
 * rows (rows past M / N may hold anything; their results are never stored). gelu selects the
 * GELU form for GPT2_EPI_BIAS_GELU. Requires K % 64 == 0. Used by the forward for c_attn,
 * attn.c_proj, mlp.c_fc, mlp.c_proj and lm_head ([复现] §2.1, §2.4; [手写] §4.1). */
gpt2_status gpt2_linear(const void* A_dev, const void* W_dev, const float* bias_dev, void* C_dev,
                        int32_t M, int32_t N, int32_t K, int64_t ldc, int32_t dtype, int32_t epilogue,
                        int32_t gelu, hipStream_t stream);

/* Sampled next-token choice for B rows of fp32 logits, the sampling branch of generation: the
 * repetition penalty, temperature, top-k and top-p knobs of [实战] §8.2, then a draw from
 * softmax(z / temperature) restricted to the kept tokens ([解析] §4.1), taken by inverse CDF. Per row:
 *   1. every distinct id of hist_dev[b, 0 .. n_hist) inside [0, V) has its logit divided by
 *      repetition_penalty when positive and multiplied by it otherwise (ids outside are ignored);
 *   2. z = x / temperature for the penalised logits x (dividing by a positive temperature keeps
 *      their order, so steps 3 and 4 compare x, in fp32, and the softmax weights are
 *      exp((x - max x) / temperature));
 *   3. top_k > 0 and < V: tokens whose z is below the k-th largest z are dropped (ties kept);
 *   4. top_p < 1: with q the softmax of z over the tokens still kept, a token is dropped when the
 *      q-mass of the kept tokens with a strictly larger z is p or more (the largest z always stays);
 *   5. out_dev[b] = the first token in vocabulary order whose cumulative q over the kept tokens
 *      exceeds u_dev[b] (u clamped into [0, 1)); n_kept_dev[b] (if not NULL) = how many were kept.
 * Each weight is rounded to 2^-31 of the largest one and the weights are summed exactly in integer
 * arithmetic, so the result does not depend on summation order (a token whose weight is below
 * 2^-31 of the largest is never drawn).
 *   logits_dev  fp32 [B, V], row stride ld >= V (elements); V <= 65536.
 *   hist_dev    int32 [B, n_hist], row stride hist_ld >= n_hist; may be NULL when n_hist == 0.
 *   u_dev       fp32 [B]: the caller's uniform random numbers (one per row).
 *   ws_dev      NULL, or a 256-byte aligned device workspace of ws_bytes >=
 *               gpt2_sample_workspace_bytes(B, V) bytes used by this call alone until the stream
 *               passes it: with it, top-k rows are screened by many workgroups per row before one
 *               wave finishes them; without it each row runs on one workgroup. The result is the
 *               same either way.
 * GPT2_EINVAL for temperature or repetition_penalty not finite and > 0, top_k < 0, top_p outside
 * (0, 1], a missing pointer or a misaligned workspace; GPT2_EWORKSPACE for a workspace below the
 * required size; GPT2_ESHAPE for B < 1, V < 1, V > 65536 or ld < V. A row whose largest logit is
 * not finite yields an unspecified token in [0, V). Needs no model handle. */
gpt2_status gpt2_sample(const float* logits_dev, int64_t ld, int32_t B, int32_t V, const int32_t* hist_dev,
                        int64_t hist_ld, int32_t n_hist, float temperature, int32_t top_k, float top_p,
                        float repetition_penalty, const float* u_dev, int32_t* out_dev, int32_t* n_kept_dev,
                        void* ws_dev, size_t ws_bytes, hipStream_t stream);

/* Bytes of the optional gpt2_sample workspace for B rows of V logits (0 for invalid B, V). */
size_t gpt2_sample_workspace_bytes(int32_t B, int32_t V);

/* Training gradients ([手写] §4 training loop: the loss and loss.backward(); §2.2: with the lm_head
 * tied to wte, the gradient of wte is the lm_head's gradient plus the embedding's).
 * gpt2_backward runs the forward keeping its activations, the mean shifted next-token
 * cross-entropy of gpt2_forward_loss (same labels rules, -100 ignored), and the backward pass,
 * writing loss_dev fp32 [1] and the fp32 gradient of every source tensor of gpt2_tensor_shape:
 * tensor i's gradient starts at byte gpt2_grad_offset(m, i) of grads_dev, in its source shape (rows
 * unpadded, row-major), and every element of every gradient is written (rows of wpe past T get 0).
 *   grads_dev   256-byte aligned, at least gpt2_grad_bytes(m) bytes.
 *   ws_dev      256-byte aligned, at least gpt2_train_workspace_bytes(m, B, T) bytes (the saved
 *               activations of every layer and the backward's buffers; gpt2_check(m, ws_dev, B, T)
 *               reports out-of-range token ids or labels afterwards).
 * Products run in the compute dtype (bf16 operands with fp32 accumulation, or fp32); gradients,
 * the residual stream and every reduction are fp32. The embedding part of the wte gradient is
 * added with floating-point atomics, so rows of tokens that repeat may differ in the last bits from
 * run to run; every other gradient is computed in a fixed order.
 * Requires 2 <= T <= n_ctx, 1 <= B, B * T <= 2^20 and loaded weights. */
size_t gpt2_grad_bytes(const gpt2_model* m);
size_t gpt2_grad_offset(const gpt2_model* m, int32_t i); /* (size_t)-1 for an invalid i */
size_t gpt2_train_workspace_bytes(const gpt2_model* m, int32_t B, int32_t T); /* 0 for invalid B, T */
gpt2_status gpt2_backward(const gpt2_model* m, const int32_t* tokens_dev, const int32_t* labels_dev, int32_t B,
                          int32_t T, float* grads_dev, size_t grads_bytes, float* loss_dev, void* ws_dev,
                          size_t ws_bytes, hipStream_t stream);

/* Static text for a status code. */
const char* gpt2_strerror(gpt2_status s);

#ifdef __cplusplus
}
#endif

#endif /* GPT2_H */
