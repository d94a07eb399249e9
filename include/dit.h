/*
 * dit.h -- C ABI of libdit.so: the forward pass of a pre-norm AdaLN
 * diffusion-transformer block, the block stack of one flow-match denoising
 * step, and the Euler update, as hand-written HIP kernels for gfx950 (MI355X).
 *
 * Sources for what each call computes (the pages the method comes from):
 *   [ERNIE]   "Porting ERNIE-Image-Turbo to Zig and Metal: An 8B Diffusion
 *             Transformer From Scratch on Apple Silicon"
 *   [ZML]     "From Python + CUDA to Pure Rust + Metal 4: How zml-flow-rs
 *             Stops Us Writing a Kernel Per Model"
 *   [MAKEPAD] makepad commit log (libs/ai/metal/shaders/ggml): the resident
 *             pre-norm ViT backbone.
 *
 * Conventions shared by every entry point
 *   - Pointers named as device memory are device memory owned by the caller;
 *     the library never frees, keeps or reallocates them, and allocates no
 *     device memory of its own: scratch space comes in through `ws`.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *     enqueued asynchronously; no call synchronises the host.  A fault inside
 *     a kernel is reported by the caller's next hipStreamSynchronize.
 *   - Every call validates its arguments before launching anything and
 *     returns a dit_status; it never aborts.  dit_last_error() then gives a
 *     thread-local message.  Without a usable GPU the compute calls return
 *     DIT_ERR_NO_DEVICE (after argument validation).
 *   - Device pointers must be 16-byte aligned (DIT_ERR_ALIGNMENT otherwise).
 *   - GEMM weights are [out_features, in_features] row-major (y = x W^T),
 *     bf16 (or int8 codes in the W8A8 H256 format).  Accumulation is fp32
 *     everywhere (exact int32 for int8 products).
 *   - Repeated calls with the same inputs are bitwise identical (no atomics).
 *   - Calls on different streams are thread-safe when their workspaces and
 *     outputs are distinct.
 */
#ifndef DIT_H
#define DIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DIT_OK = 0,
    DIT_ERR_INVALID_ARG = -1,   /* null pointer, bad dimension, illegal aliasing   */
    DIT_ERR_UNSUPPORTED = -2,   /* valid request the kernels are not built for      */
    DIT_ERR_WORKSPACE = -3,     /* ws_bytes smaller than the *_workspace_size value */
    DIT_ERR_ALIGNMENT = -4,     /* a device pointer is not 16-byte aligned          */
    DIT_ERR_NO_DEVICE = -5,     /* no HIP device visible                            */
    DIT_ERR_HIP = -6            /* a HIP runtime call or kernel launch failed       */
} dit_status;

typedef enum { DIT_F32 = 0, DIT_BF16 = 1 } dit_dtype;
typedef enum { DIT_LAYERNORM = 0, DIT_RMSNORM = 1 } dit_norm;
/* RoPE pair layout: (2m, 2m+1) interleaved, or rotate-half (m, m + hd/2). */
typedef enum { DIT_ROPE_INTERLEAVED = 0, DIT_ROPE_HALF = 1 } dit_rope;
/* Feed-forward GLU activation on the gate half: SiLU (SwiGLU), or GELU in its
 * tanh approximation with the argument clamped to +-20 and the result to
 * +-65504 ([ERNIE] §IV "GELU(gate) x up, tanh approx, clamped", §V Bug 1). */
typedef enum { DIT_ACT_SILU = 0, DIT_ACT_GELU_TANH = 1 } dit_act;
/* Function applied to gate1 / gate2 before the gated residual r + f(g) y:
 * identity ([ERNIE] §VII Decision 1), tanh or sigmoid ([ZML] §IV: the
 * semantics search chooses between them per model). */
typedef enum { DIT_GATE_IDENTITY = 0, DIT_GATE_TANH = 1, DIT_GATE_SIGMOID = 2 } dit_gate;
/* AdaLN chunks: six (shift1, scale1, gate1, shift2, scale2, gate2) ([ERNIE]
 * §IV), or four (scale1, gate1, scale2, gate2) with no shift ([ZML] §IV table:
 * "[scale, gate], 1 + scale, no shift"). */
typedef enum { DIT_MOD_SHIFT_SCALE_GATE = 0, DIT_MOD_SCALE_GATE = 1 } dit_mod;
/* qk-norm before RoPE ([ZML] §VI "QKV + norm + RoPE"), or RoPE before the
 * qk-norm ([ERNIE] §IV per-layer graph draws 3D RoPE, then qk_layernorm). */
typedef enum { DIT_QK_NORM_ROPE = 0, DIT_QK_ROPE_NORM = 1 } dit_qk_order;
/* Numeric format of the block's four projections (QKV, out, gate/up, down):
 * bf16 operands, or W8A8 H256 ([ZML] §VII "Precision Formats": the I8 per-row
 * format with a 256-point Hadamard rotation on both sides, legal because
 * (x H)(W H)^T = x W^T for orthogonal H).  In W8A8 H256 each operand row is
 * multiplied by blockdiag(H256) along the reduction axis (H256 = the
 * Sylvester-Hadamard matrix / 16 on every run of 256 elements) and stored as
 * int8 codes round-half-even(v * 127 / max|v|) with the fp32 row scale
 * max|v| / 127 (per token for activations, per output channel for weights);
 * the int32 products are exact and are scaled back before the same fused
 * epilogues.  Norms, attention and the residual stream are unchanged. */
typedef enum { DIT_FMT_BF16 = 0, DIT_FMT_W8A8_H256 = 1 } dit_fmt;

/* Shape and semantic switches of one block.
 *   tokens N = batch * seq; attention runs within each sequence.
 *   heads * head_dim must equal hidden; heads % kv_heads == 0 (grouped KV:
 *   query head h reads KV head h / (heads / kv_heads)).
 *   cond_dim > 0: AdaLN mode ([ERNIE] §IV): modulation from the conditioning
 *     vector, LayerNorm without affine, gated residuals.
 *   cond_dim == 0: plain pre-norm block ([MAKEPAD] ViT): affine LayerNorm
 *     (ln*_g / ln*_b), gates fixed at 1.
 *   qk_norm: per-(token, head) norm of q and k over head_dim with the
 *     [head_dim] gamma/beta (order against RoPE: qk_order).
 *   norm: kind of every norm of the block (the two pre-norms, the qk-norm and,
 *     in a stack, the final norm): LayerNorm (x - mean) / sqrt(var + eps), or
 *     RMSNorm x / sqrt(mean(x^2) + eps) ([ERNIE] §IV draws RMSNorm); the
 *     optional gamma/beta are applied after either.
 *   eps: epsilon of every norm of the block.
 *   x_dtype: dtype of x and out (residual arithmetic is fp32 either way).
 *   w_dtype: DIT_BF16, or DIT_F32 for the fp32 path (the fp32 run of the
 *     tiny-block workload): every weight matrix fp32 (w_ada, w_qkv, w_o,
 *     w_gate_up, w_down and, in a stack, w_in, w_fmod, w_out), x_dtype must be
 *     DIT_F32 and fmt 0; every intermediate (h, q, k, vt, the attention
 *     output, u) is then fp32, the GEMMs run on fp32 MFMA and attention on the
 *     vector ALUs, with the same fused epilogues.  DIT_ERR_UNSUPPORTED for
 *     DIT_F32 with a bf16 x or the W8A8 format.
 *   act, gate, mod, qk_order: the semantics switches above; 0 everywhere is
 *     SwiGLU, identity gate, six chunks, norm before RoPE.
 *   fmt: dit_fmt of the four projections (0 = bf16).
 * Built shapes: head_dim in {64, 128}; hidden % 256 == 0; ffn % 128 == 0;
 * (heads + 2 kv_heads) * head_dim % 256 == 0; cond_dim % 8 == 0; any seq >= 1
 * (ragged tails handled in every kernel).  W8A8 H256 also needs ffn % 256 == 0
 * with ceil(ffn / 1024) <= 7 or a multiple of 4 (up to 32). */
typedef struct {
    int32_t batch, seq, hidden, heads, kv_heads, head_dim, ffn, cond_dim;
    int32_t qk_norm;
    int32_t norm;      /* dit_norm  */
    int32_t rope;      /* dit_rope  */
    float eps;
    int32_t x_dtype;   /* dit_dtype */
    int32_t w_dtype;   /* dit_dtype */
    int32_t act;       /* dit_act */
    int32_t gate;      /* dit_gate */
    int32_t mod;       /* dit_mod */
    int32_t qk_order;  /* dit_qk_order */
    int32_t fmt;       /* dit_fmt */
} dit_block_desc;

/* Device pointers to one block's parameters (NULL where marked optional).
 *   w_ada  [6*hidden, cond_dim] bf16, b_ada [6*hidden] fp32: AdaLN linear whose
 *          output splits into (shift1, scale1, gate1, shift2, scale2, gate2)
 *          ([ERNIE] §IV); [4*hidden, ...] split (scale1, gate1, scale2, gate2)
 *          when mod is DIT_MOD_SCALE_GATE.  Required iff cond_dim > 0.
 *   ln1_g, ln1_b, ln2_g, ln2_b [hidden] fp32: affine of the pre-norms; used
 *          only when cond_dim == 0 (NULL = gamma 1 / beta 0); must be NULL in
 *          AdaLN mode.
 *   w_qkv  [(heads + 2 kv_heads) * head_dim, hidden] bf16: rows are the q heads,
 *          then the k heads, then the v heads.
 *   q_g, q_b, k_g, k_b [head_dim] fp32: qk-norm affine; required iff qk_norm.
 *   w_o    [hidden, heads * head_dim] bf16.
 *   w_gate_up [2 * ffn, hidden] bf16: the ffn gate rows first, then the ffn up
 *          rows (SwiGLU: SiLU(gate) * up).
 *   w_down [hidden, ffn] bf16.
 * In the W8A8 H256 format w_qkv, w_o, w_gate_up and w_down hold instead the
 * int8 codes of those matrices (same shapes, from dit_quantize_h256 of the
 * bf16 weights) and s_qkv, s_o, s_gate_up, s_down [rows of each] fp32 their
 * per-row scales (16-byte aligned); the scales are ignored in bf16. */
typedef struct {
    const void *w_ada;
    const float *b_ada;
    const float *ln1_g, *ln1_b, *ln2_g, *ln2_b;
    const void *w_qkv;
    const float *q_g, *q_b, *k_g, *k_b;
    const void *w_o, *w_gate_up, *w_down;
    const float *s_qkv, *s_o, *s_gate_up, *s_down;
} dit_block_weights;

/* ------------------------------------------------------------------------ */
/* Block                                                                     */
/* ------------------------------------------------------------------------ */

/* Bytes of device workspace dit_block_forward needs for `desc`. */
int dit_block_workspace_size(const dit_block_desc *desc, size_t *bytes);

/* out = block(x, cond) ([ERNIE] §IV per-layer compute graph, with the SwiGLU
 * feed-forward and the gated fp32 residual of §VII Decision 1):
 *   m   = W_ada SiLU(cond) + b_ada        -> shift1 scale1 gate1 shift2 scale2 gate2
 *   h   = N(x) (1 + scale1) + shift1      (bf16)
 *   q,k,v = h W_qkv^T; q,k <- RoPE(qkN(q,k))           (bf16)
 *   x1  = x + f(gate1) * (softmax(q k^T / sqrt(hd)) v  W_o^T)   (fp32)
 *   h2  = N(x1) (1 + scale2) + shift2     (bf16)
 *   out = x1 + f(gate2) * ((act(h2 Wg^T) * (h2 Wu^T)) W_down^T)
 * with the defaults N = LayerNorm, qkN before RoPE, f = identity, act = SiLU,
 * and the desc switches norm / qk_order / gate / act / mod (no shift chunks
 * with DIT_MOD_SCALE_GATE).
 * x, out: device [batch*seq, hidden] of desc->x_dtype; out may equal x
 *   (in-place residual, [MAKEPAD]); any other overlap is INVALID_ARG.
 * cond: device fp32 [cond_dim] (NULL iff cond_dim == 0).
 * rope_cos, rope_sin: device fp32 [seq, head_dim/2]: cos/sin of the rotation
 *   angle of pair slot m for sequence position s (see dit_rope_tables); pair
 *   slot m rotates dims (2m, 2m+1) (INTERLEAVED) or (m, m + hd/2) (HALF).
 * ws: device workspace of at least dit_block_workspace_size bytes. */
int dit_block_forward(const dit_block_desc *desc, const dit_block_weights *w,
                      const void *x, const float *cond,
                      const float *rope_cos, const float *rope_sin,
                      void *out, void *ws, size_t ws_bytes, void *stream);

/* dit_block_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same kernels, with the workspace taken from a device array
 * inside the library instead of a `ws` argument.  The array holds
 * dit_block_forward_noalloc_max_bytes() bytes (128 MiB) on every GPU the
 * library runs on, from the library's load on that GPU until the process
 * ends; a block whose dit_block_workspace_size exceeds it returns
 * DIT_ERR_WORKSPACE (nothing is launched).  The call allocates and frees
 * nothing (its first call on a GPU looks the array's address up once).
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (each call writes every scratch slot before reading it): calls
 * that overlap on one GPU (concurrent streams, or several host threads)
 * race and must be serialised by the caller.  Arguments, validation and
 * results as dit_block_forward. */
int dit_block_forward_noalloc(const dit_block_desc *desc, const dit_block_weights *w,
                              const void *x, const float *cond,
                              const float *rope_cos, const float *rope_sin,
                              void *out, void *stream);
size_t dit_block_forward_noalloc_max_bytes(void);

/* A chain of n_blocks blocks of one shape applied in place to x, all with the
 * same conditioning cond: x <- block_{n-1}(... block_0(x, cond) ..., cond)
 * ([ERNIE] §IV: the layers of one denoising step; blocks[l] is a HOST array of
 * weight sets).  When the blocks carry their own AdaLN linear (w_ada / b_ada
 * differ between blocks) and side_stream is a second stream, the modulation
 * GEMV of block l + 1, which is bound by HBM bandwidth, is issued on
 * side_stream while block l runs on `stream` ("layer pipelining", [ERNIE] §IX
 * headroom item 4); events order the two streams (side_stream first waits for
 * the work already on `stream`, and `stream` waits for each GEMV before the
 * block that reads it), so on return every write of the call is ordered on
 * `stream`.  With one shared AdaLN linear the modulation is computed once;
 * side_stream NULL (or equal to stream) runs everything on `stream`.
 * x: device [batch*seq, hidden] of desc->x_dtype; cond, rope tables as
 * dit_block_forward; ws: at least dit_block_chain_workspace_size bytes (the
 * block workspace plus a second modulation buffer).  Results are bitwise
 * those of n_blocks dit_block_forward calls with out == x.  The call creates
 * two HIP events (host-side objects) and destroys them before returning. */
int dit_block_chain_workspace_size(const dit_block_desc *desc, size_t *bytes);
int dit_block_chain_forward(const dit_block_desc *desc, const dit_block_weights *blocks, int32_t n_blocks,
                            void *x, const float *cond, const float *rope_cos, const float *rope_sin,
                            void *ws, size_t ws_bytes, void *stream, void *side_stream);

/* ------------------------------------------------------------------------ */
/* Stack step and denoising loop                                             */
/* ------------------------------------------------------------------------ */

/* A stack of `layers` blocks of one shape plus the stack edges
 * ([ERNIE] §IV and §V Bug 4).  `blocks` is a HOST array of `layers` weight
 * sets (device pointers inside).  Blocks may share one AdaLN linear: when
 * every block's (w_ada, b_ada) equals block 0's, the modulation is computed
 * once per step.  blk.x_dtype must be DIT_F32 (fp32 residual stream).
 *   w_in  [hidden, latent_dim] bf16, b_in [hidden] fp32: patch embedding.
 *   w_fmod [2*hidden, cond_dim] bf16, b_fmod [2*hidden] fp32: final
 *         modulation, chunks (scale, shift) -- the reverse of the per-layer
 *         order ([ERNIE] §V Bug 4); applied to cond without SiLU.
 *   w_out [latent_dim, hidden] bf16, b_out [latent_dim] fp32. */
typedef struct {
    dit_block_desc blk;
    int32_t layers, latent_dim;
    const dit_block_weights *blocks;
    const void *w_in;
    const float *b_in;
    const void *w_fmod;
    const float *b_fmod;
    const void *w_out;
    const float *b_out;
} dit_model;

int dit_stack_workspace_size(const dit_model *model, size_t *bytes);

/* velocity = final(block_{L-1}(... block_0(latent W_in^T + b_in, cond) ...), cond)
 * with final(x, c) = (LN(x)(1 + scale_f) + shift_f) W_out^T + b_out.
 * latent (read-only), velocity: device fp32 [batch*seq, latent_dim].
 * cond: device fp32 [cond_dim] (e.g. from dit_timestep_embedding).
 * The latent is rounded to bf16 before the patch-embedding GEMM. */
int dit_stack_step(const dit_model *model, const float *latent, const float *cond,
                   const float *rope_cos, const float *rope_sin, float *velocity,
                   void *ws, size_t ws_bytes, void *stream);

/* latent[i] += (sigma_next - sigma) * velocity[i] for i < n, fp32, in place
 * (flow-match Euler step; [ZML] §IV "Euler sign +1"). */
int euler_flowmatch_update(float *latent, const float *velocity, int64_t n,
                           float sigma, float sigma_next, void *stream);

/* cond_out[j] = cos(t w_j), cond_out[dim/2 + j] = sin(t w_j),
 * w_j = exp(-ln(10000) j / (dim/2)): the flip_sin_to_cos sinusoidal timestep
 * features ([ZML] §IV).  dim even, > 0; cond_out device fp32 [dim]. */
int dit_timestep_embedding(float t, int32_t dim, float *cond_out, void *stream);

/* The conditioning of denoising step sigma: dit_timestep_embedding at
 * t = 1000 sigma (the scheduler's timestep scale; [ZML] §IV timestep
 * sinusoid), with the product taken in fp32 inside the library.  sigma must
 * be finite; dim and cond_out as dit_timestep_embedding. */
int dit_sigma_embedding(float sigma, int32_t dim, float *cond_out, void *stream);

/* ------------------------------------------------------------------------ */
/* Whole denoising loop, recorded once as HIP graphs                         */
/* ------------------------------------------------------------------------ */

/* The flow-match Euler loop of [ERNIE] §I (8 steps, shift 4.0, sigma grid of
 * dit_flowmatch_sigmas) with each step = dit_sigma_embedding(sigma_i)
 * -> dit_stack_step -> euler_flowmatch_update(sigma_i, sigma_{i+1}), recorded
 * into one HIP graph per step so that replaying a step costs one launch
 * instead of ~300 ([ZML] §XI: host round trips dominate small steps).
 *
 * Workspace: dit_loop_workspace_size bytes = the stack workspace followed by
 * the conditioning vector [cond_dim] and the velocity [batch*seq, latent_dim]
 * (fp32).  The loop keeps the pointers it was created with: model weights,
 * rope tables, latent and ws must stay allocated and at the same addresses
 * until dit_loop_destroy; the model struct itself may be freed after create.
 * The latent (device fp32 [batch*seq, latent_dim]) is updated in place by
 * every replayed step; refill it to start a new loop.
 * The loop object owns host-side graph resources only (no device buffers). */
typedef struct dit_loop dit_loop;

int dit_loop_workspace_size(const dit_model *model, size_t *bytes);

/* Validates like dit_stack_step, then records steps graphs on a private
 * stream (nothing runs yet).  steps in [1, 1000], shift > 0.
 * On success *loop receives the handle; on error *loop is left NULL. */
int dit_loop_create(const dit_model *model, float *latent, const float *rope_cos,
                    const float *rope_sin, int32_t steps, float shift, void *ws,
                    size_t ws_bytes, dit_loop **loop);

/* Replays step `step` (0-based, < steps) on `stream`, asynchronously. */
int dit_loop_launch_step(dit_loop *loop, int32_t step, void *stream);

/* Replays all steps in order on `stream`, asynchronously. */
int dit_loop_launch(dit_loop *loop, void *stream);

/* Frees the graphs.  NULL is accepted.  The caller must not destroy a loop
 * whose replays are still running (synchronise the stream first). */
int dit_loop_destroy(dit_loop *loop);

/* ------------------------------------------------------------------------ */
/* Host helpers (no device work)                                             */
/* ------------------------------------------------------------------------ */

/* sigmas_out[i] = shift * s / (1 + (shift - 1) s), s = 1 - i/steps, i = 0..steps
 * (FlowMatchEulerDiscreteScheduler grid with the time shift, [ERNIE] §I).
 * sigmas_out: host fp32 [steps + 1]. */
int dit_flowmatch_sigmas(int32_t steps, float shift, float *sigmas_out);

/* RoPE cos/sin tables for `seq` positions.  pos: host int32 [seq, 3] (t, h, w).
 * The head dim is split into contiguous per-axis chunks of widths axes[0..n_axes)
 * (sum = head_dim); pair slot j of the chunk of axis a rotates by
 * pos_a * theta^(-2j / axes[a]).  rope == INTERLEAVED uses axes (t, h, w)
 * (n_axes 3, [ERNIE] §I axes [32,48,48] theta 256); rope == HALF uses (h, w)
 * (n_axes 2, the ViT of [MAKEPAD]).  cos_out, sin_out: host fp32 [seq, head_dim/2]. */
int dit_rope_tables(const int32_t *pos, int32_t seq, int32_t rope, const int32_t *axes,
                    int32_t n_axes, float theta, int32_t head_dim,
                    float *cos_out, float *sin_out);

/* ------------------------------------------------------------------------ */
/* Stage entry points: each stage of dit_block_forward on its own, with the  */
/* same kernels, for per-stage parity checks and timing.                     */
/* ------------------------------------------------------------------------ */

/* m[o] = sum_k W[o,k] act(c[k]) + b[o], act = SiLU if silu_input else identity.
 * W device bf16 [out_dim, in_dim]; b device fp32 [out_dim] or NULL; c device
 * fp32 [in_dim]; m device fp32 [out_dim].  in_dim % 8 == 0.
 * ([ERNIE] §IV AdaLN modulation; §V Bug 4 final modulation without SiLU.) */
int dit_adaln_modulation(const void *w, const float *b, const float *c, int32_t out_dim,
                         int32_t in_dim, int32_t silu_input, float *m, void *stream);

/* Row norm + modulation to bf16: h = norm(x) * mul + add, norm = LayerNorm or
 * RMSNorm (dit_norm), where
 * mode 0: mul = 1 + scale, add = shift (AdaLN; scale fp32 [dim] required,
 *         shift fp32 [dim] or NULL = 0 for the no-shift modulation);
 * mode 1: mul = scale, add = shift (affine norm; either may be NULL = 1 / 0).
 * x device [rows, dim] of x_dtype; h device bf16 [rows, dim]; dim % 256 == 0,
 * dim <= 8192. */
int dit_ln_modulate(const void *x, int32_t x_dtype, int64_t rows, int32_t dim, int32_t norm,
                    const float *shift, const float *scale, int32_t mode, float eps,
                    void *h, void *stream);

/* QKV GEMM with the qk-LayerNorm and RoPE epilogue.
 * h device bf16 [batch*seq, hidden]; outputs (device bf16; with
 * desc->w_dtype == DIT_F32, h, w_qkv and the outputs are fp32):
 *   q  [batch, heads, seq, head_dim]
 *   k  [batch, kv_heads, seq, head_dim]
 *   vt [batch, kv_heads, head_dim, seq_pad], seq_pad = dit_seq_pad(seq):
 *      V transposed; positions [seq, seq_pad) are written with zeros.
 * The bf16 path normalises q and k either from the fp32 projection or, for
 * 128-wide heads and seq % 16 == 0 when the GEMM fills whole rounds of
 * 256 x 256 tiles, from the projection rounded to bf16 (written to q / k,
 * then normalised in place by a second kernel on the same stream). */
int dit_qkv_rope(const dit_block_desc *desc, const void *h, const void *w_qkv,
                 const float *q_g, const float *q_b, const float *k_g, const float *k_b,
                 const float *rope_cos, const float *rope_sin,
                 void *q, void *k, void *vt, void *stream);

/* Padded key count of the transposed V layout: seq rounded up to 64. */
int32_t dit_seq_pad(int32_t seq);

/* Mask-free flash attention: out[b*seq + s, h*hd + d] =
 * sum_j softmax_j(q[b,h,s,:] . k[b,g,j,:] / sqrt(hd)) v[b,g,j,d], g = h/(H/Hkv)
 * ([ERNIE] §VII Decision 2 and §IX "Flash SDPA").  q, k, vt in the layouts of
 * dit_qkv_rope; out device bf16 [batch*seq, heads*head_dim] (all fp32 with
 * desc->w_dtype == DIT_F32).  The padded key positions of vt must hold
 * zeros (dit_qkv_rope writes them). */
int dit_flash_attention(const dit_block_desc *desc, const void *q, const void *k,
                        const void *vt, void *out, void *stream);

/* dit_flash_attention with the last, partial q tile (seq % 256 rows) of each
 * (batch, head) split over nsplit chunks of whole 64-key tiles, each chunk
 * one workgroup writing its unnormalised output, softmax reference max and
 * row sum (fp32) to ws, merged by a second kernel (the split-KV form of the
 * online softmax); dit_block_forward uses it for ragged sequences such as the
 * joint 4096 + 74 token layout ([ERNIE] "Token Layout").  nsplit in [1, 64]
 * (chunks hold at least one key tile; nsplit 1, or seq a multiple of 256,
 * is dit_flash_attention).  ws: device workspace of at least
 * dit_attention_workspace_size(desc, nsplit) bytes (may be NULL when that is 0).
 * The fp32 path (desc->w_dtype == DIT_F32) has no split form:
 * DIT_ERR_UNSUPPORTED. */
int dit_attention_workspace_size(const dit_block_desc *desc, int32_t nsplit, size_t *bytes);
int dit_flash_attention_split(const dit_block_desc *desc, const void *q, const void *k, const void *vt,
                              void *out, int32_t nsplit, void *ws, size_t ws_bytes, void *stream);

/* out = resid + f(gate) * (a W^T) + bias over an [M, N] output, f = the gate
 * function gate_fn (dit_gate):
 * a device bf16 [M, K]; W device bf16 [N, K]; resid device [M, N] of
 * resid_dtype or NULL; gate, bias device fp32 [N] or NULL (gate NULL = 1
 * whatever gate_fn, bias NULL = 0); out device [M, N] of out_dtype (may equal
 * resid).
 * N % 128 == 0, K % 64 == 0.  ([ERNIE] §VII Decision 1: gated residual with
 * fp32 accumulation; out-projection and down-projection epilogue.) */
int dit_gemm_gated_residual(const void *a, const void *w, int64_t M, int32_t N, int32_t K,
                            const void *resid, int32_t resid_dtype, const float *gate,
                            int32_t gate_fn, const float *bias, void *out, int32_t out_dtype,
                            void *stream);

/* u = act(a Wg^T) * (a Wu^T) with W = [Wg; Wu] device bf16 [2F, K], act =
 * SiLU or the clamped GELU-tanh (dit_act); a device bf16 [M, K]; u device
 * bf16 [M, F].  F % 128 == 0, K % 64 == 0. */
int dit_gemm_swiglu(const void *a, const void *w_gate_up, int64_t M, int32_t F, int32_t K,
                    int32_t act, void *u, void *stream);

/* ------------------------------------------------------------------------ */
/* W8A8 H256 stage entry points ([ZML] §VII; dit_fmt above)                  */
/* ------------------------------------------------------------------------ */

/* Per-row rotation and int8 codes: for each row r, v = x[r] blockdiag(H256),
 * scale[r] = max|v| / 127, q[r, c] = round-half-even(v_c * (127 / max|v|))
 * in [-127, 127] (a zero row: codes 0, scale 0), decided in fp32.
 * x device [rows, cols] of x_dtype; q device int8 [rows, cols]; scale device
 * fp32 [rows]; no overlap between them.  cols % 256 == 0 with
 * ceil(cols / 1024) <= 7 or a multiple of 4 (up to 32).  Prepares the weights
 * of the W8A8 format (once) and, inside the block, the attention and GLU
 * outputs before their projections. */
int dit_quantize_h256(const void *x, int32_t x_dtype, int64_t rows, int32_t cols, void *q, float *scale,
                      void *stream);

/* dit_ln_modulate followed by dit_quantize_h256 of h, with h kept in fp32
 * registers (never written): q device int8 [rows, dim], qscale device fp32
 * [rows].  Arguments and shapes as dit_ln_modulate. */
int dit_ln_modulate_h256q(const void *x, int32_t x_dtype, int64_t rows, int32_t dim, int32_t norm,
                          const float *shift, const float *scale, int32_t mode, float eps, void *q, float *qscale,
                          void *stream);

/* The projections of the W8A8 format.  a: device int8 codes [M, K] with
 * a_scale fp32 [M]; w: device int8 codes [rows, K] with w_scale fp32 [rows]
 * (rows = N, 2F or the QKV width), all 16-byte aligned.  The product
 * C[m, n] = a_scale[m] w_scale[n] sum_k a[m, k] w[n, k] is summed exactly in
 * int32, converted to fp32 and fed to the epilogue of the bf16 call of the
 * same name (dit_gemm_gated_residual, dit_gemm_swiglu, dit_qkv_rope), whose
 * other arguments, layouts and limits it keeps (for the QKV projection also
 * its choice between the fp32 and the bf16-rounded product as the input of the
 * qk-norm); K % 128 == 0. */
int dit_gemm_w8a8_gated_residual(const void *a, const float *a_scale, const void *w, const float *w_scale,
                                 int64_t M, int32_t N, int32_t K, const void *resid, int32_t resid_dtype,
                                 const float *gate, int32_t gate_fn, const float *bias, void *out,
                                 int32_t out_dtype, void *stream);
int dit_gemm_w8a8_swiglu(const void *a, const float *a_scale, const void *w_gate_up, const float *w_scale,
                         int64_t M, int32_t F, int32_t K, int32_t act, void *u, void *stream);
int dit_qkv_rope_w8a8(const dit_block_desc *desc, const void *h, const float *h_scale, const void *w_qkv,
                      const float *w_scale, const float *q_g, const float *q_b, const float *k_g,
                      const float *k_b, const float *rope_cos, const float *rope_sin, void *q, void *k,
                      void *vt, void *stream);

/* ------------------------------------------------------------------------ */
/* Tracing                                                                   */
/* ------------------------------------------------------------------------ */

/* Per-launch GPU times, the per-operation breakdown of a step ([ERNIE] §IX
 * "Per-Step Latency Breakdown", produced there by a Chrome-trace tracer).
 * While tracing is on, every kernel launch of the library records a HIP event
 * on its stream before and after its kernels, with the operation's name and
 * shape; nothing synchronises while recording, and launches into a stream
 * that is being captured into a HIP graph are not recorded.
 * dit_trace_begin: discards earlier records and starts recording at most
 * `capacity` launches (1 .. 2^24; further launches are counted as dropped).
 * dit_trace_end: waits for the recorded launches, writes Chrome trace JSON
 * (one complete "X" event per launch, "tid" = the stream, "ts"/"dur" in
 * microseconds from dit_trace_begin) to `path` (NULL: the path DIT_TRACE
 * named), releases the records and stops recording.  DIT_ERR_INVALID_ARG
 * when not tracing or the file cannot be written.
 * Environment: DIT_TRACE=<path> (or 1 for ./dit_trace.json) starts tracing at
 * the library's first launch; DIT_DEBUG_SYNC=1 synchronises the stream after
 * every launch and prints the first failing operation (debugging only).
 * Tracing is process-wide; calls from several threads are serialised. */
int dit_trace_begin(int32_t capacity);
int dit_trace_end(const char *path);

/* ------------------------------------------------------------------------ */
const char *dit_status_string(int status);
const char *dit_last_error(void);
/* Library version string. */
const char *dit_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DIT_H */
