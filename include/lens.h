/*
 * lens.h -- C ABI of the MI355X (gfx950) Lens MM-DiT denoiser library.
 *
 * The library runs the forward pass of the Lens double-stream MM-DiT
 * denoiser (48 blocks, hidden 1536 = 24 heads x 64, separate image and text
 * weights, per-stream AdaLN, RMSNorm + modulation, QK RMSNorm, 3-axis RoPE,
 * joint text+image attention, gated SwiGLU MLP) and the flow-matching Euler
 * step with classifier-free guidance, on hand-written HIP kernels.
 *
 * Sources, by page and section:
 *   Lens blog post (zjwfufu.github.io), "Overview": 48 blocks, hidden 1536,
 *     24 heads, gated MLP 1536x4096, per-stream AdaLN 1536x9216 giving a
 *     shift/scale/gate triple before attention and another before the MLP;
 *     "Exploring Text Encoder": zero-padded text is masked out of the DiT;
 *     "Exploring Image Editing": the CFG combination.
 *   Lens-Turbo-3.8B-bf16 article (wmrh.cn): per-block tensors img_qkv /
 *     txt_qkv, norm_q / norm_k / norm_added_q / norm_added_k, to_out /
 *     to_add_out, img_mod / txt_mod, img_mlp / txt_mlp w1 w2 w3; rms_norm;
 *     axes_dims_rope [8, 28, 28]; in_channels 128 (2x2 patches of 32
 *     channels); txt_norm.0..3; norm_out.linear and proj_out.
 *   "Lens: Rethinking Training Efficiency ..." summary, 前置知识: the flow
 *     matching path x_t = (1 - t) x0 + t x1 and its velocity target.
 *   SOTA image generation survey (youngju.dev), "CFG" and "Rectified Flow".
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  Config and
 *     weight-table structs are HOST memory, read only during the call.
 *   - Work is enqueued on `hip_stream` (a hipStream_t passed as void*;
 *     NULL = the default stream).  A return of LENS_OK means "enqueued":
 *     no device synchronisation is done.
 *   - Argument checks are synchronous; a failure returns a negative status
 *     and sets a thread-local message readable with lens_last_error().
 *     Nothing is enqueued when a check fails.
 *   - The library allocates no device memory; scratch space is the caller's
 *     workspace, sized by the *_workspace_bytes functions (256-byte aligned).
 *   - Matrices are row-major.  A Linear layer's weight is [out, in] (the
 *     input dimension contiguous) and its bias is [out] or NULL.
 *   - Device tensors that the kernels access in 16-byte pieces must start on
 *     a 16-byte boundary (torch allocations do): activations (x, txt_feats,
 *     h_img, h_txt), outputs (v_out, q_out), every weight, bias, gain and
 *     w_scale.  t, positions, txt_len and the flow-step vectors need only
 *     their element alignment.  A misaligned tensor is LENS_ERR_INVALID_ARG.
 *   - Arguments and fields that name a lens_dtype or lens_status value are
 *     declared int32_t, so that any integer a caller passes is checked (an
 *     unknown value is LENS_ERR_INVALID_ARG) rather than read as an enum.
 *   - Activation / weight element type is cfg->act_dtype (LENS_BF16 or
 *     LENS_F32); residual streams, the timestep embedding, latents x (in the
 *     flow step) and the velocity v are always float32.  bf16 is stored as
 *     IEEE bfloat16 bit patterns, rounded to nearest even.
 */
#ifndef LENS_H
#define LENS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LENS_OK = 0,
  LENS_ERR_INVALID_ARG = -1, /* NULL pointer, bad size, inconsistent config */
  LENS_ERR_UNSUPPORTED = -2, /* valid but not implemented (e.g. head_dim != 64) */
  LENS_ERR_WORKSPACE = -3,   /* workspace NULL or smaller than required */
  LENS_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
} lens_status;

typedef enum { LENS_F32 = 0, LENS_BF16 = 1 } lens_dtype;

/* Model configuration; lens_default_config() fills the Lens values. */
typedef struct {
  int32_t hidden;       /* 1536 = heads * head_dim */
  int32_t heads;        /* 24 */
  int32_t head_dim;     /* 64 (the only supported value) */
  int32_t mlp_hidden;   /* 4096 */
  int32_t n_blocks;     /* 48 */
  int32_t rope_axes[3]; /* 8, 28, 28: even, summing to head_dim */
  int32_t in_ch;        /* 128 features per patchified image token */
  int32_t out_ch;       /* 128 */
  int32_t txt_feat_dim; /* 2880 per encoder layer */
  int32_t txt_layers;   /* 4 */
  int32_t t_freq_dim;   /* 256 sinusoidal timestep features */
  float rope_theta;     /* 10000 */
  float eps;            /* 1e-6, all RMSNorms */
  float t_scale;        /* 1000: the sinusoid sees t_scale * t */
  int32_t act_dtype;    /* a lens_dtype: element type of weights and activations */
  int32_t gemm_fp8;     /* 1: the block projections qkv, out, w1, w3, w2 run as
                           MX fp8 GEMMs (requires act_dtype LENS_BF16; see
                           lens_quantize_mxfp8): their inputs are quantized
                           from fp32 by the kernels that produce them (the
                           two norms, attention, the SwiGLU epilogue), with
                           the same rule as lens_quantize_mxfp8;
                           0 (default): act_dtype */
} lens_config;

/* One Linear layer: w [out, in] in act_dtype, b [out] in act_dtype or NULL.
 * With cfg->gemm_fp8, the qkv, out, w1, w3 and w2 layers of every block
 * instead hold w as MX fp8: e4m3 bytes [out, in] with w_scale its E8M0
 * scales in the LENS_MX_SLABS layout (lens_quantize_mxfp8 of the act_dtype
 * weight with scale_layout LENS_MX_SLABS; in % 128 == 0); b
 * stays in act_dtype.  w_scale is ignored otherwise. */
typedef struct {
  const void *w;
  const void *b;
  const void *w_scale;
} lens_linear;

/* Weights of one stream of one block.  q_gain / k_gain: [head_dim] gains of
 * the per-head RMSNorm of q and k (norm_q / norm_k for the image stream,
 * norm_added_q / norm_added_k for the text stream).  mod: 6*hidden outputs in
 * the order shift1, scale1, gate1, shift2, scale2, gate2.  qkv: 3*hidden
 * outputs q | k | v, each heads x head_dim.  w1 = gate, w3 = up, w2 = down. */
typedef struct {
  lens_linear mod, qkv, out, w1, w3, w2;
  const void *q_gain, *k_gain;
} lens_stream_w;

typedef struct {
  lens_stream_w img, txt;
} lens_block_w;

/* Non-block weights.  t_fc1: [hidden, t_freq_dim]; t_fc2: [hidden, hidden];
 * img_in: [hidden, in_ch]; txt_gain: [txt_layers, txt_feat_dim] (one
 * device array); txt_in: [hidden, txt_layers * txt_feat_dim]; norm_out:
 * [2*hidden, hidden] giving shift then scale; proj_out: [out_ch, hidden].
 * blocks: HOST array of n_blocks block tables, run in array order. */
typedef struct {
  lens_linear t_fc1, t_fc2, img_in, txt_in, norm_out, proj_out;
  const void *txt_gain;
  const lens_block_w *blocks;
} lens_dit_w;

/* Fills *cfg with the Lens configuration and the given activation type. */
void lens_default_config(lens_config *cfg, int32_t act_dtype /* a lens_dtype */);

/* Bytes of workspace lens_block_forward / lens_dit_forward need for batch B,
 * S_img image tokens and S_txt text tokens; 0 if the arguments are invalid. */
size_t lens_block_workspace_bytes(const lens_config *cfg, int32_t B, int32_t S_img, int32_t S_txt);
size_t lens_dit_workspace_bytes(const lens_config *cfg, int32_t B, int32_t S_img, int32_t S_txt);

/*
 * One double-stream block, in place on the residual streams.
 * Sources: the MMDiT block of the Lens paper summary (前置知识: each stream
 * keeps its own weights and the two meet in one joint attention), the Lens
 * blog's "Overview" (the AdaLN triple shift/scale/gate before attention and
 * before the gated 1536x4096 MLP), and the Lens-Turbo-3.8B-bf16 article's
 * "双流注意力机制", "自适应调制与 RMSNorm" and "3D RoPE" sections (per-stream
 * qkv, per-head q/k RMSNorm with per-stream gains, RoPE axes [8, 28, 28]);
 * padded text is masked per the blog's "Exploring Text Encoder".
 *   h_img [B, S_img, hidden] f32, h_txt [B, S_txt, hidden] f32: updated.
 *   temb  [B, hidden] f32: timestep embedding; AdaLN is computed inside as
 *         mod = W_mod . SiLU(temb) + b_mod for each stream.
 *   img_pos [S_img, 3], txt_pos [S_txt, 3] int32 RoPE positions (the same
 *         for every sample of the batch).
 *   txt_len [B] int32 valid text lengths (device), or NULL = all S_txt valid.
 *         Text keys j >= txt_len[b] are masked; values are clamped to
 *         [0, S_txt].  Rows of masked text queries hold unspecified
 *         values (their attention is skipped where a whole 128-query block
 *         of them would be computed for nothing).
 * Per stream: a = RMSNorm(h)(1 + scale1) + shift1; qkv = a W_qkv^T + b;
 * q, k <- RMSNorm_64(.) * gain, then RoPE; joint softmax attention of each
 * sample's image and text queries over all of its valid keys, scale
 * 1/sqrt(head_dim); h += gate1 (O W_out^T + b); a = RMSNorm(h)(1 + scale2)
 * + shift2; h += gate2 (W2 (SiLU(W1 a + b1) (W3 a + b3)) + b2).
 * Requires B >= 1, S_img >= 1, S_txt >= 0.
 */
lens_status lens_block_forward(const lens_config *cfg, const lens_block_w *w, float *h_img, float *h_txt,
                               const float *temb, const int32_t *img_pos, const int32_t *txt_pos,
                               const int32_t *txt_len, int32_t B, int32_t S_img, int32_t S_txt,
                               void *workspace, size_t ws_bytes, void *hip_stream);

/*
 * Whole denoiser: v = proj_out(norm_out(blocks(img_in(x), txt_in(f)), temb)).
 * Sources: the Lens-Turbo-3.8B-bf16 article's architecture table and its
 * "Patchify 补丁化与输出投影" (img_in on 2x2 patches of the 32-channel latent,
 * norm_out.linear, proj_out), "多层级文本特征融合" (txt_norm.0..3 on four
 * encoder layers, concatenated and projected by txt_in; also the Lens paper
 * summary, 核心方法) and "自适应调制与 RMSNorm" (time_text_embed's timestep
 * MLP); 48 blocks per the Lens blog's "Overview".
 *   x         [B, S_img, in_ch] act_dtype: patchified latent tokens (read only).
 *   txt_feats [B, S_txt, txt_layers * txt_feat_dim] act_dtype, layer-major.
 *   t         [B] f32 timesteps (device).
 *   positions and txt_len as for lens_block_forward.
 *   v_out     [B, S_img, out_ch] f32 velocity.
 * temb = t_fc2(SiLU(t_fc1(phi(t)))), phi(t) = [cos(t_scale t w_k) | sin(...)],
 * w_k = 10000^(-k / (t_freq_dim/2)); the text input is RMSNorm(layer) *
 * txt_gain[layer] for each layer, concatenated, then txt_in.  The final layer
 * computes (shift, scale) = norm_out(SiLU(temb)) and v = proj_out(
 * RMSNorm(h_img)(1 + scale) + shift).
 * For classifier-free guidance put the cond samples in [0, n) and the uncond
 * samples in [n, 2n) of one batch (x and t duplicated) and pass the two halves
 * of v_out to lens_flow_step.
 */
lens_status lens_dit_forward(const lens_config *cfg, const lens_dit_w *w, const void *x, const void *txt_feats,
                             const float *t, const int32_t *img_pos, const int32_t *txt_pos,
                             const int32_t *txt_len, int32_t B, int32_t S_img, int32_t S_txt, float *v_out,
                             void *workspace, size_t ws_bytes, void *hip_stream);

/*
 * lens_dit_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, computation and results
 * as lens_dit_forward; its scratch is a file-scope device array of
 * LENS_NOALLOC_SCRATCH_BYTES (384 MiB: the 1024^2 cond + uncond launch, B = 2,
 * needs 274 MiB in bf16 and 325 MiB with gemm_fp8; 1440^2 at B = 1 needs
 * 245 MiB) that every GPU the library runs on holds from the library's load
 * until the process ends.  The call allocates nothing (no hipMalloc, no
 * allocating library routine).  A call whose lens_dit_workspace_bytes exceeds
 * LENS_NOALLOC_SCRATCH_BYTES returns LENS_ERR_WORKSPACE before any device
 * work.  All calls on one GPU share that GPU's array and nothing of one call
 * carries into the next (each call writes every intermediate before reading
 * it); calls that overlap on one GPU (other streams, other threads) race on
 * it and must be serialised by the caller.
 */
#define LENS_NOALLOC_SCRATCH_BYTES ((size_t)384 << 20)
lens_status lens_dit_forward_noalloc(const lens_config *cfg, const lens_dit_w *w, const void *x,
                                     const void *txt_feats, const float *t, const int32_t *img_pos,
                                     const int32_t *txt_pos, const int32_t *txt_len, int32_t B, int32_t S_img,
                                     int32_t S_txt, float *v_out, void *hip_stream);

/*
 * Flow-matching Euler step with optional classifier-free guidance, on n
 * elements:  v = v_uncond + cfg_scale (v_cond - v_uncond)  (v = v_cond when
 * v_uncond is NULL);  x <- x + dt v.
 * Sources: the SOTA image generation survey's "CFG" (the guided combination)
 * and "Rectified Flow" (integrating the learned velocity with Euler steps),
 * the Lens paper summary's 前置知识 (the straight path x_t = (1 - t) x0 +
 * t x1 whose velocity the denoiser predicts; noise at t = 1), and the
 * Lens-Turbo-3.8B-bf16 article (guidance 1.0: v_uncond NULL).  x f32 is updated in place; v_cond and
 * v_uncond are f32.  If x_lowp_out is not NULL it receives the new x in
 * lowp_dtype (the input of the next lens_dit_forward).  n >= 0.
 */
lens_status lens_flow_step(float *x, const float *v_cond, const float *v_uncond, int64_t n, float dt,
                           float cfg_scale, void *x_lowp_out, int32_t lowp_dtype, void *hip_stream);

/*
 * Flow-matching Euler step with norm-rescaled classifier-free guidance, on
 * n_tokens tokens of `channels` contiguous f32 elements each (the latent
 * token layout [.., S_img, out_ch] of v_out: channels = out_ch).  Per token:
 *   comb = v_uncond + cfg_scale (v_cond - v_uncond)   (comb = v_cond when
 *          v_uncond is NULL),
 *   comb <- comb * ||v_cond|| / ||comb||               (unchanged where
 *          ||comb|| = 0; 2-norms over the token's channels),
 *   x <- x + dt comb.
 * Source: Lens blog (zjwfufu.github.io), "Exploring Image Editing": Lens's
 * inference uses a norm-rescaled CFG; the page prints only the combination,
 * and the rescale of each token to the conditional norm is the reading
 * taken here.  x is updated in place; x_lowp_out and lowp_dtype as for
 * lens_flow_step.  Requires n_tokens >= 0, channels >= 1; x, v_cond and
 * v_uncond must not overlap x_lowp_out.
 */
lens_status lens_flow_step_rescaled(float *x, const float *v_cond, const float *v_uncond, int64_t n_tokens,
                                    int32_t channels, float dt, float cfg_scale, void *x_lowp_out,
                                    int32_t lowp_dtype, void *hip_stream);

/*
 * MX-style fp8 quantization (e4m3 elements, one E8M0 scale per 32, with a
 * non-saturating scale rule that differs from OCP MX v1.0's floor(log2 amax)
 * - 8) of a row-major matrix along its rows: src [rows, cols]
 * (src_dtype LENS_BF16 or LENS_F32, cols a positive multiple of 32) ->
 * q_out [rows, cols] e4m3 bytes and scale_out rows * cols / 32 E8M0 bytes
 * (value = 2^(byte - 127)), one per block of 32 consecutive elements of a
 * row; the scale of (row r, block j) sits at byte
 *   LENS_MX_ROWS:  r * (cols / 32) + j
 *   LENS_MX_SLABS: ((j / 4) * rows + r) * 4 + j % 4   (cols % 128 == 0)
 * (slab-major: per 128-wide slab of a row its 4 scales form one 4-byte
 * word, and the words of consecutive rows are adjacent; the layout the fp8
 * GEMMs read, so w_scale of cfg->gemm_fp8 layers uses it).  Per block the scale
 * is the smallest power of two 2^e with max|x| <= 448 2^e (e clamped to
 * [-127, 127]; an all-zero block gets e = -127), and each element is
 * x / 2^e rounded to the nearest e4m3 value, ties to even.  This is the
 * weight format of cfg->gemm_fp8 (the low-precision DiT variant of the
 * Lens-3.8B-4bit pipeline article (2kiu.com), section 4: projection weights
 * quantized, img_in, txt_in, proj_out, the embedders and norm_out kept in
 * bf16; here as MX fp8 rather than int4, the format the MI355X matrix cores
 * take directly).  Device pointers; rows >= 0.
 */
enum { LENS_MX_ROWS = 0, LENS_MX_SLABS = 1 };
lens_status lens_quantize_mxfp8(const void *src, int32_t src_dtype, int64_t rows, int32_t cols,
                                int32_t scale_layout, void *q_out, void *scale_out, void *hip_stream);

/*
 * Opt-in kernel timer for measurement.  lens_timer_start(mask) makes every
 * later launch of the kernel families whose bit (1 << lens_kernel_kind) is
 * set record a pair of HIP events around itself, on the stream it is
 * launched on.  lens_timer_stop(ms, launches) synchronises those events,
 * writes the summed kernel milliseconds and kernel launch counts per family
 * into ms[LENS_KERNEL_COUNT] and launches[LENS_KERNEL_COUNT] (either may be
 * NULL), and switches the timer off.  A call that launches two kernels of a
 * family back to back (the w1 | w3 GEMM may) records one span and counts
 * two launches.  The timer state is per calling
 * thread: start and stop on the thread that makes the timed calls.
 */
typedef enum {
  LENS_KERNEL_GEMM = 0,        /* bf16 MFMA GEMM (all projections) */
  LENS_KERNEL_ATTENTION = 1,   /* joint flash attention */
  LENS_KERNEL_NORM = 2,        /* RMSNorm + modulation (bf16 or MX fp8 output) */
  LENS_KERNEL_QKNORM_ROPE = 3, /* QK RMSNorm + RoPE + joint layout */
  LENS_KERNEL_ADALN = 4,       /* skinny GEMV (AdaLN, timestep MLP) */
  LENS_KERNEL_COUNT = 5
} lens_kernel_kind;
lens_status lens_timer_start(uint32_t kind_mask);
lens_status lens_timer_stop(double *ms, int64_t *launches);

/*
 * Sampling grid of the flow-matching Euler loop (HOST computation, host
 * pointers).  t_out[k], k = 0..steps, and dt_out[k] = t_out[k + 1] -
 * t_out[k], k < steps (either may be NULL), as float:
 *   t_k = 1 - k / steps           (noise at t = 1, data at t = 0: the path
 *                                  x_t = (1 - t) x0 + t x1 of the Lens paper
 *                                  summary, 前置知识),
 *   and with has_mu != 0 each point moved to e^mu t / (e^mu t + 1 - t), a
 *   translation by mu in logit space that keeps t = 0 and t = 1 fixed.  The
 *   same summary (前置知识, 方法步骤详情) trains on logit-normal timesteps
 *   whose location mu grows linearly with the token count (mu = 1.06 for
 *   the 512^2 stage); shifting the inference grid by that mu is the
 *   reading taken here.  Computed in double, rounded once to float.
 * Requires steps >= 1 and a finite mu; otherwise LENS_ERR_INVALID_ARG.
 */
lens_status lens_time_grid(int32_t steps, float mu, int32_t has_mu, float *t_out, float *dt_out);

/*
 * mu of the timestep shift at n_tokens image tokens, on the straight line
 * through (n0, mu0) and (n1, mu1) (Lens paper summary, 方法步骤详情: mu is
 * interpolated linearly in the token count; the pages give one point,
 * mu = 1.06 at 512^2 = 1024 tokens, so the second is the caller's).
 * HOST computation; *mu_out receives the value.  Requires n0 != n1, finite
 * arguments and mu_out non-NULL; otherwise LENS_ERR_INVALID_ARG.
 */
lens_status lens_mu_for_tokens(int64_t n_tokens, double n0, double mu0, double n1, double mu1, double *mu_out);

const char *lens_status_string(int32_t status /* a lens_status */);
const char *lens_last_error(void);
const char *lens_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LENS_H */
