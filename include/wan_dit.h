/*
 * wan_dit.h -- C ABI of libwandit, the gfx950 (MI355X) implementation of one
 * Wan2.1 Diffusion-Transformer denoising step.
 *
 * Sources the operations follow (page title, section):
 *   [Note] "Wan: Open and Advanced Large-Scale Video Generative Models
 *          (Wan 2.1)", sections 模型架构 (Wan-VAE, Diffusion Transformer),
 *          配置表, I2V 架构扩展, 训练方法.
 *   [News] "超越Sora！阿里正式完全开源最新、最强大的视频生成模型 Wan2.1",
 *          sections 核心创新二 (视频扩散 DiT) and 核心创新四 (Image-to-Video).
 *   [Guide] "Wan 2.1 AI：下一代开源视频生成技术的突破性实践", section 工作原理
 *          (the sampling knobs: number of inference steps, guidance scale).
 *
 * Conventions shared by every entry point
 *   - Row-major.  Linear weights are [out, in] (y = x W^T + b), so both GEMM
 *     operands are contiguous along the reduction axis.
 *   - Weight / bias / context dtype is cfg->dtype (WAN_BF16 or WAN_F32).
 *     The residual stream x, the modulation, the timestep, the latent and the
 *     step output are always float32.  The per-block modulation bias is float32.
 *   - Every pointer named "device" is device memory owned by the caller; the
 *     library never allocates or frees memory.  Temporaries live in the
 *     caller's workspace (ws, ws_bytes), sized by wan_workspace_bytes(); the
 *     one exception, wan_dit_block_fwd_noalloc, keeps them in a static device
 *     array of the library.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and the call returns without waiting.  Calls are stateless;
 *     concurrent calls need distinct workspaces and outputs.
 *   - Errors: every argument is validated on the host before anything is
 *     enqueued, so a call that returns an error has enqueued nothing.  The
 *     one exception is WAN_ERR_HIP, returned when a kernel launch fails
 *     (hipGetLastError); kernels enqueued before the failing one may run.
 */
#ifndef WAN_DIT_H
#define WAN_DIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define WAN_OK             0
#define WAN_ERR_NULL      -1  /* a required pointer is NULL                         */
#define WAN_ERR_SHAPE     -2  /* sizes inconsistent: odd H/8 or W/8, dim != heads*head_dim,
                                 unsupported head_dim, empty sequence, ...          */
#define WAN_ERR_DTYPE     -3  /* cfg->dtype is neither WAN_F32 nor WAN_BF16, or is
                                 WAN_F32 for an FP8 entry point or with cfg->attn8  */
#define WAN_ERR_WORKSPACE -4  /* ws_bytes smaller than wan_workspace_bytes()         */
#define WAN_ERR_CONFIG    -5  /* I2V pointers inconsistent with in_ch / img_len, or
                                 cfg->attn8 neither 0 nor 1                         */
#define WAN_ERR_HIP       -6  /* a HIP launch failed                                 */

/* operand dtypes */
#define WAN_F32  0
#define WAN_BF16 1

/* Model configuration ([Note] 配置表: 1.3B = 1536/8960/12 heads/30 layers,
 * 14B = 5120/13824/40/40; latent in/out 16 channels; frequency dim 256).   */
typedef struct {
    int dim;        /* model width d                                         */
    int heads;      /* attention heads H                                     */
    int head_dim;   /* d / H. WAN_BF16: 128.  WAN_F32: 64 or 128              */
    int ffn;        /* FFN width F                                           */
    int n_blocks;   /* blocks in a step                                      */
    int in_ch;      /* latent channels fed to patchify: 16 (T2V) or 36 (I2V) */
    int out_ch;     /* predicted latent channels: 16                         */
    int freq_dim;   /* timestep embedding width: 256                          */
    int text_len;   /* text tokens Lc (512)                                   */
    int img_len;    /* image tokens Li: 0 (T2V) or 257 (I2V)                  */
    int img_feat;   /* CLIP feature width (1280), I2V only                    */
    float eps;      /* LayerNorm epsilon (1e-6)                               */
    int dtype;      /* WAN_F32 or WAN_BF16                                    */
    int attn8;      /* 1: every block's self-attention in 8 bits (Int8 Q K^T, E4M3 P V,
                       the 8-bit attention below) with bf16 or FP8 Linear layers, the
                       cross-attention unchanged ([Note] Infra / 推理优化: 8-bit
                       FlashAttention); WAN_BF16 only (else WAN_ERR_DTYPE).  0: bf16
                       self-attention.  Other values: WAN_ERR_CONFIG               */
} wan_cfg_t;

/* Shared timestep MLP ([Note] Diffusion Transformer; [News] 核心创新二):
 * w1 [d, freq_dim], b1 [d], w2 [6d, d], b2 [6d]; dtype cfg->dtype; device.   */
typedef struct {
    const void *w1, *b1, *w2, *b2;
} wan_tmlp_weights_t;

/* One block.  All device, dtype cfg->dtype unless noted.
 *   sa_wqkv [3d, d] (rows: q | k | v), sa_bqkv [3d], sa_wo [d, d], sa_bo [d]
 *   ca_wq [d, d], ca_bq [d], ca_wkv [2d, d] (rows: k | v), ca_bkv [2d]
 *   ca_wkv_img [2d, d], ca_bkv_img [2d]  (image tokens; NULL unless img_len)
 *   ca_wo [d, d], ca_bo [d]
 *   ffn_w1 [F, d], ffn_b1 [F], ffn_w2 [d, F], ffn_b2 [d]
 *   mod_bias [6d] float32: this block's own modulation bias, added to the
 *            shared MLP output (order shift1, scale1, gate1, shift2, scale2, gate2). */
typedef struct {
    const void *sa_wqkv, *sa_bqkv, *sa_wo, *sa_bo;
    const void *ca_wq, *ca_bq, *ca_wkv, *ca_bkv, *ca_wkv_img, *ca_bkv_img, *ca_wo, *ca_bo;
    const void *ffn_w1, *ffn_b1, *ffn_w2, *ffn_b2;
    const float *mod_bias;
} wan_block_weights_t;

/* Whole model.  patch_w [d, in_ch*4] is the Conv3d weight [d, in_ch, 1, 2, 2]
 * flattened (feature k = c*4 + a*2 + b); for I2V the columns of channels
 * 16..35 carry the zero-initialised extra projection ([News] 核心创新四).
 * head_w [out_ch*4, d], head_b [out_ch*4].  img_w1 [d, img_feat], img_w2/w3
 * [d, d] (+ biases [d]): the 3-layer image MLP, NULL unless img_len.
 * `blocks` is a HOST array of n_blocks descriptors (device pointers inside). */
typedef struct {
    const void *patch_w, *patch_b;
    wan_tmlp_weights_t tmlp;
    const wan_block_weights_t *blocks;
    const void *head_w, *head_b;
    const void *img_w1, *img_b1, *img_w2, *img_b2, *img_w3, *img_b3;
} wan_model_weights_t;

/* Workspace bytes needed by any entry point for batch B and a latent of
 * lat_f x H8 x W8 (H8 = H/8, W8 = W/8).  Returns 0 for an invalid cfg/shape.
 * Shapes every entry point accepts (WAN_ERR_SHAPE otherwise): B <= 8,
 * B * L <= 2^30 tokens; for bf16 also L * max(ffn, 2d) * 2 bytes (one sample's
 * largest GEMM operand) and d * B * round_up(L, 64) * 2 bytes (the
 * self-attention's V^T) below 2^31.  A GEMM operand of several samples that
 * reaches 2 GiB runs as launches over groups of samples. */
size_t wan_workspace_bytes(const wan_cfg_t *cfg, int B, int lat_f, int H8, int W8);

/* Human-readable text of a status code (static storage). */
const char *wan_status_str(int status);

/* Shared AdaLN MLP ([Note] Diffusion Transformer; [News] 核心创新二;
 * frequency dim 256 from [Note] 配置表):
 *   e = [cos(t w_k) | sin(t w_k)], w_k = 10000^(-k/(freq_dim/2)), t raw;
 *   mod = W2 SiLU(W1 e + b1) + b2.
 * t [B] float32 device; mod [B, 6d] float32 device (written). */
int wan_tmlp_fwd(const wan_cfg_t *cfg, const float *t, int B, const wan_tmlp_weights_t *w,
                 float *mod, void *ws, size_t ws_bytes, void *stream);

/* One DiT block, in place on the residual stream ([Note] Diffusion
 * Transformer: full spatio-temporal self-attention; text cross-attention in
 * every block; shared AdaLN with per-block biases):
 *   x += gate1 * SA(LN(x)(1+scale1)+shift1)
 *   x += CA(LN(x), ctx [, img_ctx])          (ungated, unmodulated)
 *   x += gate2 * FFN(LN(x)(1+scale2)+shift2)
 * x [B, L, d] float32 device (read and written), L = lat_f*Hp*Wp tokens in
 * (frame, row, column) order; mod [B, 6d] float32 device (wan_tmlp_fwd);
 * ctx [B, text_len, d] device; img_ctx [B, img_len, d] device when
 * cfg->img_len > 0 (the output of the image MLP), else NULL. */
int wan_dit_block_fwd(const wan_cfg_t *cfg, float *x, int B, int lat_f, int Hp, int Wp,
                      const float *mod, const wan_block_weights_t *w, const void *ctx,
                      const void *img_ctx, void *ws, size_t ws_bytes, void *stream);

/* ---- the block without a caller workspace --------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the block
 * of wan_dit_block_fwd with its temporaries in a static device array of
 * WAN_NOALLOC_SCRATCH_BYTES owned by the library (one per GPU, held until
 * the process ends) instead of a caller workspace.  The caller still passes
 * every input and the residual stream x.  It allocates nothing and calls no
 * allocating routine.  Results equal wan_dit_block_fwd's bit for bit (same
 * kernels, same order).
 *   - Sizes whose temporaries exceed WAN_NOALLOC_SCRATCH_BYTES return
 *     WAN_ERR_WORKSPACE before anything is enqueued
 *     (wan_dit_block_noalloc_bytes gives the need; at the 1.3B width about
 *     36 KB per token, so up to ~7000 tokens per call).
 *   - All calls on one GPU share the array and it keeps the last call's
 *     contents (every byte a call reads it has written first): calls that
 *     overlap on one GPU (other streams, other host threads) race and must
 *     be serialised by the caller.
 *   - WAN_ERR_HIP when the array's device address cannot be looked up.
 * Other arguments and errors as wan_dit_block_fwd. */
#define WAN_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

/* Scratch bytes one wan_dit_block_fwd_noalloc call needs (0 for an invalid
 * cfg / shape); the call succeeds when this is at most
 * WAN_NOALLOC_SCRATCH_BYTES. */
size_t wan_dit_block_noalloc_bytes(const wan_cfg_t *cfg, int B, int lat_f, int Hp, int Wp);

int wan_dit_block_fwd_noalloc(const wan_cfg_t *cfg, float *x, int B, int lat_f, int Hp, int Wp,
                              const float *mod, const wan_block_weights_t *w, const void *ctx,
                              const void *img_ctx, void *stream);

/* One denoising step ([Note] Diffusion Transformer: patchify with a (1,2,2)
 * 3D convolution, N blocks, unpatchify; [Note] I2V 架构扩展 for the I2V
 * inputs): latent [B, in_ch, lat_f, H8, W8] float32 device (for I2V: noise
 * 16 | condition 16 | mask 4 channels); t [B] float32 device; ctx
 * [B, text_len, d] device; clip_feat [B, img_len, img_feat] device or NULL
 * (T2V); out [B, out_ch, lat_f, H8, W8] float32 device: the predicted
 * flow-matching velocity ([Note] 训练方法). */
int wan_dit_step_fwd(const wan_cfg_t *cfg, const float *latent, const float *t, int B,
                     int lat_f, int H8, int W8, const void *ctx, const void *clip_feat,
                     const wan_model_weights_t *w, float *out, void *ws, size_t ws_bytes,
                     void *stream);

/* Host helper ([News] 核心创新四; [Note] I2V 架构扩展): binary frame mask of
 * the video (n_frames = 1+T bytes, 1 = keep, 0 = generate) -> 4 mask
 * channels [4, lat_f, H8, W8] float32 HOST buffer.  Frame 0 is repeated four
 * times, then every 4 consecutive frames form one latent frame (the VAE's
 * temporal stride) and the position within the group is the channel.
 * Requires n_frames = 4*(lat_f-1)+1.  Touches no device. */
int wan_i2v_mask(const uint8_t *frame_mask, int n_frames, int lat_f, int H8, int W8, float *out);

/* ---- sampler around the step -------------------------------------------- */
/* [Note] 训练方法: the flow x_tau = tau x1 + (1 - tau) x0 runs from noise x0
 * (tau = 0) to data x1 (tau = 1) with velocity x1 - x0, which the step
 * predicts; [Note] Infra (推理优化): about 50 sampling steps, work that does
 * not change between steps is reused; [Guide] 工作原理: step count and
 * guidance scale.  Integration: explicit Euler on tau_k = k / n_steps with the
 * model's timestep input 1000 tau_k; guidance v = v_u + s (v_c - v_u). */

/* Bytes of the cross-attention key / value cache for B samples: per block the
 * text keys [B*text_len, d] and V^T [d, B*round_up(text_len, 64)] (for I2V
 * also the image pair), in cfg->dtype, each region 256-byte aligned.  The
 * float32 path stores keys and values side by side ([B*len, 2d], no V^T).
 * 0 for an invalid configuration or B outside 1..8. */
size_t wan_kv_cache_bytes(const wan_cfg_t *cfg, int B);

/* Fill the cache: for every block, the keys and V^T of the text context
 * ctx [B, text_len, d] (device) and, for I2V, of the image context (the image
 * MLP of clip_feat [B, img_len, img_feat], device; NULL for T2V).  These
 * depend only on the contexts and the weights, so a sampler fills the cache
 * once and every step reads it.  cache (device, cache_bytes >=
 * wan_kv_cache_bytes) is written; ws (device) holds the image MLP's
 * temporaries: at least 3 regions of round_up(B*img_len*d*elem, 256) bytes
 * for I2V (any step workspace of the same B is large enough); unused (may be
 * NULL) for T2V.  Errors: WAN_ERR_WORKSPACE for a short cache or ws,
 * WAN_ERR_CONFIG when clip_feat does not match cfg->img_len. */
int wan_kv_cache_fwd(const wan_cfg_t *cfg, int B, const void *ctx, const void *clip_feat,
                     const wan_model_weights_t *w, void *cache, size_t cache_bytes, void *ws,
                     size_t ws_bytes, void *stream);

/* wan_dit_step_fwd with the cross-attention keys / values read from a cache
 * that wan_kv_cache_fwd filled for the same cfg, B and weights (the image
 * MLP weights are not read).  Same latent, t, out and workspace contract as
 * wan_dit_step_fwd; its output equals wan_dit_step_fwd's bit for bit. */
int wan_dit_step_cached_fwd(const wan_cfg_t *cfg, const float *latent, const float *t, int B,
                            int lat_f, int H8, int W8, const void *kv_cache, size_t cache_bytes,
                            const wan_model_weights_t *w, float *out, void *ws, size_t ws_bytes,
                            void *stream);

/* One Euler step on the moving channels: latent [B, in_ch, lat_f, H8, W8]
 * float32 device, channels 0..out_ch-1 updated in place, the rest (I2V
 * condition and mask) untouched; vel [B, out_ch, lat_f, H8, W8] float32
 * device.  guided == 0: latent[b] += dt * vel[b] for every sample.
 * guided != 0: B must be 2 (sample 0 conditional, 1 unconditional, same
 * latent); both samples become latent[0] + dt * (vel[1] + scale (vel[0] - vel[1])).
 * WAN_ERR_SHAPE for in_ch < out_ch, guided with B != 2, or non-finite dt / scale. */
int wan_euler_fwd(float *latent, const float *vel, int B, int in_ch, int out_ch, int lat_f, int H8,
                  int W8, float dt, int guided, float scale, void *stream);

/* Workspace of wan_sample_fwd: the step workspace plus the timestep [B] and
 * velocity [B, out_ch, lat_f, H8, W8] buffers.  0 on invalid arguments. */
size_t wan_sample_workspace_bytes(const wan_cfg_t *cfg, int B, int lat_f, int H8, int W8);

/* The whole sampler: n_steps evaluations of the step (cross-attention K/V
 * from kv_cache, filled by wan_kv_cache_fwd for the same B), each followed by
 * wan_euler_fwd with dt = 1/n_steps, timestep input 1000 k / n_steps for
 * step k.  latent [B, in_ch, lat_f, H8, W8] float32 device: on entry the
 * noise (tau = 0) in channels 0..out_ch-1 (+ I2V condition and mask), on
 * return the sample at tau = 1.  guided / scale as in wan_euler_fwd (the
 * pair's two latents must be equal on entry). */
int wan_sample_fwd(const wan_cfg_t *cfg, float *latent, int B, int lat_f, int H8, int W8,
                   int n_steps, int guided, float scale, const void *kv_cache, size_t cache_bytes,
                   const wan_model_weights_t *w, void *ws, size_t ws_bytes, void *stream);

/* ---- component entry points (the kernels the block is made of) ---------- */

/* Multi-head attention O = softmax(Q K^T / sqrt(hd)) V per (batch, head)
 * ([Note] Diffusion Transformer).  bf16 only, hd = 128, device pointers:
 *   q  [B, Lq, *] row stride ldq elements, head h at column h*128; with
 *      q_scaled = 1 the caller has multiplied q by log2(e)/sqrt(128) (as the
 *      block's query projections do), and the result is the same attention
 *      of q / (log2(e)/sqrt(128)); q_scaled = 0 for a plain q
 *   k  [B, Lk, *] row stride ldk, head h at column h*128
 *   vt [H*128, *] row stride ldv: V transposed; batch b's key j sits at
 *      column b*vt_bstride + j.  ldv and vt_bstride are multiples of 8,
 *      vt_bstride >= round_up(Lk, 64), every row holds at least B*vt_bstride
 *      columns, and columns Lk .. round_up(Lk, 64)-1 of each batch segment
 *      hold zeros (whole 64-key tiles are read; finite padding times a zero
 *      probability must stay zero)
 *   o  [B, Lq, H*128] bf16, row stride ldo.
 * No mask.  Returns WAN_ERR_SHAPE for unsupported strides or sizes. */
int wan_attention_fwd(const void *q, int ldq, const void *k, int ldk, const void *vt, int ldv, int vt_bstride,
                      void *o, int ldo, int B, int H, int Lq, int Lk, int q_scaled, void *stream);

/* ---- 8-bit attention ([Note] Infra / 推理优化: 8-bit FlashAttention, Int8 for
 * S = QK^T, FP8 for O = PV, FP32 accumulation across key blocks) -----------
 * Quantised copies, hd = 128, all device:
 *   q8  [B*Lq, H*128] Int8 codes, qs [B*Lq, H] float32: q per token and head
 *   k8  [B*Lk, H*128] Int8 codes, ks [B, H, ceil(Lk/64)] float32: k per block
 *       of 64 keys and head (block b = keys 64b .. 64b+63, the last ragged)
 *   v8t [H*128, B*Lkp] E4M3 bytes, Lkp = round_up(Lk, 64), batch b at column
 *       b*Lkp (columns Lk .. Lkp-1 of a segment are zero), vs [B, H*128]
 *       float32: V per channel (one head feature over the Lk keys)
 * Int8: inv = 127 / amax (float32 division), code = round-half-even(
 * clamp(x * inv, +-127)), scale = amax / 127.  E4M3: the FP8 GEMM's rule
 * with 448.  An all-zero group gets scale 1.  The attention scores with the
 * integer dot products times qs ks, scales its probabilities so the row max
 * maps to at most 448 (2^7 where the running max is set), rounds them to
 * E4M3, and divides sum_j P_j v8_j vs by sum_j P_j (float32 accumulation).
 * Limits: Lk*H*128 and H*128*B*Lkp below 2^31 (WAN_ERR_SHAPE beyond). */

/* Workspace bytes of wan_attention_8bit_fwd (the six copies, each 256-byte
 * aligned); 0 for invalid or too large sizes. */
size_t wan_attention_8bit_workspace_bytes(int B, int H, int Lq, int Lk);

/* The quantisers: q, k, vt as in wan_attention_fwd (bf16; vt's padding
 * columns Lk .. round_up(Lk, 64)-1 must be readable, their values are
 * ignored) -> the six copies above, caller-allocated. */
int wan_attention_8bit_quantize(const void *q, int ldq, const void *k, int ldk, const void *vt, int ldv,
                                int vt_bstride, int B, int H, int Lq, int Lk, void *q8, float *qs, void *k8,
                                float *ks, void *v8t, float *vs, void *stream);

/* The 8-bit attention on quantised copies (layouts above).  q_scaled as in
 * wan_attention_fwd: 1 when the q that was quantised had been multiplied by
 * log2(e)/sqrt(128).  o [B, Lq, H*128] bf16, row stride ldo (>= H*128, % 4). */
int wan_attention_8bit_q_fwd(const void *q8, const float *qs, const void *k8, const float *ks, const void *v8t,
                             const float *vs, void *o, int ldo, int B, int H, int Lq, int Lk, int q_scaled,
                             void *stream);

/* Both: arguments as wan_attention_fwd plus ws (device, at least
 * wan_attention_8bit_workspace_bytes, else WAN_ERR_WORKSPACE) holding the
 * copies.  The result approximates wan_attention_fwd's within the 8-bit
 * rounding (a few percent of |O|). */
int wan_attention_8bit_fwd(const void *q, int ldq, const void *k, int ldk, const void *vt, int ldv,
                           int vt_bstride, void *o, int ldo, int B, int H, int Lq, int Lk, int q_scaled,
                           void *ws, size_t ws_bytes, void *stream);

/* Measurement hook (for timing the dominant kernel of [Note] Infra's workload
 * split, the full self-attention, inside the block's own launch sequence):
 * start / stop are hipEvent_t handles the library records on the call's
 * stream immediately before and after every bf16 or 8-bit self-attention of
 * the block, step and sampler calls this host thread makes next (a call with
 * several blocks records them for each block; the last pair stays).  Both
 * NULL: no recording (the default).  Per host thread; the caller owns the
 * events.  Errors: WAN_ERR_NULL when only one of the two is NULL.  A failed
 * record surfaces as WAN_ERR_HIP from the block call. */
int wan_set_attention_events(void *start, void *stop);

/* The block's normalisation before a branch ([Note] Diffusion Transformer:
 * shared AdaLN; LayerNorm without affine, eps inside the square root):
 *   h = (x - mean) / sqrt(var + eps) * (1 + scale) + shift  over the last axis
 *   (biased variance), rounded to bf16.
 * x [B, L, d] float32 device; mod [B, 6d] float32 device: a block's combined
 * modulation (the shared MLP output plus the block's own bias; order shift1,
 * scale1, gate1, shift2, scale2, gate2), or NULL for the plain LayerNorm of
 * the cross-attention; branch 0 takes (shift1, scale1), branch 1 (shift2,
 * scale2); h [B*L, d] bf16 device.  Errors: WAN_ERR_NULL for a NULL x / h,
 * WAN_ERR_SHAPE for B outside 1..8, L or d <= 0, B*L > 2^30 or eps not
 * positive and finite, WAN_ERR_CONFIG for another branch with mod given. */
int wan_ln_modulate_fwd(const float *x, int B, int L, int d, const float *mod, int branch, float eps,
                        void *h, void *stream);

/* One Linear layer of the block ([Note] Diffusion Transformer: the attention
 * projections; [Note] 配置表: the FFN of width ffn with GELU):
 *   y = x W^T + b for a bf16 x [M, K], W [N, K], b [N] or NULL (all device,
 *   rows contiguous), K % 64 == 0, M, N > 0.
 * mode 0: y bf16 [M, N];  mode 1: y float32 [M, N];  mode 2: y bf16 =
 * GELU_tanh(.) (tanh form).  float32 accumulation.  Operands of 2 GiB or
 * more run as launches over row / column slices.  Errors: WAN_ERR_NULL for
 * a NULL x / W / y, WAN_ERR_SHAPE for the sizes above, WAN_ERR_CONFIG for
 * another mode. */
int wan_linear_fwd(const void *x, const void *w, const void *b, void *y, int M, int N, int K,
                   int mode, void *stream);

/* ---- FP8 GEMM ------------------------------------------------------------- */
/* [Note] Infra (推理优化): FP8 GEMM with per-tensor weight scales and
 * per-token activation scales.  Format: OCP E4M3 (one byte, largest finite
 * 448, round to nearest even).  A scale maps the largest magnitude to 448:
 * inv = 448 / amax (float32, correctly rounded), code = E4M3(clamp(x * inv,
 * +-448)), scale = amax / 448 (so x ~= code * scale); an all-zero row or
 * tensor gets scale 1. */

/* Per-token quantisation: x bf16 [M, K] row stride ldx (device) -> q E4M3
 * [M, K] row stride ldq bytes (device), scale float32 [M] (device).
 * K, ldx and ldq multiples of 8 (16-byte / 8-byte aligned rows). */
int wan_quantize_rows_fp8(const void *x, int M, int K, int ldx, void *q, int ldq, float *scale,
                          void *stream);

/* Per-tensor quantisation of n bf16 values (n % 8 == 0, device) -> q E4M3 [n]
 * (device) and one float32 scale (device).  ws: at least 4 bytes of device
 * scratch (the running maximum). */
int wan_quantize_tensor_fp8(const void *w, long n, void *q, float *scale, void *ws, size_t ws_bytes,
                            void *stream);

/* y = (xq wq^T) * x_scale[m] * w_scale[0] + b: xq E4M3 [M, K], wq E4M3 [N, K]
 * (rows contiguous, K % 64 == 0), x_scale float32 [M], w_scale float32 [1],
 * b bf16 [N] or NULL (all device).  mode 0: y bf16 [M, N]; 1: y float32;
 * 2: y bf16 = GELU_tanh(.).  float32 accumulation. */
int wan_linear_fp8_fwd(const void *xq, const float *x_scale, const void *wq, const float *w_scale,
                       const void *b, void *y, int M, int N, int K, int mode, void *stream);

/* ---- FP8 block -------------------------------------------------------------- */
/* The block of wan_dit_block_fwd with its six Linear layers -- QKV, self-
 * attention out, cross-attention query, cross-attention out, FFN up, FFN
 * down -- on E4M3 operands ([Note] Infra (推理优化): FP8 GEMM; the block of
 * [Note] Diffusion Transformer): each weight quantised per tensor (Wqkv as one
 * [3d, d] tensor), each bf16 activation quantised per token right before the
 * GEMM that reads it, float32 accumulation, dequantisation and bias in the
 * epilogue.  LayerNorm, modulation, attention, GELU, gates and the residual
 * stream are those of wan_dit_block_fwd; the text / image keys and values are
 * projected in bf16.  bf16 configurations only (WAN_ERR_DTYPE otherwise). */

/* Bytes of one block's packed FP8 weights; 0 for an invalid or float32 cfg. */
size_t wan_block_fp8_bytes(const wan_cfg_t *cfg);

/* Quantise the six Linear weights of block w (bf16, device) into qbuf (device,
 * 256-byte aligned, at least wan_block_fp8_bytes; the layout is private to the
 * library).  Done once per set of weights; every wan_dit_block_fp8_fwd call
 * with those weights reads the result. */
int wan_quantize_block_fp8(const wan_cfg_t *cfg, const wan_block_weights_t *w, void *qbuf,
                           size_t qbuf_bytes, void *stream);

/* Workspace bytes of wan_dit_block_fp8_fwd (0 for an invalid cfg / shape). */
size_t wan_block_fp8_workspace_bytes(const wan_cfg_t *cfg, int B, int lat_f, int Hp, int Wp);

/* wan_dit_block_fwd with FP8 Linear layers.  Arguments as there, plus qbuf
 * written by wan_quantize_block_fp8 from the same w.  From w only the biases,
 * mod_bias and the text / image K/V weights are read: the six quantised weight
 * pointers may be NULL.  L * max(d, ffn) < 2^31 (one sample's FP8 operands;
 * larger batches are split into launches over samples). */
int wan_dit_block_fp8_fwd(const wan_cfg_t *cfg, float *x, int B, int lat_f, int Hp, int Wp,
                          const float *mod, const wan_block_weights_t *w, const void *qbuf,
                          const void *ctx, const void *img_ctx, void *ws, size_t ws_bytes,
                          void *stream);

/* ---- FP8 step and sampler -------------------------------------------------- */
/* The step and the sampler of the bf16 model with every block in FP8 as in
 * wan_dit_block_fp8_fwd (patchify, t-MLP, image MLP, cross-attention K/V,
 * attention and head unchanged).  bf16 configurations only. */

/* Bytes of a model's packed FP8 block weights: n_blocks regions of
 * wan_block_fp8_bytes each (0 for an invalid or float32 cfg). */
size_t wan_model_fp8_bytes(const wan_cfg_t *cfg);

/* Quantise every block of w (bf16, device) into qbuf (device, 256-byte aligned,
 * at least wan_model_fp8_bytes; block i at i * wan_block_fp8_bytes). */
int wan_quantize_model_fp8(const wan_cfg_t *cfg, const wan_model_weights_t *w, void *qbuf,
                           size_t qbuf_bytes, void *stream);

/* Workspace of wan_dit_step_fp8_fwd (sampler = 0) or wan_sample_fp8_fwd
 * (sampler = 1); 0 for an invalid cfg / shape. */
size_t wan_fp8_workspace_bytes(const wan_cfg_t *cfg, int B, int lat_f, int H8, int W8, int sampler);

/* wan_dit_step_fwd with FP8 blocks: arguments as there, plus qbuf from
 * wan_quantize_model_fp8 for the same w (the blocks' six quantised weight
 * pointers are not read and may be NULL).  L * max(d, ffn) < 2^31 (one
 * sample's FP8 operands; larger batches are split into launches over samples). */
int wan_dit_step_fp8_fwd(const wan_cfg_t *cfg, const float *latent, const float *t, int B,
                         int lat_f, int H8, int W8, const void *ctx, const void *clip_feat,
                         const wan_model_weights_t *w, const void *qbuf, float *out, void *ws,
                         size_t ws_bytes, void *stream);

/* wan_sample_fwd with FP8 blocks (cross-attention K/V from the bf16 cache of
 * wan_kv_cache_fwd): arguments as there, plus qbuf as above. */
int wan_sample_fp8_fwd(const wan_cfg_t *cfg, float *latent, int B, int lat_f, int H8, int W8,
                       int n_steps, int guided, float scale, const void *kv_cache, size_t cache_bytes,
                       const wan_model_weights_t *w, const void *qbuf, void *ws, size_t ws_bytes,
                       void *stream);

#ifdef __cplusplus
}
#endif
#endif /* WAN_DIT_H */
