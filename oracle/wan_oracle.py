"""CPU oracle of the Wan2.1 DiT denoising step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP library and
its Python binding) never calls it and shares no code with it.

What it is: a plain, slow, obviously correct numpy implementation in float64
of what one denoising step computes, written from the pages' description.
Every function names the passage it follows.  Page tags used below:

  [Note]  "Wan: Open and Advanced Large-Scale Video Generative Models (Wan 2.1)"
          (AI Research 技术调研 note).  Sections: 模型架构 / Wan-VAE,
          模型架构 / Diffusion Transformer, 配置表（来自 HF model card）,
          I2V 架构扩展, 训练方法, 关键消融.
  [News]  "超越Sora！阿里正式完全开源最新、最强大的视频生成模型 Wan2.1"
          (163.com).  Sections: 核心创新一 (3D VAE, feature cache),
          核心创新二 (视频扩散 DiT), 核心创新四 (Image-to-Video).
  [Guide] "Wan 2.1 AI：下一代开源视频生成技术的突破性实践" (cloud.baidu.com).
          Section 工作原理 (the sampling knobs: number of inference steps,
          guidance scale).

Where the pages leave a step open the plainest reading is taken; every such
reading is listed in the module-level ``READINGS`` table and repeated where it
is used.  Inputs arrive as float32 arrays (bf16-representable for bf16
workloads) and are upcast to float64; nothing is rounded in between.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, library routines, brute force, invariants).  The numeric value
of a block or step with random weights has no worked example on the pages;
it is pinned only through those parts.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

F64 = np.float64

READINGS = {
    "R1 t-MLP shape": "Linear(256->d), SiLU, Linear(d->6d); one MLP shared by all blocks "
                      "[Note, Diffusion Transformer; News, 核心创新二]",
    "R2 sinusoid": "w_k = 10000^(-k/128), k=0..127; e = [cos(t w) | sin(t w)] on raw t "
                   "(the pages give only the width 256 [Note, 配置表])",
    "R3 modulation order": "[shift1, scale1, gate1, shift2, scale2, gate2]; block i uses m + beta_i",
    "R4 biases": "every Linear has a bias",
    "R5 cross-attention": "pre-LayerNorm without affine and without modulation; ungated residual",
    "R6 attention": "softmax(q k^T / sqrt(hd)) v; no mask, no positional term, no QK-norm",
    "R7 GELU": "tanh approximation (FFN and image MLP)",
    "R8 head": "plain Linear d -> 16*1*2*2, no final norm or modulation",
    "R9 patch order": "token n = (f*Hp + i)*Wp + j; feature k = c*4 + a*2 + b; "
                      "value latent[c, f, 2i+a, 2j+b] (Conv3d weight order)",
    "R10 I2V mask": "frame mask of the video (1+T frames) -> repeat frame 0 four times -> "
                    "[1+T/4, 4] -> 4 channels x (1+T/4) frames, broadcast over H/8 x W/8",
    "R11 image MLP": "Linear(1280->d), GELU, Linear(d->d), GELU, Linear(d->d)",
    "R12 decoupled CA": "two softmaxes (text / image), separate K,V weights, shared Q and "
                        "out-projection, outputs summed with weight 1",
    "R13 LayerNorm": "biased variance over d, eps inside the sqrt, no affine",
    "R19 sampler time": "flow time tau runs from 0 (noise x0) to 1 (data x1), x_tau = tau x1 + "
                        "(1 - tau) x0 [Note, 训练方法]; explicit Euler on a uniform grid tau_k = k/N "
                        "(N about 50 [Note, Infra / 推理优化]); the model's timestep input is "
                        "1000 tau (the range of R2)",
    "R20 guidance": "v = v_u + s (v_c - v_u) with s the guidance scale [Guide, 工作原理]; in a "
                    "two-sample guidance batch sample 0 is conditional, sample 1 unconditional, "
                    "and both carry the same latent",
    "R21 I2V sampling": "only the 16 noise channels move; the condition latent and the mask "
                        "channels of the 36-channel input stay as given",
    "R22 FP8 GEMM": "[Note, Infra / 推理优化]: per-tensor weight scale, per-token activation "
                    "scale; format OCP E4M3 (largest finite 448, round to nearest even); "
                    "scale = amax / 448 so the largest magnitude maps to 448; the code is "
                    "decided in float32 as the kernel does: inv = 448 / amax (float32 "
                    "division), v = x * inv (float32), clamp to +-448, round to E4M3; an "
                    "all-zero row or tensor gets scale 1; y = (xq wq^T) sx sw + b",
    "R23 FP8 activations": "the input of an FP8 GEMM is the bf16 activation a bf16 model holds "
                           "(the pages run the model in bf16 and quantise for the GEMM); it is "
                           "rounded to bf16 (nearest even) before its per-token quantisation, so "
                           "the E4M3 code is decided from a bf16 value on both sides",
    "R24 FP8 layers": "the FP8 block runs its six Linear layers on the token stream in FP8 (QKV "
                      "quantised as one [3d, d] tensor, SA out, CA query, CA out, FFN up, FFN "
                      "down); text / image K/V, LayerNorm, attention, GELU and the residual "
                      "stay exact",
    "R25 8-bit attention": "[Note, Infra / 推理优化: 8-bit FlashAttention, Int8 for S = QK^T, FP8 "
                           "for O = PV, FP32 accumulation across key blocks]: per (batch, head) "
                           "q is quantised per token (its hd features) and k per block of 64 keys "
                           "(block b = keys 64b .. 64b+63, the last block ragged) to symmetric "
                           "Int8: inv = 127 / amax (float32 division), code = round-half-even of "
                           "clamp(x * inv (float32), +-127), scale = amax / 127, an all-zero group "
                           "scale 1; v is quantised per channel (one feature over the Lk keys) to "
                           "E4M3 by R22's rule; S = (q8 . k8) sq sk (exact integer dot product); "
                           "the probabilities are scaled so that the row max maps to 2^7 and "
                           "rounded to E4M3 (nearest even); O = sv * (sum_j P8_j v8_j) / sum_j "
                           "P8_j: the normaliser adds the rounded probabilities, so O is a convex "
                           "combination of the dequantised values; inputs are the bf16 q, k, v "
                           "the block holds",
    "R26 8-bit attention in the block": "only the self-attention runs in 8 bits (R25), on the bf16-"
                                        "rounded q, k, v of the block's projections (bf16 or FP8 "
                                        "Linear layers); the cross-attention to the short text / "
                                        "image contexts stays exact",
}


def _f(a) -> np.ndarray:
    return np.asarray(a, dtype=F64)


# ---------------------------------------------------------------------------
# shapes  -- [Note, 模型架构 (Wan-VAE: latent (1+T/4) x H/8 x W/8, 16 ch) and
#            Diffusion Transformer: (1,2,2) patchify, L = (1+T/4) * H/16 * W/16]

def latent_shape(frames: int, height: int, width: int):
    """Video of ``frames`` = 1+T frames at H x W -> latent [16, 1+T/4, H/8, W/8]."""
    T = frames - 1
    if T % 4 or height % 8 or width % 8:
        raise ValueError("video shape not compatible with the 4x8x8 compression")
    return (16, 1 + T // 4, height // 8, width // 8)


def seq_len(frames: int, height: int, width: int) -> int:
    """L = (1+T/4) * H/16 * W/16 for a video of 1+T frames at H x W."""
    T = frames - 1
    if T % 4 or height % 16 or width % 16:
        raise ValueError("video shape not compatible with 4x8x8 VAE + (1,2,2) patch")
    return (1 + T // 4) * (height // 16) * (width // 16)


# ---------------------------------------------------------------------------
# elementwise pieces

def silu(z):
    """SiLU(z) = z * sigmoid(z).  [Note, Diffusion Transformer: Linear+SiLU]"""
    z = _f(z)
    return z / (1.0 + np.exp(-z))


def gelu_tanh(u):
    """GELU, tanh form: 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3))).  (R7)"""
    u = _f(u)
    return 0.5 * u * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (u + 0.044715 * (u * u * u))))


def linear(x, w, b):
    """y = x W^T + b with W stored [out, in].  (R4)"""
    return _f(x) @ _f(w).T + _f(b)


def layer_norm(x, eps: float = 1e-6):
    """(x - mean) / sqrt(var + eps) over the last axis, biased variance, no affine (R13)."""
    x = _f(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def modulate(xhat, shift, scale):
    """AdaLN modulation x * (1 + scale) + shift.
    [Note, Diffusion Transformer: shared AdaLN predicts the modulation]"""
    return _f(xhat) * (1.0 + _f(scale)) + _f(shift)


# ---------------------------------------------------------------------------
# timestep embedding and the shared AdaLN MLP
# [Note, Diffusion Transformer; News, 核心创新二: one Linear+SiLU MLP on the time
#  embedding predicts six modulation parameters, shared by every block, each
#  block learning its own biases; Note, 配置表: frequency dimension 256]

def sinusoid(t, freq_dim: int = 256):
    """e(t) = [cos(t w_0..w_{h-1}) | sin(t w_0..w_{h-1})], w_k = 10000^(-k/h), h = freq_dim/2 (R2)."""
    t = _f(t).reshape(-1)
    half = freq_dim // 2
    k = np.arange(half, dtype=F64)
    w = np.exp(-math.log(10000.0) * k / half)
    arg = t[:, None] * w[None, :]
    return np.concatenate([np.cos(arg), np.sin(arg)], axis=1)


def tmlp(t, w1, b1, w2, b2, freq_dim: int = 256):
    """m = W2 SiLU(W1 e(t) + b1) + b2  -> [B, 6d]  (R1)."""
    e = sinusoid(t, freq_dim)
    return linear(silu(linear(e, w1, b1)), w2, b2)


def block_modulation(m, beta):
    """m_i = m + beta_i, split into the six [B, d] vectors (R3)."""
    mi = _f(m) + _f(beta)[None, :]
    d = mi.shape[1] // 6
    names = ("shift1", "scale1", "gate1", "shift2", "scale2", "gate2")
    return {n: mi[:, j * d:(j + 1) * d] for j, n in enumerate(names)}


# ---------------------------------------------------------------------------
# attention  (R6)  [Note, Diffusion Transformer: full spatio-temporal attention;
#                   text injected through cross-attention in every block]

def attention(q, k, v, chunk: int = 256):
    """softmax(q k^T / sqrt(hd)) v for one head.  q [Lq, hd], k/v [Lk, hd].
    The softmax is materialised one query chunk at a time (rows are
    independent), with the row maximum subtracted before exp."""
    q, k, v = _f(q), _f(k), _f(v)
    hd = q.shape[1]
    out = np.empty((q.shape[0], v.shape[1]), dtype=F64)
    scale = 1.0 / math.sqrt(hd)
    for s in range(0, q.shape[0], chunk):
        S = (q[s:s + chunk] @ k.T) * scale
        S -= S.max(axis=1, keepdims=True)
        P = np.exp(S)
        P /= P.sum(axis=1, keepdims=True)
        out[s:s + chunk] = P @ v
    return out


# Heads are independent, so a long run may attend to several heads at once:
# HEAD_THREADS > 1 hands the heads to a pool of that many threads (each head's
# arithmetic is unchanged; the BLAS inside each head then runs on one thread).
HEAD_THREADS = 1


def multihead(q, k, v, heads: int):
    """Split the feature axis into ``heads`` equal heads (head h = columns
    h*hd .. (h+1)*hd), attend per head, concatenate."""
    hd = q.shape[1] // heads
    one = lambda h: attention(q[:, h * hd:(h + 1) * hd], k[:, h * hd:(h + 1) * hd],
                              v[:, h * hd:(h + 1) * hd])
    if HEAD_THREADS <= 1 or heads == 1:
        return np.concatenate([one(h) for h in range(heads)], axis=1)
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(HEAD_THREADS) as ex:
        outs = list(ex.map(one, range(heads)))
    return np.concatenate(outs, axis=1)


def self_attention(hmod, wqkv, bqkv, wo, bo, heads: int, rows: Optional[np.ndarray] = None,
                   fp8: bool = False, attn8: bool = False):
    """Self-attention of one sample: qkv = h Wqkv^T + b (q | k | v blocks of d
    rows in Wqkv), o = MHA(q, k, v), y = o Wo^T + bo.  ``rows`` restricts the
    query side (and the returned rows) to a subset of tokens; keys and values
    always cover all tokens.  ``fp8``: both projections in FP8 (R22), the
    stored Wqkv quantised as one tensor.  ``attn8``: the attention in 8 bits
    on the bf16-rounded q, k, v (R25, R26)."""
    hmod = _f(hmod)
    d = hmod.shape[1]
    wqkv, bqkv = _f(wqkv), _f(bqkv)
    if fp8:
        qw, sw = quantize_tensor_fp8(wqkv)
        lin = lambda x, sl, b: linear_fp8_q(x, qw[sl], sw, b)
        lin_o = linear_fp8
    else:
        lin = lambda x, sl, b: linear(x, wqkv[sl], b)
        lin_o = linear
    k = lin(hmod, slice(d, 2 * d), bqkv[d:2 * d])
    v = lin(hmod, slice(2 * d, 3 * d), bqkv[2 * d:])
    hq = hmod if rows is None else hmod[rows]
    q = lin(hq, slice(0, d), bqkv[:d])
    if attn8:
        o = multihead_8bit(bf16_round(q), bf16_round(k), bf16_round(v), heads)
    else:
        o = multihead(q, k, v, heads)
    return lin_o(o, wo, bo)


def cross_attention(xq, ctx, wq, bq, wkv, bkv, wo, bo, heads: int, eps: float = 1e-6,
                    img=None, wkv_img=None, bkv_img=None, fp8: bool = False):
    """Cross-attention of one sample (R5, R12): q from LayerNorm(x) without
    modulation, keys/values from the text context; with ``img`` a second,
    separately normalised attention over the image tokens is added before the
    shared out-projection.  [News, 核心创新二; Note, I2V 架构扩展: decoupled
    cross-attention in the manner of IP-Adapter].  ``fp8``: the query and
    out-projections in FP8 (R22); the text / image keys and values stay exact."""
    d = ctx.shape[1]
    lin = linear_fp8 if fp8 else linear
    q = lin(layer_norm(xq, eps), wq, bq)
    wkv, bkv = _f(wkv), _f(bkv)
    kt = linear(ctx, wkv[:d], bkv[:d])
    vt = linear(ctx, wkv[d:], bkv[d:])
    o = multihead(q, kt, vt, heads)
    if img is not None:
        wkv_img, bkv_img = _f(wkv_img), _f(bkv_img)
        ki = linear(img, wkv_img[:d], bkv_img[:d])
        vi = linear(img, wkv_img[d:], bkv_img[d:])
        o = o + multihead(q, ki, vi, heads)
    return lin(o, wo, bo)


def ffn(hmod, w1, b1, w2, b2, fp8: bool = False):
    """z = GELU_tanh(h W1^T + b1) W2^T + b2.  [Note, 配置表: FFN dimension]
    ``fp8``: both projections in FP8 (R22)."""
    lin = linear_fp8 if fp8 else linear
    return lin(gelu_tanh(lin(hmod, w1, b1)), w2, b2)


# ---------------------------------------------------------------------------
# one DiT block

def block(x, m, wts: Dict[str, np.ndarray], ctx, heads: int, eps: float = 1e-6,
          img=None, rows: Optional[np.ndarray] = None, return_parts: bool = False,
          fp8: bool = False, attn8: bool = False):
    """One block for a batch.  x [B, L, d]; m [B, 6d] (shared t-MLP output);
    ctx [B, Lc, d]; img [B, Li, d] or None.

      x1 = x  + gate1 * SA(LN(x) (1+scale1) + shift1)
      x2 = x1 + CA(LN(x1), ctx [, img])
      x3 = x2 + gate2 * FFN(LN(x2) (1+scale2) + shift2)

    [News, 核心创新二 and Note, Diffusion Transformer: shared AdaLN, full
    self-attention, text cross-attention in every block; readings R3, R5.]
    With ``rows`` only those token rows of the output are computed (self-
    attention still reads all tokens' keys and values).  ``fp8``: the six
    Linear layers (QKV, SA out, CA query, CA out, FFN up, FFN down) in FP8
    with per-token activation and per-tensor weight scales (R22 - R24)
    [Note, Infra / 推理优化: FP8 GEMM].  ``attn8``: the self-attention in 8 bits
    (R25, R26) [Note, Infra / 推理优化: 8-bit FlashAttention]."""
    x = _f(x)
    mod = block_modulation(m, wts["mod_bias"])
    outs, parts = [], []
    for b in range(x.shape[0]):
        xb = x[b]
        h1 = modulate(layer_norm(xb, eps), mod["shift1"][b], mod["scale1"][b])
        sa = self_attention(h1, wts["sa_wqkv"], wts["sa_bqkv"], wts["sa_wo"], wts["sa_bo"],
                            heads, rows=rows, fp8=fp8, attn8=attn8)
        xr = xb if rows is None else xb[rows]
        x1 = xr + mod["gate1"][b] * sa
        ca = cross_attention(x1, _f(ctx[b]), wts["ca_wq"], wts["ca_bq"], wts["ca_wkv"],
                             wts["ca_bkv"], wts["ca_wo"], wts["ca_bo"], heads, eps,
                             img=None if img is None else _f(img[b]),
                             wkv_img=wts.get("ca_wkv_img"), bkv_img=wts.get("ca_bkv_img"),
                             fp8=fp8)
        x2 = x1 + ca
        h2 = modulate(layer_norm(x2, eps), mod["shift2"][b], mod["scale2"][b])
        z = ffn(h2, wts["ffn_w1"], wts["ffn_b1"], wts["ffn_w2"], wts["ffn_b2"], fp8=fp8)
        x3 = x2 + mod["gate2"][b] * z
        outs.append(x3)
        parts.append({"sa": sa, "ca": ca, "ffn": z})
    out = np.stack(outs)
    return (out, parts) if return_parts else out


# ---------------------------------------------------------------------------
# patchify / unpatchify  [Note, Diffusion Transformer: (1,2,2) 3D convolution;
#                         Note, 配置表: in/out latent dimension 16]  (R9)

def patch_gather(latent):
    """latent [C, F, H8, W8] -> P [L, 4C] with P[(f*Hp+i)*Wp+j, c*4+a*2+b] =
    latent[c, f, 2i+a, 2j+b]."""
    lat = _f(latent)
    C, F, H8, W8 = lat.shape
    Hp, Wp = H8 // 2, W8 // 2
    # [C, F, Hp, 2, Wp, 2] -> [F, Hp, Wp, C, 2, 2]
    r = lat.reshape(C, F, Hp, 2, Wp, 2).transpose(1, 2, 4, 0, 3, 5)
    return r.reshape(F * Hp * Wp, C * 4)


def patchify(latent, w, b):
    """Conv3d with kernel = stride = (1,2,2) as gather + matmul: x0 = P W^T + b.
    latent [B, C, F, H8, W8]; w [d, 4C] (Conv3d weight [d, C, 1, 2, 2] flattened)."""
    return np.stack([linear(patch_gather(latent[s]), w, b) for s in range(latent.shape[0])])


def unpatch_scatter(o, F: int, Hp: int, Wp: int, C: int = 16):
    """Inverse of patch_gather: o [L, 4C] -> [C, F, 2Hp, 2Wp]."""
    o = _f(o)
    r = o.reshape(F, Hp, Wp, C, 2, 2).transpose(3, 0, 1, 4, 2, 5)
    return r.reshape(C, F, 2 * Hp, 2 * Wp)


def head_unpatchify(x, w, b, F: int, Hp: int, Wp: int, C: int = 16):
    """Head Linear d -> 4C (R8) then unpatchify.  x [B, L, d] -> [B, C, F, H8, W8]."""
    return np.stack([unpatch_scatter(linear(x[i], w, b), F, Hp, Wp, C) for i in range(x.shape[0])])


# ---------------------------------------------------------------------------
# I2V inputs  [News, 核心创新四; Note, I2V 架构扩展]

def i2v_mask(frame_mask: Sequence[int], lat_f: int, H8: int, W8: int):
    """Binary mask over the 1+T video frames (1 = keep, 0 = generate) -> the 4
    mask channels [4, 1+T/4, H8, W8] (R10).  Frame 0 is repeated to make 4T/4+4
    values, grouped by 4 along time (the VAE's temporal stride), and the group
    member index becomes the channel."""
    fm = np.asarray(frame_mask, dtype=F64).reshape(-1)
    T = fm.shape[0] - 1
    if T % 4 or 1 + T // 4 != lat_f:
        raise ValueError("frame mask length does not match the latent frames")
    ext = np.concatenate([np.repeat(fm[:1], 4), fm[1:]])        # 4 + T values
    grp = ext.reshape(lat_f, 4).T                               # [4, lat_f]
    return np.broadcast_to(grp[:, :, None, None], (4, lat_f, H8, W8)).copy()


def image_context(clip, w1, b1, w2, b2, w3, b3):
    """Three-layer MLP from CLIP features to the model width (R11)."""
    return linear(gelu_tanh(linear(gelu_tanh(linear(clip, w1, b1)), w2, b2)), w3, b3)


# ---------------------------------------------------------------------------
# one denoising step

def step(latent, t, ctx, mw: Dict[str, object], heads: int, eps: float = 1e-6,
         clip=None, blocks: Optional[List[Dict[str, np.ndarray]]] = None,
         return_hidden: bool = False, fp8: bool = False, attn8: bool = False):
    """patchify -> shared t-MLP -> N blocks -> head -> unpatchify.
    latent [B, Cin, F, H8, W8]; t [B]; ctx [B, Lc, d]; clip [B, Li, 1280] or None.
    Returns the predicted velocity [B, 16, F, H8, W8] (the flow-matching
    target of [Note, 训练方法]).  ``blocks`` may be an iterable that yields the
    block weights one at a time (to bound host memory).  ``fp8``: every block
    with its six Linear layers in FP8 (R22 - R24); patchify, t-MLP, image MLP
    and head stay exact.  ``attn8``: every block's self-attention in 8 bits
    (R25, R26)."""
    lat = _f(latent)
    B, Cin, F, H8, W8 = lat.shape
    Hp, Wp = H8 // 2, W8 // 2
    x = patchify(lat, mw["patch_w"], mw["patch_b"])
    tw = mw["tmlp"]
    m = tmlp(t, tw["w1"], tw["b1"], tw["w2"], tw["b2"])
    img = None
    if clip is not None:
        iw = mw["img"]
        img = np.stack([image_context(clip[b], iw["w1"], iw["b1"], iw["w2"], iw["b2"],
                                      iw["w3"], iw["b3"]) for b in range(B)])
    for wts in (blocks if blocks is not None else mw["blocks"]):
        x = block(x, m, wts, ctx, heads, eps, img=img, fp8=fp8, attn8=attn8)
    out = head_unpatchify(x, mw["head_w"], mw["head_b"], F, Hp, Wp, 16)
    return (out, x) if return_hidden else out


# ---------------------------------------------------------------------------
# Sampler around the step (R19 - R21)


def cfg_combine(v_cond, v_uncond, scale: float):
    """Guided velocity v_u + s (v_c - v_u)  [Guide, 工作原理: guidance scale] (R20)."""
    vc, vu = _f(v_cond), _f(v_uncond)
    return vu + F64(scale) * (vc - vu)


def sampler_times(n_steps: int):
    """Flow times tau_k = k / N, k = 0..N (0 = noise, 1 = data), and the model's
    timestep input 1000 tau_k for the N evaluations  [Note, 训练方法; Infra] (R19)."""
    tau = np.arange(n_steps + 1, dtype=F64) / F64(n_steps)
    return tau, 1000.0 * tau[:-1]


def sample(latent0, n_steps: int, velocity, guidance: Optional[float] = None, out_ch: int = 16):
    """Explicit Euler along the flow from tau = 0 to tau = 1 (R19).

    latent0 [B, Cin, F, H8, W8]: channels 0..out_ch-1 hold the noise x0, the
    rest (I2V: condition latent and mask) stay fixed (R21).  ``velocity(latent,
    t)`` returns [B, out_ch, F, H8, W8] for timestep inputs t [B].  With a
    guidance scale the batch is one conditional / unconditional pair (R20):
    both samples move by the guided velocity.  Returns the latent at tau = 1."""
    x = _f(latent0).copy()
    B = x.shape[0]
    tau, tmodel = sampler_times(n_steps)
    if guidance is not None and B != 2:
        raise ValueError("guidance needs a conditional / unconditional pair")
    for k in range(n_steps):
        v = _f(velocity(x, np.full(B, tmodel[k])))
        if guidance is not None:
            g = cfg_combine(v[0], v[1], guidance)
            v = np.stack([g, g])
        x[:, :out_ch] = x[:, :out_ch] + (tau[k + 1] - tau[k]) * v
    return x


def text_kv(ctx, wts: Dict[str, np.ndarray], img=None):
    """The cross-attention keys and values of one block: they depend only on
    the text context (and image context) and the block's weights, not on the
    latent or the timestep, so a sampler computes them once
    [Note, Infra / 推理优化: work shared across sampling steps].
    ctx [Lc, d] -> (k [Lc, d], v [Lc, d]) (+ the image pair)."""
    d = _f(ctx).shape[-1]
    kv = linear(ctx, wts["ca_wkv"], wts["ca_bkv"])
    out = (kv[:, :d], kv[:, d:])
    if img is not None:
        kvi = linear(img, wts["ca_wkv_img"], wts["ca_bkv_img"])
        out = out + (kvi[:, :d], kvi[:, d:])
    return out


# ---------------------------------------------------------------------------
# FP8 (E4M3) GEMM emulation (R22)

E4M3_MAX = 448.0


def e4m3_values() -> np.ndarray:
    """All finite non-negative OCP E4M3 values, ascending: subnormals m/8 * 2^-6
    (m = 0..7), normals (1 + m/8) * 2^(e-7) for e = 1..15 except the NaN code
    e = 15, m = 7 (largest finite 1.75 * 2^8 = 448)."""
    v = [m / 8.0 * 2.0 ** -6 for m in range(8)]
    for e in range(1, 16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            v.append((1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(v, dtype=F64)


_E4M3 = e4m3_values()


def e4m3_round(v):
    """Round to the nearest E4M3 value, ties to the even code (the value whose
    3-bit mantissa is even); |v| must be <= 448 (R22 clamps first)."""
    a = np.abs(_f(v))
    if np.any(a > E4M3_MAX):
        raise ValueError("E4M3 rounding input beyond 448")
    idx = np.searchsorted(_E4M3, a)                 # first value >= a
    hi = np.minimum(idx, len(_E4M3) - 1)
    lo = np.maximum(idx - 1, 0)
    dlo, dhi = a - _E4M3[lo], _E4M3[hi] - a
    take_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))   # code index parity = mantissa parity
    q = np.where(take_hi, _E4M3[hi], _E4M3[lo])
    return np.sign(_f(v)) * q


def _scale_f32(amax):
    """(inv, scale) in float32 for an amax (float32): inv = 448 / amax, scale =
    amax / 448; amax = 0 gives (1, 1)."""
    amax = np.float32(amax)
    if amax == 0:
        return np.float32(1.0), np.float32(1.0)
    return np.float32(E4M3_MAX) / amax, amax / np.float32(E4M3_MAX)


def _quant_f32(x, inv):
    v = np.asarray(x, np.float32) * np.float32(inv)            # float32 product, as on the GPU
    v = np.clip(v, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_round(v.astype(F64))


def quantize_rows_fp8(x):
    """Per-token quantisation of x [M, K] (R22): returns (q [M, K] E4M3 values,
    scale [M]) with x ~= q * scale[:, None]."""
    x32 = np.asarray(x, np.float32)
    q = np.empty(x32.shape, F64)
    sc = np.empty(x32.shape[0], F64)
    for i in range(x32.shape[0]):
        inv, s = _scale_f32(np.max(np.abs(x32[i])) if x32.shape[1] else 0.0)
        q[i] = _quant_f32(x32[i], inv)
        sc[i] = s
    return q, sc


def quantize_tensor_fp8(w):
    """Per-tensor quantisation of a weight (R22): (q, scale) with w ~= q * scale."""
    w32 = np.asarray(w, np.float32)
    inv, s = _scale_f32(np.max(np.abs(w32)) if w32.size else 0.0)
    return _quant_f32(w32, inv), F64(s)


def bf16_round(x):
    """Round to the nearest bfloat16 value, ties to even, returned as float64:
    the float32 value's low 16 bits are dropped after adding 0x7FFF plus the
    lowest kept bit (finite inputs)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(F64)


def linear_fp8_q(x, qw, sw, b=None):
    """y = (xq qw^T) * sx[:, None] * sw + b for a weight already quantised
    (qw, sw) -- possibly a row slice of a tensor quantised as a whole -- and
    the per-token quantisation of the bf16 activation x (R22, R23)."""
    qx, sx = quantize_rows_fp8(bf16_round(x))
    y = (qx @ _f(qw).T) * sx[:, None] * F64(sw)
    if b is not None:
        y = y + _f(b)[None, :]
    return y


def linear_fp8(x, w, b=None):
    """y = (xq wq^T) * sx[:, None] * sw + b with per-token xq, per-tensor wq (R22)
    [Note, Infra / 推理优化: FP8 GEMM, per-tensor weights + per-token activations]."""
    qw, sw = quantize_tensor_fp8(w)
    return linear_fp8_q(x, qw, sw, b)


# ---------------------------------------------------------------------------
# 8-bit attention (R25)  [Note, Infra / 推理优化: 8-bit FlashAttention -- Int8
# for S = QK^T, FP8 for O = PV, FP32 accumulation across blocks]

I8_MAX = 127.0
ATTN8_KBLOCK = 64        # keys per K quantisation block
ATTN8_PSCALE = 128.0     # the row max of the probabilities maps to 2^7 before rounding


def _i8_scale_f32(amax):
    """(inv, scale) in float32: inv = 127 / amax, scale = amax / 127; amax = 0
    gives (1, 1)."""
    amax = np.float32(amax)
    if amax == 0:
        return np.float32(1.0), np.float32(1.0)
    return np.float32(I8_MAX) / amax, amax / np.float32(I8_MAX)


def quantize_int8(x):
    """Symmetric Int8 quantisation of x as one group (R25): (codes, scale) with
    x ~= codes * scale; the code is decided in float32 (x * inv, clamp to
    +-127, round half to even)."""
    x32 = np.asarray(x, np.float32)
    inv, s = _i8_scale_f32(np.max(np.abs(x32)) if x32.size else 0.0)
    v = np.clip(x32 * np.float32(inv), np.float32(-I8_MAX), np.float32(I8_MAX))
    return np.rint(v.astype(F64)), F64(s)


def quantize_q_int8(q):
    """Per-token Int8 quantisation of one head's q [L, hd] (R25): (codes [L, hd],
    scale [L])."""
    q = np.asarray(q, np.float32)
    codes = np.empty(q.shape, F64)
    sc = np.empty(q.shape[0], F64)
    for i in range(q.shape[0]):
        codes[i], sc[i] = quantize_int8(q[i])
    return codes, sc


def quantize_k_int8(k, block: int = ATTN8_KBLOCK):
    """Per-block Int8 quantisation of one head's k [L, hd] (R25): blocks of
    ``block`` consecutive keys share a scale.  Returns (codes [L, hd], scale
    of each block [ceil(L / block)])."""
    k = np.asarray(k, np.float32)
    nb = (k.shape[0] + block - 1) // block
    codes = np.empty(k.shape, F64)
    sc = np.empty(nb, F64)
    for bi in range(nb):
        codes[bi * block:(bi + 1) * block], sc[bi] = quantize_int8(k[bi * block:(bi + 1) * block])
    return codes, sc


def quantize_v_fp8(v):
    """Per-channel E4M3 quantisation of one head's v [L, hd] (R25 with R22's
    rule): each feature column gets its own scale.  Returns (codes [L, hd],
    scale [hd])."""
    q, sc = quantize_rows_fp8(np.asarray(v, np.float32).T)
    return q.T, sc


def attention_8bit(q, k, v, q_scaled: bool = False):
    """One head of the 8-bit attention (R25).  q [Lq, hd], k / v [Lk, hd] hold
    bf16 values.  q_scaled: q was multiplied by log2(e)/sqrt(hd) beforehand
    (the score is then in log2 units) -- the same attention of the unscaled q.
    Steps: quantise q per token, k per 64-key block (Int8) and v per channel
    (E4M3); integer scores times the two scales; probabilities relative to the
    row max, times 2^7, rounded to E4M3; PV on the rounded values, normalised
    by their sum, times the channel scales."""
    q8, sq = quantize_q_int8(q)
    k8, sk = quantize_k_int8(k)
    v8, sv = quantize_v_fp8(v)
    skey = np.repeat(sk, ATTN8_KBLOCK)[:k8.shape[0]]
    S = (q8 @ k8.T) * sq[:, None] * skey[None, :]
    if q_scaled:
        P = ATTN8_PSCALE * np.exp2(S - S.max(axis=1, keepdims=True))
    else:
        S = S / math.sqrt(q8.shape[1])
        P = ATTN8_PSCALE * np.exp(S - S.max(axis=1, keepdims=True))
    P8 = e4m3_round(P)
    return (P8 @ v8) * sv[None, :] / P8.sum(axis=1, keepdims=True)


def multihead_8bit(q, k, v, heads: int, q_scaled: bool = False):
    """attention_8bit per head (head h = columns h*hd .. (h+1)*hd) of one
    batch sample, concatenated."""
    hd = q.shape[1] // heads
    return np.concatenate([attention_8bit(q[:, h * hd:(h + 1) * hd], k[:, h * hd:(h + 1) * hd],
                                          v[:, h * hd:(h + 1) * hd], q_scaled)
                           for h in range(heads)], axis=1)
