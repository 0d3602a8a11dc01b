"""Seeded synthetic inputs for the Wan2.1 DiT denoising step.

This module is the only code shared by the CPU oracle (``oracle/``) and the
GPU path (tests, ``bench.py``).  It holds *no* arithmetic of the method: only
model/workload shapes, seeded random draws and the bf16 rounding that turns a
draw into the exact value both sides consume.

Workloads (the five configurations both sides run):
  C1  tiny single block, fp32, L=128, dim 128, 2 heads of 64, FFN 512, 32 text tokens
  C2  1.3B-shaped block, bf16, 480x832x81 video -> latent 21x60x104, L=32760
  C3  1.3B-shaped full step (30 blocks), batch 2 (two text contexts), L=32760
  C4  14B-shaped block, bf16, 720x1280x81 video -> latent 21x90x160, L=75600
  C5  14B-shaped I2V full step (40 blocks), 36 input channels, 257 image tokens

Model widths follow the configuration table of the Wan 2.1 research note
("Wan: Open and Advanced Large-Scale Video Generative Models (Wan 2.1)",
table 配置表): 1.3B = dim 1536 / FFN 8960 / 12 heads / 30 layers, 14B = dim
5120 / FFN 13824 / 40 heads / 40 layers, latent in/out 16 channels, frequency
dimension 256.  Text length 512 comes from the same note's umT5 section.

Value recipe: every tensor gets its own PCG64 stream seeded by
``SeedSequence([2025, config_id, tensor_id, block_idx])``.  Weights and biases
are N(0, 0.02); latents, text context, CLIP features and block activations are
N(0, 1); the timestep is U[0, 1000).  For bf16 workloads every value is rounded
to bf16 (round to nearest, ties to even) here, so that both sides start from
identical numbers.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

__all__ = [
    "ModelCfg", "Workload", "WORKLOADS", "by_id", "bf16_round", "to_bf16_bits",
    "from_bf16_bits", "draw", "block_weights", "model_weights", "tmlp_weights",
    "workload_inputs", "mini",
]

WEIGHT_STD = 0.02


@dataclasses.dataclass(frozen=True)
class ModelCfg:
    dim: int
    heads: int
    ffn: int
    n_blocks: int
    in_ch: int = 16
    out_ch: int = 16
    freq_dim: int = 256
    text_len: int = 512
    img_len: int = 0          # 257 for the I2V model, else 0
    img_feat: int = 1280      # CLIP feature width (I2V only)
    eps: float = 1e-6
    dtype: str = "bf16"       # "bf16" or "f32": weight / activation operand type

    @property
    def head_dim(self) -> int:
        return self.dim // self.heads


@dataclasses.dataclass(frozen=True)
class Workload:
    cid: int                  # workload id, part of every seed
    name: str
    model: ModelCfg
    batch: int
    lat_f: int                # latent frames = 1 + T/4
    lat_h: int                # H/8
    lat_w: int                # W/8
    kind: str                 # "block" or "step"

    @property
    def Hp(self) -> int:
        return self.lat_h // 2

    @property
    def Wp(self) -> int:
        return self.lat_w // 2

    @property
    def L(self) -> int:
        return self.lat_f * self.Hp * self.Wp


_M13 = dict(dim=1536, heads=12, ffn=8960)
_M14 = dict(dim=5120, heads=40, ffn=13824)

# The full-size workloads, by name.  A workload's integer id seeds its
# inputs and weights (synth draws every array from it), so it stays fixed.
WORKLOADS: Dict[str, Workload] = {w.name: w for w in (
    Workload(1, "tiny-block-f32",
             ModelCfg(dim=128, heads=2, ffn=512, n_blocks=1, text_len=32, dtype="f32"),
             batch=1, lat_f=2, lat_h=16, lat_w=16, kind="block"),
    Workload(2, "wan1.3b-block-480p",
             ModelCfg(n_blocks=1, **_M13), batch=1, lat_f=21, lat_h=60, lat_w=104, kind="block"),
    Workload(3, "wan1.3b-step-480p-cfg2",
             ModelCfg(n_blocks=30, **_M13), batch=2, lat_f=21, lat_h=60, lat_w=104, kind="step"),
    Workload(4, "wan14b-block-720p",
             ModelCfg(n_blocks=1, **_M14), batch=1, lat_f=21, lat_h=90, lat_w=160, kind="block"),
    Workload(5, "wan14b-i2v-step-480p",
             ModelCfg(n_blocks=40, in_ch=36, img_len=257, **_M14),
             batch=1, lat_f=21, lat_h=60, lat_w=104, kind="step"),
)}


def by_id(cid: int) -> Workload:
    """The full-size workload with integer id cid."""
    for w in WORKLOADS.values():
        if w.cid == cid:
            return w
    raise KeyError(cid)


def mini(cid: int, name: str, *, dim: int, heads: int, ffn: int, n_blocks: int,
         lat_f: int, lat_h: int, lat_w: int, batch: int = 1, text_len: int = 40,
         in_ch: int = 16, img_len: int = 0, img_feat: int = 1280,
         dtype: str = "bf16", kind: str = "step") -> Workload:
    """A reduced workload with the structure of the full ones (for parity at
    sizes the oracle finishes in seconds)."""
    return Workload(cid, name, ModelCfg(dim=dim, heads=heads, ffn=ffn, n_blocks=n_blocks,
                                        in_ch=in_ch, text_len=text_len, img_len=img_len,
                                        img_feat=img_feat, dtype=dtype),
                    batch=batch, lat_f=lat_f, lat_h=lat_h, lat_w=lat_w, kind=kind)


# ----------------------------------------------------------------------------
# bf16 rounding (round to nearest, ties to even) on the host.

def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns (RNE).  Inputs are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Values of ``a`` rounded to the nearest bf16 (ties to even), as float32."""
    return from_bf16_bits(to_bf16_bits(a))


# ----------------------------------------------------------------------------
# tensor ids (stable: part of every seed)

TID = {
    # model-level
    "latent": 1, "t": 2, "ctx": 3, "clip": 4, "cond": 5, "x": 6,
    "patch_w": 10, "patch_b": 11, "head_w": 12, "head_b": 13,
    "tmlp_w1": 14, "tmlp_b1": 15, "tmlp_w2": 16, "tmlp_b2": 17,
    "img_w1": 18, "img_b1": 19, "img_w2": 20, "img_b2": 21, "img_w3": 22, "img_b3": 23,
    # per block
    "sa_wqkv": 30, "sa_bqkv": 31, "sa_wo": 32, "sa_bo": 33,
    "ca_wq": 34, "ca_bq": 35, "ca_wkv": 36, "ca_bkv": 37, "ca_wkv_img": 38, "ca_bkv_img": 39,
    "ca_wo": 40, "ca_bo": 41, "ffn_w1": 42, "ffn_b1": 43, "ffn_w2": 44, "ffn_b2": 45,
    "mod_bias": 46,
}


def _rng(cid: int, tensor: str, block: int = 0, sample: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([2025, cid, TID[tensor], block, sample])))


def draw(cid: int, tensor: str, shape, *, std: float = 1.0, block: int = 0,
         sample: int = 0, dtype: str = "bf16", uniform_hi: Optional[float] = None) -> np.ndarray:
    """One seeded tensor as float32.  bf16 workloads get bf16-representable
    values.  ``uniform_hi`` switches to U[0, uniform_hi)."""
    g = _rng(cid, tensor, block, sample)
    if uniform_hi is not None:
        a = (g.random(shape, dtype=np.float32) * np.float32(uniform_hi)).astype(np.float32)
        return a  # timesteps stay fp32 on both sides
    a = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if dtype == "bf16":
        a = bf16_round(a)
    return a


def tmlp_weights(w: Workload) -> Dict[str, np.ndarray]:
    m, c = w.model, w.cid
    s = dict(std=WEIGHT_STD, dtype=m.dtype)
    return {
        "w1": draw(c, "tmlp_w1", (m.dim, m.freq_dim), **s),
        "b1": draw(c, "tmlp_b1", (m.dim,), **s),
        "w2": draw(c, "tmlp_w2", (6 * m.dim, m.dim), **s),
        "b2": draw(c, "tmlp_b2", (6 * m.dim,), **s),
    }


def block_weights(w: Workload, i: int) -> Dict[str, np.ndarray]:
    """Weights of block ``i``.  Linear weights are [out, in].  ``mod_bias`` is
    kept fp32-valued-as-drawn for f32 workloads, bf16-rounded otherwise (the
    residual-side parameters are fp32 in memory either way)."""
    m, c = w.model, w.cid
    d, F = m.dim, m.ffn
    s = dict(std=WEIGHT_STD, dtype=m.dtype, block=i)
    out = {
        "sa_wqkv": draw(c, "sa_wqkv", (3 * d, d), **s),
        "sa_bqkv": draw(c, "sa_bqkv", (3 * d,), **s),
        "sa_wo": draw(c, "sa_wo", (d, d), **s),
        "sa_bo": draw(c, "sa_bo", (d,), **s),
        "ca_wq": draw(c, "ca_wq", (d, d), **s),
        "ca_bq": draw(c, "ca_bq", (d,), **s),
        "ca_wkv": draw(c, "ca_wkv", (2 * d, d), **s),
        "ca_bkv": draw(c, "ca_bkv", (2 * d,), **s),
        "ca_wo": draw(c, "ca_wo", (d, d), **s),
        "ca_bo": draw(c, "ca_bo", (d,), **s),
        "ffn_w1": draw(c, "ffn_w1", (F, d), **s),
        "ffn_b1": draw(c, "ffn_b1", (F,), **s),
        "ffn_w2": draw(c, "ffn_w2", (d, F), **s),
        "ffn_b2": draw(c, "ffn_b2", (d,), **s),
        "mod_bias": draw(c, "mod_bias", (6 * d,), **s),
    }
    if m.img_len:
        out["ca_wkv_img"] = draw(c, "ca_wkv_img", (2 * d, d), **s)
        out["ca_bkv_img"] = draw(c, "ca_bkv_img", (2 * d,), **s)
    return out


def model_weights(w: Workload, with_blocks: bool = True) -> Dict[str, object]:
    """Patchify / head / t-MLP / image-MLP weights (+ all blocks if asked).

    The I2V patchify weight has its 20 extra input channels (condition latent
    and mask) zero, the zero-initialised projection of the I2V design."""
    m, c = w.model, w.cid
    d = m.dim
    s = dict(std=WEIGHT_STD, dtype=m.dtype)
    pw = draw(c, "patch_w", (d, 16 * 4), **s)
    if m.in_ch > 16:
        full = np.zeros((d, m.in_ch * 4), np.float32)
        full[:, :64] = pw
        pw = full
    out: Dict[str, object] = {
        "patch_w": pw,
        "patch_b": draw(c, "patch_b", (d,), **s),
        "head_w": draw(c, "head_w", (m.out_ch * 4, d), **s),
        "head_b": draw(c, "head_b", (m.out_ch * 4,), **s),
        "tmlp": tmlp_weights(w),
    }
    if m.img_len:
        out["img"] = {
            "w1": draw(c, "img_w1", (d, m.img_feat), **s), "b1": draw(c, "img_b1", (d,), **s),
            "w2": draw(c, "img_w2", (d, d), **s), "b2": draw(c, "img_b2", (d,), **s),
            "w3": draw(c, "img_w3", (d, d), **s), "b3": draw(c, "img_b3", (d,), **s),
        }
    if with_blocks:
        out["blocks"] = [block_weights(w, i) for i in range(m.n_blocks)]
    return out


def workload_inputs(w: Workload) -> Dict[str, np.ndarray]:
    """Activations of a workload.

    * ``t``      [B]                 U[0,1000); one value shared by the batch
    * ``ctx``    [B, Lc, d]          one independent context per sample
    * ``latent`` [B, in_ch, F, H8, W8]  noise latent (same for every sample);
                  for I2V channels 16..31 are the condition latent (N(0,1)) and
                  channels 32..35 are left zero for the caller to fill with the
                  expanded binary mask.
    * ``x``      [B, L, d]           block input (block workloads only)
    * ``clip``   [B, Li, img_feat]   I2V image features
    """
    m, c = w.model, w.cid
    B, d = w.batch, m.dim
    dt = m.dtype
    t1 = draw(c, "t", (1,), uniform_hi=1000.0)
    out = {"t": np.repeat(t1, B).astype(np.float32)}
    out["ctx"] = np.stack([draw(c, "ctx", (m.text_len, d), sample=b, dtype=dt) for b in range(B)])
    lat = draw(c, "latent", (16, w.lat_f, w.lat_h, w.lat_w), dtype=dt)
    full = np.zeros((B, m.in_ch, w.lat_f, w.lat_h, w.lat_w), np.float32)
    full[:, :16] = lat
    if m.in_ch > 16:
        full[:, 16:32] = draw(c, "cond", (16, w.lat_f, w.lat_h, w.lat_w), dtype=dt)
    out["latent"] = full
    if w.kind == "block":
        out["x"] = np.stack([draw(c, "x", (w.L, d), sample=b, dtype=dt) for b in range(B)])
    if m.img_len:
        out["clip"] = np.stack([draw(c, "clip", (m.img_len, m.img_feat), sample=b, dtype=dt)
                                for b in range(B)])
    return out


def attention_inputs(seed: int, B: int, H: int, Lq: int, Lk: int, hd: int = 128,
                     qk_std: float = 2.0, v_std: float = 1.0):
    """Q, K, V for kernel-level attention stress tests, bf16-rounded float32.

    With q, k ~ N(0, qk_std^2) the logits q.k/sqrt(hd) have std qk_std^2 (4
    by default): a peaked softmax that exercises the running-max rescaling."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([2025, 99, seed, B, H, Lq, Lk])))
    q = bf16_round(g.standard_normal((B, Lq, H * hd), dtype=np.float32) * np.float32(qk_std))
    k = bf16_round(g.standard_normal((B, Lk, H * hd), dtype=np.float32) * np.float32(qk_std))
    v = bf16_round(g.standard_normal((B, Lk, H * hd), dtype=np.float32) * np.float32(v_std))
    return q, k, v


def attention_inputs_full(seed: int, H: int, L: int, hd: int = 128, qk_std: float = 2.0,
                          threads: int = 8):
    """Q, K, V [L, H*hd] (one batch sample) for attention stress tests at the
    full sequence lengths, bf16-rounded float32; each head's slice of each
    tensor has its own PCG64 stream (drawn on ``threads`` host threads).
    q, k ~ N(0, qk_std^2) (logits std qk_std^2), v ~ N(0, 1)."""
    from concurrent.futures import ThreadPoolExecutor
    out = [np.empty((L, H * hd), np.float32) for _ in range(3)]

    def fill(job):
        which, h = job
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([2025, 97, seed, H, L, which, h])))
        a = g.standard_normal((L, hd), dtype=np.float32)
        if which < 2:
            a *= np.float32(qk_std)
        out[which][:, h * hd:(h + 1) * hd] = bf16_round(a)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(fill, [(w, h) for w in range(3) for h in range(H)]))
    return out[0], out[1], out[2]


def block_weights_iter(w: "Workload", threads: int = 8):
    """Yield ``block_weights(w, i)`` for i = 0 .. n_blocks-1 in order, with up
    to ``threads`` blocks drawn ahead on host threads (the values are those
    of ``block_weights``: every tensor keeps its own seeded stream)."""
    from concurrent.futures import ThreadPoolExecutor
    n = w.model.n_blocks
    ahead = max(1, threads)
    with ThreadPoolExecutor(ahead) as ex:
        futs = {j: ex.submit(block_weights, w, j) for j in range(min(n, ahead))}
        for i in range(n):
            bw = futs.pop(i).result()
            if i + ahead < n:
                futs[i + ahead] = ex.submit(block_weights, w, i + ahead)
            yield bw


def linear_inputs(seed: int, M: int, N: int, K: int):
    """x ~ N(0,1), W ~ N(0, 1/K), b ~ N(0, 1), all bf16-rounded float32."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([2025, 98, seed, M, N, K])))
    x = bf16_round(g.standard_normal((M, K), dtype=np.float32))
    w = bf16_round(g.standard_normal((N, K), dtype=np.float32) / np.float32(np.sqrt(K)))
    b = bf16_round(g.standard_normal((N,), dtype=np.float32))
    return x, w, b


# ----------------------------------------------------------------------------
# On-device seeded weights for the full-size step checks that compare the GPU
# path with itself (batch independence, zero extra projection, determinism):
# the 14B model's 16 G parameters would take minutes to draw on the host.

def _dev_gen(device, cid: int, tensor: str, block: int = 0):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence([2025, cid, TID[tensor], block, 7]).generate_state(1)[0]))
    return g


def device_model_weights(w: Workload, device="cuda"):
    """Model weights of workload ``w`` drawn on the device (bf16 values of
    N(0, 0.02); per-block modulation bias float32), in the layout the C ABI
    takes.  The I2V patchify weight has its extra input channels zero."""
    import torch
    m, c = w.model, w.cid
    d, F = m.dim, m.ffn
    dt = torch.bfloat16 if m.dtype == "bf16" else torch.float32

    def rn(tensor, shape, block=0, dtype=dt):
        g = _dev_gen(device, c, tensor, block)
        return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * WEIGHT_STD).to(dtype)

    pw = rn("patch_w", (d, 16 * 4))
    if m.in_ch > 16:
        pw = torch.cat([pw, torch.zeros((d, (m.in_ch - 16) * 4), dtype=dt, device=device)], dim=1)
    out = {"patch_w": pw.contiguous(), "patch_b": rn("patch_b", (d,)),
           "head_w": rn("head_w", (m.out_ch * 4, d)), "head_b": rn("head_b", (m.out_ch * 4,)),
           "tmlp": {"w1": rn("tmlp_w1", (d, m.freq_dim)), "b1": rn("tmlp_b1", (d,)),
                    "w2": rn("tmlp_w2", (6 * d, d)), "b2": rn("tmlp_b2", (6 * d,))}}
    if m.img_len:
        out["img"] = {"w1": rn("img_w1", (d, m.img_feat)), "b1": rn("img_b1", (d,)),
                      "w2": rn("img_w2", (d, d)), "b2": rn("img_b2", (d,)),
                      "w3": rn("img_w3", (d, d)), "b3": rn("img_b3", (d,))}
    blocks = []
    for i in range(m.n_blocks):
        b = {"sa_wqkv": rn("sa_wqkv", (3 * d, d), i), "sa_bqkv": rn("sa_bqkv", (3 * d,), i),
             "sa_wo": rn("sa_wo", (d, d), i), "sa_bo": rn("sa_bo", (d,), i),
             "ca_wq": rn("ca_wq", (d, d), i), "ca_bq": rn("ca_bq", (d,), i),
             "ca_wkv": rn("ca_wkv", (2 * d, d), i), "ca_bkv": rn("ca_bkv", (2 * d,), i),
             "ca_wo": rn("ca_wo", (d, d), i), "ca_bo": rn("ca_bo", (d,), i),
             "ffn_w1": rn("ffn_w1", (F, d), i), "ffn_b1": rn("ffn_b1", (F,), i),
             "ffn_w2": rn("ffn_w2", (d, F), i), "ffn_b2": rn("ffn_b2", (d,), i),
             "mod_bias": rn("mod_bias", (6 * d,), i, dtype=torch.float32)}
        if m.img_len:
            b["ca_wkv_img"] = rn("ca_wkv_img", (2 * d, d), i)
            b["ca_bkv_img"] = rn("ca_bkv_img", (2 * d,), i)
        blocks.append(b)
    out["blocks"] = blocks
    return out
