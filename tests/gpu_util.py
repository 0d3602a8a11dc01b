"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path
through the C ABI, compare with the CPU oracle."""
from __future__ import annotations

from typing import Dict

import numpy as np
import torch

import video_diffusion_transformer_block_amd as W

DEV = "cuda"


def up(a: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 host array (bf16-representable for bf16) -> device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.to(DEV)


def up_block(wts: Dict[str, np.ndarray], dtype: str) -> Dict[str, torch.Tensor]:
    return {k: up(v, "f32" if k == "mod_bias" else dtype) for k, v in wts.items()}


def up_model(mw: Dict[str, object], dtype: str) -> Dict[str, object]:
    out = {k: up(v, dtype) for k, v in mw.items() if isinstance(v, np.ndarray)}
    out["tmlp"] = {k: up(v, dtype) for k, v in mw["tmlp"].items()}
    if "img" in mw:
        out["img"] = {k: up(v, dtype) for k, v in mw["img"].items()}
    return out


def cfg_of(work) -> W.Cfg:
    m = work.model
    return W.make_cfg(dim=m.dim, heads=m.heads, ffn=m.ffn, n_blocks=m.n_blocks, in_ch=m.in_ch,
                      out_ch=m.out_ch, freq_dim=m.freq_dim, text_len=m.text_len, img_len=m.img_len,
                      img_feat=m.img_feat, eps=m.eps, dtype=m.dtype)


def workspace(cfg, work) -> torch.Tensor:
    n = W.workspace_bytes(cfg, work.batch, work.lat_f, work.lat_h, work.lat_w)
    assert n > 0
    return torch.empty(n, dtype=torch.uint8, device=DEV)


def metrics(g, o) -> Dict[str, float]:
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    err = np.abs(g - o)
    return {"max_abs": float(err.max()) if err.size else 0.0,
            "mean_rel": float(err.sum() / max(np.abs(o).sum(), 1e-30))}


def assert_parity(g, o, max_abs=3e-2, mean_rel=1e-2, what=""):
    m = metrics(g, o)
    assert m["max_abs"] <= max_abs and m["mean_rel"] <= mean_rel, f"{what}: {m}"
    return m


def run_tmlp(cfg, work, tw_dev, t_dev):
    B = work.batch
    mod = torch.empty((B, 6 * work.model.dim), dtype=torch.float32, device=DEV)
    ws = torch.empty(B * (work.model.dim + work.model.freq_dim) * 4, dtype=torch.uint8, device=DEV)
    W.tmlp_fwd(cfg, t_dev, W.tmlp_weights(tw_dev), mod, ws)
    return mod
