"""ctypes binding of libwandit (include/wan_dit.h): argument marshalling only.

Every computation runs in the HIP library; this module converts torch device
tensors into the plain pointers and sizes of the C ABI and turns a non-zero
status into an exception.  It never computes anything itself and raises if
the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# WANDIT_LIB may point at another build of the same library (e.g. a tuning variant)
LIB_PATH = os.environ.get("WANDIT_LIB") or os.path.join(_HERE, "libwandit.so")

WAN_F32, WAN_BF16 = 0, 1
# the static scratch of wan_dit_block_fwd_noalloc (WAN_NOALLOC_SCRATCH_BYTES in the header)
NOALLOC_SCRATCH_BYTES = 256 << 20

EXPORTS = ("wan_workspace_bytes", "wan_kv_cache_bytes", "wan_sample_workspace_bytes",
           "wan_status_str", "wan_tmlp_fwd", "wan_dit_block_fwd", "wan_dit_step_fwd",
           "wan_i2v_mask", "wan_attention_fwd", "wan_linear_fwd", "wan_kv_cache_fwd",
           "wan_dit_step_cached_fwd", "wan_euler_fwd", "wan_sample_fwd", "wan_quantize_rows_fp8",
           "wan_quantize_tensor_fp8", "wan_linear_fp8_fwd", "wan_block_fp8_bytes",
           "wan_quantize_block_fp8", "wan_block_fp8_workspace_bytes", "wan_dit_block_fp8_fwd",
           "wan_model_fp8_bytes", "wan_quantize_model_fp8", "wan_fp8_workspace_bytes",
           "wan_dit_step_fp8_fwd", "wan_sample_fp8_fwd", "wan_attention_8bit_workspace_bytes",
           "wan_attention_8bit_quantize", "wan_attention_8bit_q_fwd", "wan_attention_8bit_fwd",
           "wan_dit_block_noalloc_bytes", "wan_dit_block_fwd_noalloc", "wan_ln_modulate_fwd",
           "wan_set_attention_events")
_SIZE_FNS = ("wan_workspace_bytes", "wan_kv_cache_bytes", "wan_sample_workspace_bytes",
             "wan_block_fp8_bytes", "wan_block_fp8_workspace_bytes", "wan_model_fp8_bytes",
             "wan_fp8_workspace_bytes", "wan_attention_8bit_workspace_bytes",
             "wan_dit_block_noalloc_bytes")


class WanError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: status {status} ({text})")
        self.status = status


class Cfg(C.Structure):
    _fields_ = [(n, C.c_int) for n in ("dim", "heads", "head_dim", "ffn", "n_blocks", "in_ch",
                                         "out_ch", "freq_dim", "text_len", "img_len", "img_feat")] \
        + [("eps", C.c_float), ("dtype", C.c_int), ("attn8", C.c_int)]


class TmlpW(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("w1", "b1", "w2", "b2")]


_BLOCK_FIELDS = ("sa_wqkv", "sa_bqkv", "sa_wo", "sa_bo", "ca_wq", "ca_bq", "ca_wkv", "ca_bkv",
                 "ca_wkv_img", "ca_bkv_img", "ca_wo", "ca_bo", "ffn_w1", "ffn_b1", "ffn_w2",
                 "ffn_b2", "mod_bias")


class BlockW(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in _BLOCK_FIELDS]


class ModelW(C.Structure):
    _fields_ = [("patch_w", C.c_void_p), ("patch_b", C.c_void_p), ("tmlp", TmlpW),
                ("blocks", C.POINTER(BlockW)), ("head_w", C.c_void_p), ("head_b", C.c_void_p)] \
        + [(n, C.c_void_p) for n in ("img_w1", "img_b1", "img_w2", "img_b2", "img_w3", "img_b3")]


_lib = None


def lib() -> C.CDLL:
    """Load libwandit.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python video_diffusion_transformer_block_amd/build.py`")
        L = C.CDLL(LIB_PATH)
        vp, i, sz = C.c_void_p, C.c_int, C.c_size_t
        L.wan_workspace_bytes.argtypes = [C.POINTER(Cfg), i, i, i, i]
        L.wan_workspace_bytes.restype = sz
        L.wan_status_str.argtypes = [i]
        L.wan_status_str.restype = C.c_char_p
        L.wan_tmlp_fwd.argtypes = [C.POINTER(Cfg), vp, i, C.POINTER(TmlpW), vp, vp, sz, vp]
        L.wan_dit_block_fwd.argtypes = [C.POINTER(Cfg), vp, i, i, i, i, vp, C.POINTER(BlockW), vp,
                                        vp, vp, sz, vp]
        L.wan_dit_block_noalloc_bytes.argtypes = [C.POINTER(Cfg), i, i, i, i]
        L.wan_dit_block_fwd_noalloc.argtypes = [C.POINTER(Cfg), vp, i, i, i, i, vp, C.POINTER(BlockW),
                                                vp, vp, vp]
        L.wan_dit_step_fwd.argtypes = [C.POINTER(Cfg), vp, vp, i, i, i, i, vp, vp, C.POINTER(ModelW),
                                       vp, vp, sz, vp]
        L.wan_i2v_mask.argtypes = [vp, i, i, i, i, vp]
        L.wan_attention_fwd.argtypes = [vp, i, vp, i, vp, i, i, vp, i, i, i, i, i, i, vp]
        L.wan_linear_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, vp]
        L.wan_ln_modulate_fwd.argtypes = [vp, i, i, i, vp, i, C.c_float, vp, vp]
        L.wan_set_attention_events.argtypes = [vp, vp]
        L.wan_kv_cache_bytes.argtypes = [C.POINTER(Cfg), i]
        L.wan_kv_cache_bytes.restype = sz
        L.wan_sample_workspace_bytes.argtypes = [C.POINTER(Cfg), i, i, i, i]
        L.wan_sample_workspace_bytes.restype = sz
        L.wan_kv_cache_fwd.argtypes = [C.POINTER(Cfg), i, vp, vp, C.POINTER(ModelW), vp, sz, vp, sz, vp]
        L.wan_dit_step_cached_fwd.argtypes = [C.POINTER(Cfg), vp, vp, i, i, i, i, vp, sz,
                                              C.POINTER(ModelW), vp, vp, sz, vp]
        L.wan_euler_fwd.argtypes = [vp, vp, i, i, i, i, i, i, C.c_float, i, C.c_float, vp]
        L.wan_sample_fwd.argtypes = [C.POINTER(Cfg), vp, i, i, i, i, i, i, C.c_float, vp, sz,
                                     C.POINTER(ModelW), vp, sz, vp]
        L.wan_quantize_rows_fp8.argtypes = [vp, i, i, i, vp, i, vp, vp]
        L.wan_quantize_tensor_fp8.argtypes = [vp, C.c_long, vp, vp, vp, sz, vp]
        L.wan_linear_fp8_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, vp]
        L.wan_block_fp8_bytes.argtypes = [C.POINTER(Cfg)]
        L.wan_quantize_block_fp8.argtypes = [C.POINTER(Cfg), C.POINTER(BlockW), vp, sz, vp]
        L.wan_block_fp8_workspace_bytes.argtypes = [C.POINTER(Cfg), i, i, i, i]
        L.wan_dit_block_fp8_fwd.argtypes = [C.POINTER(Cfg), vp, i, i, i, i, vp, C.POINTER(BlockW), vp,
                                            vp, vp, vp, sz, vp]
        L.wan_model_fp8_bytes.argtypes = [C.POINTER(Cfg)]
        L.wan_quantize_model_fp8.argtypes = [C.POINTER(Cfg), C.POINTER(ModelW), vp, sz, vp]
        L.wan_fp8_workspace_bytes.argtypes = [C.POINTER(Cfg), i, i, i, i, i]
        L.wan_dit_step_fp8_fwd.argtypes = [C.POINTER(Cfg), vp, vp, i, i, i, i, vp, vp, C.POINTER(ModelW),
                                           vp, vp, vp, sz, vp]
        L.wan_sample_fp8_fwd.argtypes = [C.POINTER(Cfg), vp, i, i, i, i, i, i, C.c_float, vp, sz,
                                         C.POINTER(ModelW), vp, vp, sz, vp]
        L.wan_attention_8bit_workspace_bytes.argtypes = [i, i, i, i]
        L.wan_attention_8bit_quantize.argtypes = [vp, i, vp, i, vp, i, i, i, i, i, i, vp, vp, vp, vp, vp, vp,
                                                  vp]
        L.wan_attention_8bit_q_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
        L.wan_attention_8bit_fwd.argtypes = [vp, i, vp, i, vp, i, i, vp, i, i, i, i, i, i, vp, sz, vp]
        for n in EXPORTS:
            if n in _SIZE_FNS:
                getattr(L, n).restype = sz
            elif n != "wan_status_str":
                getattr(L, n).restype = i
        _lib = L
    return _lib


def status_str(st: int) -> str:
    return lib().wan_status_str(st).decode()


def _check(fn: str, st: int):
    if st != 0:
        raise WanError(fn, st, status_str(st))


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    return stream if isinstance(stream, int) else stream.cuda_stream


def make_cfg(*, dim, heads, ffn, n_blocks=1, in_ch=16, out_ch=16, freq_dim=256, text_len=512,
             img_len=0, img_feat=1280, eps=1e-6, dtype="bf16", attn8=False) -> Cfg:
    return Cfg(dim, heads, dim // heads, ffn, n_blocks, in_ch, out_ch, freq_dim, text_len,
               img_len, img_feat, eps, WAN_BF16 if dtype == "bf16" else WAN_F32, int(bool(attn8)))


def workspace_bytes(cfg: Cfg, B: int, lat_f: int, H8: int, W8: int) -> int:
    return int(lib().wan_workspace_bytes(C.byref(cfg), B, lat_f, H8, W8))


def tmlp_weights(d: Dict[str, torch.Tensor]) -> TmlpW:
    return TmlpW(_p(d["w1"]), _p(d["b1"]), _p(d["w2"]), _p(d["b2"]))


def block_weights(d: Dict[str, torch.Tensor]) -> BlockW:
    return BlockW(*[_p(d.get(n)) for n in _BLOCK_FIELDS])


def model_weights(d: Dict[str, object], blocks: Sequence[BlockW]):
    """Returns (ModelW, keep-alive array of block descriptors)."""
    arr = (BlockW * max(1, len(blocks)))(*blocks)
    img = d.get("img") or {}
    mw = ModelW(_p(d["patch_w"]), _p(d["patch_b"]), tmlp_weights(d["tmlp"]),
                C.cast(arr, C.POINTER(BlockW)), _p(d["head_w"]), _p(d["head_b"]),
                *[_p(img.get(n)) for n in ("w1", "b1", "w2", "b2", "w3", "b3")])
    return mw, arr


def tmlp_fwd(cfg: Cfg, t: torch.Tensor, tw: TmlpW, mod: torch.Tensor, ws: torch.Tensor,
             stream=None):
    _check("wan_tmlp_fwd", lib().wan_tmlp_fwd(C.byref(cfg), _p(t), t.numel(), C.byref(tw), _p(mod),
                                              _p(ws), ws.numel() * ws.element_size(),
                                              _stream(stream)))


def dit_block_fwd(cfg: Cfg, x: torch.Tensor, B: int, lat_f: int, Hp: int, Wp: int,
                  mod: torch.Tensor, bw: BlockW, ctx: torch.Tensor, img_ctx: Optional[torch.Tensor],
                  ws: torch.Tensor, stream=None):
    _check("wan_dit_block_fwd",
           lib().wan_dit_block_fwd(C.byref(cfg), _p(x), B, lat_f, Hp, Wp, _p(mod), C.byref(bw),
                                   _p(ctx), _p(img_ctx), _p(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)))


def dit_block_noalloc_bytes(cfg: Cfg, B: int, lat_f: int, Hp: int, Wp: int) -> int:
    return int(lib().wan_dit_block_noalloc_bytes(C.byref(cfg), B, lat_f, Hp, Wp))


def dit_block_fwd_noalloc(cfg: Cfg, x: torch.Tensor, B: int, lat_f: int, Hp: int, Wp: int,
                          mod: torch.Tensor, bw: BlockW, ctx: torch.Tensor,
                          img_ctx: Optional[torch.Tensor], stream=None):
    _check("wan_dit_block_fwd_noalloc",
           lib().wan_dit_block_fwd_noalloc(C.byref(cfg), _p(x), B, lat_f, Hp, Wp, _p(mod),
                                           C.byref(bw), _p(ctx), _p(img_ctx), _stream(stream)))


def dit_step_fwd(cfg: Cfg, latent: torch.Tensor, t: torch.Tensor, ctx: torch.Tensor,
                 clip: Optional[torch.Tensor], mw: ModelW, out: torch.Tensor, ws: torch.Tensor,
                 stream=None):
    B, _, F, H8, W8 = latent.shape
    _check("wan_dit_step_fwd",
           lib().wan_dit_step_fwd(C.byref(cfg), _p(latent), _p(t), B, F, H8, W8, _p(ctx), _p(clip),
                                  C.byref(mw), _p(out), _p(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)))


def attention_fwd(q, ldq, k, ldk, vt, ldv, vt_bstride, o, ldo, B, H, Lq, Lk, stream=None,
                  q_scaled=False):
    _check("wan_attention_fwd",
           lib().wan_attention_fwd(_p(q), ldq, _p(k), ldk, _p(vt), ldv, vt_bstride, _p(o), ldo,
                                   B, H, Lq, Lk, int(bool(q_scaled)), _stream(stream)))


def attention_8bit_workspace_bytes(B, H, Lq, Lk) -> int:
    return int(lib().wan_attention_8bit_workspace_bytes(B, H, Lq, Lk))


def attention_8bit_quantize(q, ldq, k, ldk, vt, ldv, vt_bstride, B, H, Lq, Lk, q8, qs, k8, ks, v8t, vs,
                            stream=None):
    _check("wan_attention_8bit_quantize",
           lib().wan_attention_8bit_quantize(_p(q), ldq, _p(k), ldk, _p(vt), ldv, vt_bstride, B, H, Lq, Lk,
                                             _p(q8), _p(qs), _p(k8), _p(ks), _p(v8t), _p(vs), _stream(stream)))


def attention_8bit_q_fwd(q8, qs, k8, ks, v8t, vs, o, ldo, B, H, Lq, Lk, q_scaled=False, stream=None):
    _check("wan_attention_8bit_q_fwd",
           lib().wan_attention_8bit_q_fwd(_p(q8), _p(qs), _p(k8), _p(ks), _p(v8t), _p(vs), _p(o), ldo, B, H,
                                          Lq, Lk, int(bool(q_scaled)), _stream(stream)))


def attention_8bit_fwd(q, ldq, k, ldk, vt, ldv, vt_bstride, o, ldo, B, H, Lq, Lk, ws, q_scaled=False,
                       stream=None):
    _check("wan_attention_8bit_fwd",
           lib().wan_attention_8bit_fwd(_p(q), ldq, _p(k), ldk, _p(vt), ldv, vt_bstride, _p(o), ldo, B, H,
                                        Lq, Lk, int(bool(q_scaled)), _p(ws),
                                        ws.numel() * ws.element_size(), _stream(stream)))


def linear_fwd(x, w, b, y, M, N, K, mode, stream=None):
    _check("wan_linear_fwd", lib().wan_linear_fwd(_p(x), _p(w), _p(b), _p(y), M, N, K, mode,
                                                  _stream(stream)))


def set_attention_events(start=None, stop=None):
    """Events (torch.cuda.Event, already created by a first record) the library
    records around the self-attention launches of this thread's next block
    calls; None, None clears them."""
    ev = lambda e: None if e is None else e.cuda_event
    _check("wan_set_attention_events", lib().wan_set_attention_events(ev(start), ev(stop)))


def ln_modulate_fwd(x, B, L, d, mod, branch, eps, h, stream=None):
    _check("wan_ln_modulate_fwd", lib().wan_ln_modulate_fwd(_p(x), B, L, d, _p(mod), branch, eps, _p(h),
                                                            _stream(stream)))


def i2v_mask(frame_mask: Sequence[int], lat_f: int, H8: int, W8: int):
    """Host helper: the 4 I2V mask channels [4, lat_f, H8, W8] as a float32 CPU tensor."""
    fm = (C.c_uint8 * len(frame_mask))(*[1 if v else 0 for v in frame_mask])
    out = torch.empty((4, lat_f, H8, W8), dtype=torch.float32)
    _check("wan_i2v_mask", lib().wan_i2v_mask(C.cast(fm, C.c_void_p), len(frame_mask), lat_f, H8, W8,
                                              _p(out)))
    return out


# ---- sampler around the step

def kv_cache_bytes(cfg: Cfg, B: int) -> int:
    return int(lib().wan_kv_cache_bytes(C.byref(cfg), B))


def sample_workspace_bytes(cfg: Cfg, B: int, lat_f: int, H8: int, W8: int) -> int:
    return int(lib().wan_sample_workspace_bytes(C.byref(cfg), B, lat_f, H8, W8))


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def kv_cache_fwd(cfg: Cfg, B: int, ctx: torch.Tensor, clip: Optional[torch.Tensor], mw: ModelW,
                 cache: torch.Tensor, ws: Optional[torch.Tensor], stream=None):
    _check("wan_kv_cache_fwd",
           lib().wan_kv_cache_fwd(C.byref(cfg), B, _p(ctx), _p(clip), C.byref(mw), _p(cache),
                                  _nbytes(cache), _p(ws), _nbytes(ws), _stream(stream)))


def dit_step_cached_fwd(cfg: Cfg, latent: torch.Tensor, t: torch.Tensor, cache: torch.Tensor,
                        mw: ModelW, out: torch.Tensor, ws: torch.Tensor, stream=None):
    B, _, F, H8, W8 = latent.shape
    _check("wan_dit_step_cached_fwd",
           lib().wan_dit_step_cached_fwd(C.byref(cfg), _p(latent), _p(t), B, F, H8, W8, _p(cache),
                                         _nbytes(cache), C.byref(mw), _p(out), _p(ws), _nbytes(ws),
                                         _stream(stream)))


def euler_fwd(latent: torch.Tensor, vel: torch.Tensor, dt: float, guided: bool = False,
              scale: float = 1.0, stream=None):
    B, cin, F, H8, W8 = latent.shape
    _check("wan_euler_fwd",
           lib().wan_euler_fwd(_p(latent), _p(vel), B, cin, vel.shape[1], F, H8, W8, dt,
                               1 if guided else 0, scale, _stream(stream)))


def sample_fwd(cfg: Cfg, latent: torch.Tensor, n_steps: int, cache: torch.Tensor, mw: ModelW,
               ws: torch.Tensor, guided: bool = False, scale: float = 1.0, stream=None):
    B, _, F, H8, W8 = latent.shape
    _check("wan_sample_fwd",
           lib().wan_sample_fwd(C.byref(cfg), _p(latent), B, F, H8, W8, n_steps, 1 if guided else 0,
                                scale, _p(cache), _nbytes(cache), C.byref(mw), _p(ws), _nbytes(ws),
                                _stream(stream)))


# ---- FP8 GEMM (OCP E4M3 operands, per-token / per-tensor scales)

def quantize_rows_fp8(x: torch.Tensor, q: torch.Tensor, scale: torch.Tensor, stream=None):
    M, K = x.shape
    _check("wan_quantize_rows_fp8", lib().wan_quantize_rows_fp8(_p(x), M, K, x.stride(0), _p(q),
                                                                q.stride(0), _p(scale),
                                                                _stream(stream)))


def quantize_tensor_fp8(w: torch.Tensor, q: torch.Tensor, scale: torch.Tensor, ws: torch.Tensor,
                        stream=None):
    _check("wan_quantize_tensor_fp8", lib().wan_quantize_tensor_fp8(_p(w), w.numel(), _p(q), _p(scale),
                                                                    _p(ws), _nbytes(ws),
                                                                    _stream(stream)))


def linear_fp8_fwd(xq, x_scale, wq, w_scale, b, y, M, N, K, mode, stream=None):
    _check("wan_linear_fp8_fwd", lib().wan_linear_fp8_fwd(_p(xq), _p(x_scale), _p(wq), _p(w_scale),
                                                          _p(b), _p(y), M, N, K, mode,
                                                          _stream(stream)))


def block_fp8_bytes(cfg: Cfg) -> int:
    return int(lib().wan_block_fp8_bytes(C.byref(cfg)))


def block_fp8_workspace_bytes(cfg: Cfg, B: int, lat_f: int, Hp: int, Wp: int) -> int:
    return int(lib().wan_block_fp8_workspace_bytes(C.byref(cfg), B, lat_f, Hp, Wp))


def quantize_block_fp8(cfg: Cfg, bw: BlockW, qbuf: torch.Tensor, stream=None):
    _check("wan_quantize_block_fp8", lib().wan_quantize_block_fp8(C.byref(cfg), C.byref(bw), _p(qbuf),
                                                                  _nbytes(qbuf), _stream(stream)))


def dit_block_fp8_fwd(cfg: Cfg, x: torch.Tensor, B: int, lat_f: int, Hp: int, Wp: int,
                      mod: torch.Tensor, bw: BlockW, qbuf: torch.Tensor, ctx: torch.Tensor,
                      img_ctx: Optional[torch.Tensor], ws: torch.Tensor, stream=None):
    _check("wan_dit_block_fp8_fwd",
           lib().wan_dit_block_fp8_fwd(C.byref(cfg), _p(x), B, lat_f, Hp, Wp, _p(mod), C.byref(bw),
                                       _p(qbuf), _p(ctx), _p(img_ctx), _p(ws), _nbytes(ws),
                                       _stream(stream)))


def model_fp8_bytes(cfg: Cfg) -> int:
    return int(lib().wan_model_fp8_bytes(C.byref(cfg)))


def fp8_workspace_bytes(cfg: Cfg, B: int, lat_f: int, H8: int, W8: int, sampler: bool = False) -> int:
    return int(lib().wan_fp8_workspace_bytes(C.byref(cfg), B, lat_f, H8, W8, int(bool(sampler))))


def quantize_model_fp8(cfg: Cfg, mw: ModelW, qbuf: torch.Tensor, stream=None):
    _check("wan_quantize_model_fp8", lib().wan_quantize_model_fp8(C.byref(cfg), C.byref(mw), _p(qbuf),
                                                                  _nbytes(qbuf), _stream(stream)))


def dit_step_fp8_fwd(cfg: Cfg, latent: torch.Tensor, t: torch.Tensor, ctx: torch.Tensor,
                     clip: Optional[torch.Tensor], mw: ModelW, qbuf: torch.Tensor, out: torch.Tensor,
                     ws: torch.Tensor, stream=None):
    B, _, F, H8, W8 = latent.shape
    _check("wan_dit_step_fp8_fwd",
           lib().wan_dit_step_fp8_fwd(C.byref(cfg), _p(latent), _p(t), B, F, H8, W8, _p(ctx), _p(clip),
                                      C.byref(mw), _p(qbuf), _p(out), _p(ws), _nbytes(ws),
                                      _stream(stream)))


def sample_fp8_fwd(cfg: Cfg, latent: torch.Tensor, n_steps: int, cache: torch.Tensor, mw: ModelW,
                   qbuf: torch.Tensor, ws: torch.Tensor, guided: bool = False, scale: float = 1.0,
                   stream=None):
    B, _, F, H8, W8 = latent.shape
    _check("wan_sample_fp8_fwd",
           lib().wan_sample_fp8_fwd(C.byref(cfg), _p(latent), B, F, H8, W8, n_steps, int(bool(guided)),
                                    float(scale), _p(cache), _nbytes(cache), C.byref(mw), _p(qbuf),
                                    _p(ws), _nbytes(ws), _stream(stream)))
