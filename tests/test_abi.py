"""The C ABI on the host (no GPU needed): libwandit.so loads and exports every
function include/wan_dit.h declares; the host-only entry points (status
strings, workspace / cache sizing, the I2V mask helper) behave as declared;
invalid arguments are rejected before anything is enqueued."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle.wan_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wan_dit.h")


def _declared():
    src = open(HEADER, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w \*]*?\b(wan_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def W():
    import video_diffusion_transformer_block_amd as W
    W.lib()   # raises if the library has not been built
    return W


def test_every_declared_symbol_is_exported(W):
    names = _declared()
    assert len(names) >= 14, names
    L = C.CDLL(W.binding.LIB_PATH)
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    assert set(names) == set(W.binding.EXPORTS), "binding EXPORTS out of date with the header"


def test_status_strings(W):
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert W.status_str(st) and W.status_str(st) != "unknown status"
    assert W.status_str(-99) == "unknown status"


def _cfg(W, **kw):
    base = dict(dim=256, heads=2, ffn=512, n_blocks=3, text_len=40, dtype="bf16")
    base.update(kw)
    return W.make_cfg(**base)


def test_workspace_and_cache_sizes(W):
    c = _cfg(W)
    ws = W.workspace_bytes(c, 2, 3, 8, 12)
    assert ws > 0 and ws % 256 == 0
    # sampler workspace = step workspace + timestep and velocity buffers
    sw = W.sample_workspace_bytes(c, 2, 3, 8, 12)
    assert sw == ws + 256 + (2 * 16 * 3 * 8 * 12 * 4 + 255) // 256 * 256
    # cache: per block text K [B*Lc, d] and V^T [d, B*round_up(Lc, 64)] in bf16
    per = (2 * 40 * 256 * 2 + 255) // 256 * 256 + 256 * 2 * 64 * 2
    assert W.kv_cache_bytes(c, 2) == 3 * per
    ci = _cfg(W, in_ch=36, img_len=257, img_feat=1280)
    assert W.kv_cache_bytes(ci, 1) > W.kv_cache_bytes(_cfg(W, in_ch=36), 1)
    # invalid configurations size to 0
    assert W.workspace_bytes(_cfg(W, heads=3), 1, 1, 8, 8) == 0        # head_dim != 128
    assert W.workspace_bytes(c, 1, 1, 7, 8) == 0                        # odd H8
    assert W.workspace_bytes(c, 9, 1, 8, 8) == 0                        # B > 8
    assert W.kv_cache_bytes(c, 0) == 0
    assert W.sample_workspace_bytes(_cfg(W, ffn=500), 1, 1, 8, 8) == 0  # ffn % 64


def test_i2v_mask_matches_oracle(W):
    rng = np.random.default_rng(3)
    for n in (1, 5, 81):
        lat_f = (n - 1) // 4 + 1
        fm = rng.integers(0, 2, n)
        fm[0] = 1
        got = W.i2v_mask(fm.tolist(), lat_f, 6, 4).numpy()
        assert np.array_equal(got, O.i2v_mask(fm, lat_f, 6, 4).astype(np.float32))
    with pytest.raises(W.WanError):
        W.i2v_mask([1] * 6, 2, 4, 4)      # 6 frames is not 4k+1


def test_invalid_arguments_enqueue_nothing(W):
    L = W.lib()
    c = _cfg(W)
    dummy = C.c_void_p(16)   # never dereferenced: every call below fails validation first
    # guidance needs a pair; in_ch < out_ch; non-finite dt
    assert L.wan_euler_fwd(dummy, dummy, 3, 16, 16, 1, 2, 2, 0.1, 1, 1.0, None) == -2
    assert L.wan_euler_fwd(dummy, dummy, 2, 8, 16, 1, 2, 2, 0.1, 0, 1.0, None) == -2
    assert L.wan_euler_fwd(dummy, dummy, 1, 16, 16, 1, 2, 2, float("nan"), 0, 1.0, None) == -2
    assert L.wan_euler_fwd(None, dummy, 1, 16, 16, 1, 2, 2, 0.1, 0, 1.0, None) == -1
    mw, keep = W.model_weights({"patch_w": None, "patch_b": None, "tmlp": {"w1": None, "b1": None,
                                "w2": None, "b2": None}, "head_w": None, "head_b": None}, [])
    # NULL weights, zero steps, short cache / workspace
    assert L.wan_sample_fwd(C.byref(c), dummy, 2, 3, 8, 12, 4, 1, 5.0, dummy, 1 << 30, C.byref(mw),
                            dummy, 1 << 40, None) == -1
    assert L.wan_sample_fwd(C.byref(c), dummy, 2, 3, 8, 12, 0, 1, 5.0, dummy, 1 << 30, C.byref(mw),
                            dummy, 1 << 40, None) == -2
    assert L.wan_kv_cache_fwd(C.byref(c), 2, None, None, C.byref(mw), dummy, 1 << 30, None, 0,
                              None) == -1
    assert L.wan_dit_step_cached_fwd(C.byref(c), dummy, dummy, 2, 3, 7, 12, dummy, 1 << 30,
                                     C.byref(mw), dummy, dummy, 1 << 40, None) == -2   # odd H8
    assert L.wan_attention_fwd(dummy, 100, dummy, 256, dummy, 64, 64, dummy, 256, 1, 2, 4, 4, 0,
                               None) == -2                                          # ldq < H*128
    assert L.wan_linear_fwd(dummy, dummy, None, dummy, 4, 4, 100, 0, None) == -2   # K % 64


def test_fp8_block_sizes(W):
    c = _cfg(W)
    d, F = 256, 512
    # six scales, six running-maximum words, then the E4M3 weights, each region 256-aligned
    want = 256 + 256 + 3 * d * d + 3 * d * d + 2 * F * d
    assert W.block_fp8_bytes(c) == want
    assert W.block_fp8_bytes(_cfg(W, dtype="f32", heads=4)) == 0
    # the FP8 block workspace is a bf16 block workspace plus one activation's
    # codes (the widest, [B*L, ffn]) and its per-token scales
    B, L = 2, 3 * 4 * 6
    ws8 = W.block_fp8_workspace_bytes(c, B, 3, 4, 6)
    assert ws8 >= B * L * F + B * L * 4 and ws8 % 256 == 0
    assert W.block_fp8_workspace_bytes(c, 9, 3, 4, 6) == 0


def test_fp8_block_invalid_arguments(W):
    L = W.lib()
    c = _cfg(W)
    cf = _cfg(W, dtype="f32", heads=4)
    dummy = C.c_void_p(256)   # never dereferenced: every call below fails validation first
    bw = W.block_weights({})
    assert L.wan_quantize_block_fp8(C.byref(cf), C.byref(bw), dummy, 1 << 30, None) == -3
    assert L.wan_quantize_block_fp8(C.byref(c), C.byref(bw), dummy, 1 << 30, None) == -1
    args = (dummy, 2, 3, 4, 6, dummy, C.byref(bw))
    assert L.wan_dit_block_fp8_fwd(C.byref(cf), *args, dummy, dummy, None, dummy, 1 << 40, None) == -3
    assert L.wan_dit_block_fp8_fwd(C.byref(c), *args, None, dummy, None, dummy, 1 << 40, None) == -1
    assert L.wan_dit_block_fp8_fwd(C.byref(c), *args, C.c_void_p(272), dummy, None, dummy, 1 << 40,
                                   None) == -2                                     # qbuf misaligned
    assert L.wan_dit_block_fp8_fwd(C.byref(c), *args, dummy, dummy, None, dummy, 1 << 40, None) == -1



def test_fp8_model_sizes_and_invalid_arguments(W):
    c = _cfg(W)   # 3 blocks
    assert W.model_fp8_bytes(c) == 3 * W.block_fp8_bytes(c)
    assert W.model_fp8_bytes(_cfg(W, dtype="f32", heads=4)) == 0
    step = W.fp8_workspace_bytes(c, 2, 3, 8, 12)
    samp = W.fp8_workspace_bytes(c, 2, 3, 8, 12, True)
    assert step > W.workspace_bytes(c, 2, 3, 8, 12) and samp > step
    assert W.fp8_workspace_bytes(c, 2, 3, 7, 12) == 0                 # odd H8
    L = W.lib()
    cf = _cfg(W, dtype="f32", heads=4)
    dummy = C.c_void_p(256)   # never dereferenced: every call below fails validation first
    mw, keep = W.model_weights({"patch_w": None, "patch_b": None, "tmlp": {"w1": None, "b1": None,
                                "w2": None, "b2": None}, "head_w": None, "head_b": None}, [])
    assert L.wan_quantize_model_fp8(C.byref(cf), C.byref(mw), dummy, 1 << 30, None) == -3
    assert L.wan_quantize_model_fp8(C.byref(c), C.byref(mw), dummy, 1 << 30, None) == -1
    assert L.wan_dit_step_fp8_fwd(C.byref(cf), dummy, dummy, 2, 3, 8, 12, dummy, None, C.byref(mw),
                                  dummy, dummy, dummy, 1 << 40, None) == -3
    assert L.wan_dit_step_fp8_fwd(C.byref(c), dummy, dummy, 2, 3, 8, 12, dummy, None, C.byref(mw),
                                  None, dummy, dummy, 1 << 40, None) == -1
    assert L.wan_sample_fp8_fwd(C.byref(c), dummy, 2, 3, 8, 12, 0, 1, 5.0, dummy, 1 << 30,
                                C.byref(mw), dummy, dummy, 1 << 40, None) == -2   # zero steps


def test_attn8_sizes_and_invalid_arguments(W):
    # six copies, each 256-aligned: q8, qs, k8, ks, v8t, vs
    B, H, Lq, Lk = 2, 3, 100, 70
    d, Lkp = H * 128, 128
    parts = [B * Lq * d, B * Lq * H * 4, B * Lk * d, B * H * 2 * 4, d * B * Lkp, B * d * 4]
    assert W.attention_8bit_workspace_bytes(B, H, Lq, Lk) == sum((p + 255) // 256 * 256 for p in parts)
    assert W.attention_8bit_workspace_bytes(0, H, Lq, Lk) == 0
    assert W.attention_8bit_workspace_bytes(1, 40, 10, 500000) == 0          # beyond 32-bit offsets
    L = W.lib()
    dummy = C.c_void_p(256)   # never dereferenced: every call below fails validation first
    ws = 1 << 40
    assert L.wan_attention_8bit_fwd(dummy, 384, dummy, 384, dummy, 256, 128, dummy, 384, 2, 3, 100, 70, 0,
                                    None, ws, None) == -1
    assert L.wan_attention_8bit_fwd(dummy, 100, dummy, 384, dummy, 256, 128, dummy, 384, 2, 3, 100, 70, 0,
                                    dummy, ws, None) == -2                  # ldq < H*128
    assert L.wan_attention_8bit_fwd(dummy, 384, dummy, 384, dummy, 256, 64, dummy, 384, 2, 3, 100, 70, 0,
                                    dummy, ws, None) == -2                  # vt_bstride < round_up(Lk, 64)
    assert L.wan_attention_8bit_fwd(dummy, 384, dummy, 384, dummy, 256, 128, dummy, 384, 2, 3, 100, 70, 0,
                                    dummy, 1024, None) == -4                # short workspace
    assert L.wan_attention_8bit_quantize(dummy, 384, dummy, 384, dummy, 256, 128, 2, 3, 100, 70, dummy, None,
                                         dummy, dummy, dummy, dummy, None) == -1
    assert L.wan_attention_8bit_q_fwd(dummy, dummy, dummy, dummy, dummy, dummy, dummy, 100, 2, 3, 100, 70, 0,
                                      None) == -2                           # ldo < H*128
    # a head count whose row width does not fit an int is a shape error, not an overflow
    assert L.wan_attention_8bit_fwd(dummy, 384, dummy, 384, dummy, 256, 128, dummy, 384, 2, 1 << 25, 100, 70,
                                    0, dummy, ws, None) == -2
    assert L.wan_attention_fwd(dummy, 384, dummy, 384, dummy, 256, 128, dummy, 384, 2, 1 << 25, 100, 70, 0,
                               None) == -2


def test_size_limits(W):
    """Shapes the 32-bit operand offsets allow: the 14B block at 720P takes a
    guided pair in bf16 (V^T of both samples under 2 GiB) but not three
    samples; in FP8 only one sample's operands must fit."""
    c = W.make_cfg(dim=5120, heads=40, ffn=13824)
    assert W.workspace_bytes(c, 2, 21, 90, 160) > 0
    assert W.workspace_bytes(c, 3, 21, 90, 160) == 0
    assert W.fp8_workspace_bytes(c, 2, 21, 90, 160) > 0
    # one sample whose FFN hidden state reaches 2 GiB (L * ffn * 2 bytes)
    assert W.workspace_bytes(c, 1, 21, 96, 160) == 0


def test_attn8_cfg_checks(W):
    """cfg attn8: bf16 only, 0 or 1, and the block workspace grows by the
    8-bit copies of q, k, V^T."""
    c = W.make_cfg(dim=128, heads=2, ffn=256, dtype="f32", attn8=True)
    assert W.workspace_bytes(c, 1, 2, 4, 4) == 0
    c = W.make_cfg(dim=256, heads=2, ffn=256, attn8=True)
    c.attn8 = 2
    assert W.workspace_bytes(c, 1, 2, 4, 4) == 0
    c.attn8 = 1
    base = W.workspace_bytes(W.make_cfg(dim=256, heads=2, ffn=256), 1, 2, 4, 4)
    assert W.workspace_bytes(c, 1, 2, 4, 4) == base + W.attention_8bit_workspace_bytes(1, 2, 8, 8)


def test_noalloc_scratch_limit(W):
    """The allocation-free block: the header's scratch size matches the
    binding's, the need grows with the tokens, and a size beyond the scratch
    is refused with WAN_ERR_WORKSPACE before any device work."""
    src = open(HEADER, encoding="utf-8").read()
    m = re.search(r"#define\s+WAN_NOALLOC_SCRATCH_BYTES\s+\(\(size_t\)(\d+)\s*<<\s*(\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == W.NOALLOC_SCRATCH_BYTES
    c = W.make_cfg(dim=1536, heads=12, ffn=8960)
    small = W.dit_block_noalloc_bytes(c, 1, 2, 30, 52)
    assert 0 < small <= W.NOALLOC_SCRATCH_BYTES
    assert small < W.dit_block_noalloc_bytes(c, 2, 2, 30, 52)
    assert W.dit_block_noalloc_bytes(c, 1, 21, 30, 52) > W.NOALLOC_SCRATCH_BYTES
    assert W.dit_block_noalloc_bytes(c, 9, 2, 30, 52) == 0
    L = W.lib()
    dummy = C.c_void_p(256)   # never dereferenced: every call below fails validation first
    bw = W.binding.BlockW(*([256] * 17))
    assert L.wan_dit_block_fwd_noalloc(C.byref(c), dummy, 1, 21, 30, 52, dummy, C.byref(bw), dummy,
                                       None, None) == -4
    assert L.wan_dit_block_fwd_noalloc(C.byref(c), None, 1, 2, 30, 52, dummy, C.byref(bw), dummy,
                                       None, None) == -1
    assert L.wan_dit_block_fwd_noalloc(C.byref(c), dummy, 1, 2, 30, 52, dummy, C.byref(bw), dummy,
                                       dummy, None) == -5                  # image context without img_len


def test_ln_modulate_invalid_arguments(W):
    L = W.lib()
    dummy = C.c_void_p(256)   # never dereferenced: every call below fails validation first
    assert L.wan_ln_modulate_fwd(None, 1, 4, 8, None, 0, 1e-6, dummy, None) == -1
    assert L.wan_ln_modulate_fwd(dummy, 9, 4, 8, None, 0, 1e-6, dummy, None) == -2     # B > 8
    assert L.wan_ln_modulate_fwd(dummy, 1, 0, 8, None, 0, 1e-6, dummy, None) == -2     # L = 0
    assert L.wan_ln_modulate_fwd(dummy, 1, 4, 8, None, 0, 0.0, dummy, None) == -2      # eps
    assert L.wan_ln_modulate_fwd(dummy, 1, 4, 8, dummy, 2, 1e-6, dummy, None) == -5    # branch
