"""Plant plausible mistakes in copies of the oracle (on the CPU) and require
that at least one pin catches each of them."""
import importlib.util
import os
import types

import pytest

from tests import oracle_pins as P

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "wan_oracle.py")

MUTATIONS = {
    "no attention scale": ("scale = 1.0 / math.sqrt(hd)", "scale = 1.0"),
    "k/v weights swapped": ("k = lin(hmod, slice(d, 2 * d), bqkv[d:2 * d])",
                            "k = lin(hmod, slice(2 * d, 3 * d), bqkv[2 * d:])"),
    "modulate sign": ("_f(xhat) * (1.0 + _f(scale))", "_f(xhat) * (1.0 - _f(scale))"),
    "sin/cos order": ("[np.cos(arg), np.sin(arg)]", "[np.sin(arg), np.cos(arg)]"),
    "unbiased variance": ("var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)",
                          "var = ((x - mu) ** 2).sum(axis=-1, keepdims=True) / (x.shape[-1] - 1)"),
    "eps outside sqrt": ("np.sqrt(var + eps)", "(np.sqrt(var) + eps)"),
    "gelu constant": ("0.044715", "0.0447"),
    "gated cross-attention": ("x2 = x1 + ca", "x2 = x1 + mod[\"gate1\"][b] * ca"),
    "modulation order": ('names = ("shift1", "scale1"', 'names = ("scale1", "shift1"'),
    "patch a/b swapped": ("transpose(1, 2, 4, 0, 3, 5)", "transpose(1, 2, 4, 0, 5, 3)"),
    "unpatch a/b swapped": ("transpose(3, 0, 1, 4, 2, 5)", "transpose(3, 0, 1, 5, 2, 4)"),
    "mask zero-pad reading": ("np.repeat(fm[:1], 4)", "np.concatenate([fm[:1], np.zeros(3)])"),
    "softmax wrong axis": ("P /= P.sum(axis=1, keepdims=True)", "P /= P.sum(axis=0, keepdims=True)"),
    "ungated FFN": ('x3 = x2 + mod["gate2"][b] * z', "x3 = x2 + z"),
    "silu slope": ("z / (1.0 + np.exp(-z))", "z / (1.0 + np.exp(-2 * z))"),
    "image V from K": ("o = o + multihead(q, ki, vi, heads)", "o = o + multihead(q, ki, ki, heads)"),
    "image MLP missing GELU": ("linear(gelu_tanh(linear(gelu_tanh(linear(clip, w1, b1)), w2, b2)), w3, b3)",
                               "linear(linear(gelu_tanh(linear(clip, w1, b1)), w2, b2), w3, b3)"),
    "t-MLP without SiLU": ("linear(silu(linear(e, w1, b1)), w2, b2)", "linear(linear(e, w1, b1), w2, b2)"),
    "block bias sign": ("_f(m) + _f(beta)[None, :]", "_f(m) - _f(beta)[None, :]"),
    "sinusoid base": ("math.log(10000.0)", "math.log(1000.0)"),
    "LN on modulated input for CA": ("q = lin(layer_norm(xq, eps), wq, bq)", "q = lin(xq, wq, bq)"),
    "seq_len off by one": ("return (1 + T // 4) * (height // 16)", "return (T // 4) * (height // 16)"),
    "Euler step sign": ("x[:, :out_ch] = x[:, :out_ch] + (tau[k + 1] - tau[k]) * v",
                        "x[:, :out_ch] = x[:, :out_ch] - (tau[k + 1] - tau[k]) * v"),
    "model time reversed": ("return tau, 1000.0 * tau[:-1]", "return tau, 1000.0 * (1.0 - tau[:-1])"),
    "guidance pair order": ("g = cfg_combine(v[0], v[1], guidance)", "g = cfg_combine(v[1], v[0], guidance)"),
    "guidance base": ("return vu + F64(scale) * (vc - vu)", "return vc + F64(scale) * (vc - vu)"),
    "text V from K": ("out = (kv[:, :d], kv[:, d:])", "out = (kv[:, :d], kv[:, :d])"),
    "e4m3 ties away from zero": ("take_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))",
                                 "take_hi = (dhi <= dlo)"),
    "fp8 scale to 240": ("return np.float32(E4M3_MAX) / amax, amax / np.float32(E4M3_MAX)",
                         "return np.float32(240.0) / amax, amax / np.float32(240.0)"),
    "fp8 activation scale per tensor": ("inv, s = _scale_f32(np.max(np.abs(x32[i])) if x32.shape[1] else 0.0)",
                                        "inv, s = _scale_f32(np.max(np.abs(x32)))"),
    "fp8 dequant without weight scale": ("y = (qx @ _f(qw).T) * sx[:, None] * F64(sw)",
                                         "y = (qx @ _f(qw).T) * sx[:, None]"),
    "fp8 activation not bf16": ("qx, sx = quantize_rows_fp8(bf16_round(x))", "qx, sx = quantize_rows_fp8(x)"),
    "bf16 ties away from zero": ("u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000",
                                 "u = (u + 0x8000) & 0xFFFF0000"),
    "fp8 Wqkv scale per slice": ("lin = lambda x, sl, b: linear_fp8_q(x, qw[sl], sw, b)",
                                 "lin = lambda x, sl, b: linear_fp8(x, wqkv[sl], b)"),
    "fp8 FFN down left exact": ("return lin(gelu_tanh(lin(hmod, w1, b1)), w2, b2)",
                                "return linear(gelu_tanh(lin(hmod, w1, b1)), w2, b2)"),
    "fp8 flag dropped for CA": ("wkv_img=wts.get(\"ca_wkv_img\"), bkv_img=wts.get(\"ca_bkv_img\"),\n                             fp8=fp8)",
                                "wkv_img=wts.get(\"ca_wkv_img\"), bkv_img=wts.get(\"ca_bkv_img\"))"),
    "fp8 flag not passed to the blocks": ("x = block(x, m, wts, ctx, heads, eps, img=img, fp8=fp8, attn8=attn8)",
                                          "x = block(x, m, wts, ctx, heads, eps, img=img, attn8=attn8)"),
    "attn8 flag not passed to the blocks": ("x = block(x, m, wts, ctx, heads, eps, img=img, fp8=fp8, attn8=attn8)",
                                            "x = block(x, m, wts, ctx, heads, eps, img=img, fp8=fp8)"),
    "attn8 K scales tiled, not repeated": ("skey = np.repeat(sk, ATTN8_KBLOCK)[:k8.shape[0]]",
                                           "skey = np.resize(sk, k8.shape[0])"),
    "attn8 K block of 32": ("def quantize_k_int8(k, block: int = ATTN8_KBLOCK):",
                            "def quantize_k_int8(k, block: int = 32):"),
    "attn8 normaliser unrounded": ("return (P8 @ v8) * sv[None, :] / P8.sum(axis=1, keepdims=True)",
                                   "return (P8 @ v8) * sv[None, :] / P.sum(axis=1, keepdims=True)"),
    "attn8 probabilities not scaled": ("P = ATTN8_PSCALE * np.exp(S - S.max(axis=1, keepdims=True))",
                                       "P = np.exp(S - S.max(axis=1, keepdims=True))"),
    "attn8 V scale per token": ("q, sc = quantize_rows_fp8(np.asarray(v, np.float32).T)\n    return q.T, sc",
                                "q, sc = quantize_rows_fp8(np.asarray(v, np.float32))\n    return q, sc[:q.shape[1]]"),
    "attn8 Int8 truncates": ("return np.rint(v.astype(F64)), F64(s)", "return np.trunc(v.astype(F64)), F64(s)"),
    "attn8 Int8 scale 128": ("return np.float32(I8_MAX) / amax, amax / np.float32(I8_MAX)",
                             "return np.float32(128.0) / amax, amax / np.float32(128.0)"),
    "attn8 pre-scaled q scaled again": ("        S = S / math.sqrt(q8.shape[1])\n        P = ATTN8_PSCALE * np.exp(",
                                        "        S = S / math.sqrt(q8.shape[1])\n        P = ATTN8_PSCALE * np.exp2("),
    "attn8 switch ignored": ("    if attn8:\n        o = multihead_8bit(", "    if False:\n        o = multihead_8bit("),
    "attn8 inputs not rounded to bf16": ("o = multihead_8bit(bf16_round(q), bf16_round(k), bf16_round(v), heads)",
                                         "o = multihead_8bit(q, k, v, heads)"),
    "attn8 flag not passed to the SA": ("heads, rows=rows, fp8=fp8, attn8=attn8)", "heads, rows=rows, fp8=fp8)"),
    "step drops the image context": ("x = block(x, m, wts, ctx, heads, eps, img=img, fp8=fp8, attn8=attn8)",
                                     "x = block(x, m, wts, ctx, heads, eps, img=None, fp8=fp8, attn8=attn8)"),
    "t-MLP fed t/1000": ("m = tmlp(t, tw[\"w1\"]", "m = tmlp(_f(t) / 1000.0, tw[\"w1\"]"),
    "blocks in reverse order": ("for wts in (blocks if blocks is not None else mw[\"blocks\"]):",
                                "for wts in list(blocks if blocks is not None else mw[\"blocks\"])[::-1]:"),
    "clip of sample 0 for every sample": ("img = np.stack([image_context(clip[b],", "img = np.stack([image_context(clip[0],"),
    "text context of sample 0 for every sample": ("ca = cross_attention(x1, _f(ctx[b]),", "ca = cross_attention(x1, _f(ctx[0]),"),
    "modulation of sample 0 for every sample": ('h1 = modulate(layer_norm(xb, eps), mod["shift1"][b], mod["scale1"][b])',
                                                'h1 = modulate(layer_norm(xb, eps), mod["shift1"][0], mod["scale1"][0])'),
    "head split strided": ("k[:, h * hd:(h + 1) * hd],\n                              v[:, h * hd:(h + 1) * hd])",
                           "k[:, h::heads],\n                              v[:, h::heads])"),
}


def _mutant(name, old, new):
    src = open(SRC, encoding="utf-8").read()
    assert src.count(old) >= 1, f"mutation site not found: {name}"
    src = src.replace(old, new)
    mod = types.ModuleType("wan_oracle_mutant")
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name):
    old, new = MUTATIONS[name]
    M = _mutant(name, old, new)
    caught = []
    for pname in dir(P):
        if not pname.startswith("pin_"):
            continue
        try:
            getattr(P, pname)(M)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append(f"{pname}: {type(e).__name__}")
    assert caught, f"no pin caught the planted mistake '{name}'"
