"""Pins of the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` takes the oracle module ``O`` and raises AssertionError when
the oracle disagrees with a closed form, a library routine (torch CPU), a
brute-force loop on tiny inputs, or an invariant the method must satisfy.
``tests/test_oracle_pins.py`` runs them on the real oracle;
``tests/test_oracle_mutations.py`` runs them on oracles with planted mistakes
and requires that at least one pin fails for each mistake.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as TF

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _t(a):
    return torch.from_numpy(np.asarray(a, np.float64))


# ---------------------------------------------------------------- shapes
def pin_shapes(O):
    """L and latent shapes of the pages' workloads (tests/golden/shapes.json)."""
    with open(os.path.join(GOLDEN, "shapes.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        fr, h, w = case["frames"], case["height"], case["width"]
        assert O.seq_len(fr, h, w) == case["L"], case
        assert tuple(O.latent_shape(fr, h, w)) == tuple(case["latent"]), case
    # 5 s at 16 fps is 80 frame intervals: 1 + T = 81 frames
    assert 1 + 5 * 16 == g["frames_5s_16fps"]


# ---------------------------------------------------------------- elementwise
def pin_silu_gelu(O):
    z = np.linspace(-8, 8, 97)
    _close(O.silu(z), TF.silu(_t(z)).numpy(), 1e-13, "silu vs torch")
    _close(O.gelu_tanh(z), TF.gelu(_t(z), approximate="tanh").numpy(), 1e-13, "gelu vs torch")
    assert O.gelu_tanh(np.array([0.0]))[0] == 0.0
    _close(O.gelu_tanh(np.array([30.0])), [30.0], 1e-12, "gelu large")


def pin_layer_norm(O):
    x = _rng(1).normal(size=(7, 33)) * 3 + 5
    _close(O.layer_norm(x, 1e-6), TF.layer_norm(_t(x), (33,), eps=1e-6).numpy(), 1e-12,
           "layer_norm vs torch")
    _close(O.layer_norm(x + 17.0, 1e-6), O.layer_norm(x, 1e-6), 1e-9, "LN shift invariance")
    c = np.full((2, 16), 3.25)
    assert np.all(O.layer_norm(c, 1e-6) == 0.0), "LN of a constant row"
    # eps enters inside the sqrt: row (-1, 1) has var 1 -> x/sqrt(1+eps)
    _close(O.layer_norm(np.array([[-1.0, 1.0]]), 0.5), [[-1 / math.sqrt(1.5), 1 / math.sqrt(1.5)]],
           1e-15, "LN eps placement")


def pin_modulate(O):
    x = _rng(2).normal(size=(5, 8))
    sh, sc = _rng(3).normal(size=8), _rng(4).normal(size=8)
    assert np.array_equal(O.modulate(x, np.zeros(8), np.zeros(8)), x)
    _close(O.modulate(x, sh, np.full(8, -1.0)), np.broadcast_to(sh, x.shape), 0, "scale=-1 -> shift")
    _close(O.modulate(np.ones((1, 8)), sh, sc), (1 + sc + sh)[None], 1e-15, "x=1")


# ---------------------------------------------------------------- timestep
def pin_sinusoid(O):
    e0 = O.sinusoid(np.array([0.0]), 256)
    assert e0.shape == (1, 256)
    assert np.all(e0[0, :128] == 1.0) and np.all(e0[0, 128:] == 0.0), "t = 0"
    t = np.array([0.5, 3.0, 999.0])
    e = O.sinusoid(t, 256)
    _close(e[:, :128] ** 2 + e[:, 128:] ** 2, np.ones((3, 128)), 1e-12, "cos^2+sin^2")
    # w_0 = 1, w_64 = 10000^(-1/2) = 0.01, w_127 = 10000^(-127/128)
    _close(e[:, 0], np.cos(t), 1e-14, "w_0")
    _close(e[:, 128], np.sin(t), 1e-14, "sin w_0")
    _close(e[:, 64], np.cos(0.01 * t), 1e-12, "w_64")
    _close(e[:, 128 + 127], np.sin(t * 10000.0 ** (-127 / 128)), 1e-12, "w_127")


def pin_tmlp(O):
    r = _rng(5)
    d = 6
    w1, b1 = r.normal(size=(d, 256)) * 0.1, r.normal(size=d)
    w2, b2 = r.normal(size=(6 * d, d)), r.normal(size=6 * d)
    t = np.array([0.0, 412.5])
    m = O.tmlp(t, w1, b1, np.zeros_like(w2), b2)
    assert np.array_equal(m, np.broadcast_to(b2, (2, 6 * d))), "W2 = 0 -> m = b2"
    # W1 = 0 -> hidden = SiLU(b1) for every t; SiLU(b) = b / (1 + e^-b)
    m0 = O.tmlp(t, np.zeros_like(w1), b1, w2, b2)
    h = np.array([bb / (1 + math.exp(-bb)) for bb in b1])
    _close(m0, np.broadcast_to(w2 @ h + b2, (2, 6 * d)), 1e-12, "W1 = 0")
    # t = 0: the embedding is [1]*128 | [0]*128, so the first layer sums the cos-half columns
    z = w1[:, :128].sum(axis=1) + b1
    h = z / (1 + np.exp(-z))
    _close(O.tmlp(np.array([0.0]), w1, b1, w2, b2)[0], w2 @ h + b2, 1e-12, "t = 0 closed form")
    # torch composition (library Linear + SiLU)
    tt = torch.tensor([412.5], dtype=torch.float64)
    e = _t(O.sinusoid(np.array([412.5])))
    ref = TF.linear(TF.silu(TF.linear(e, _t(w1), _t(b1))), _t(w2), _t(b2)).numpy()
    _close(O.tmlp(tt.numpy(), w1, b1, w2, b2), ref, 1e-12, "tmlp vs torch")
    # block modulation: beta adds, order shift1, scale1, gate1, shift2, scale2, gate2
    beta = np.arange(6 * d, dtype=np.float64)
    mm = O.block_modulation(np.zeros((1, 6 * d)), beta)
    for j, n in enumerate(("shift1", "scale1", "gate1", "shift2", "scale2", "gate2")):
        assert np.array_equal(mm[n][0], beta[j * d:(j + 1) * d]), n


# ---------------------------------------------------------------- attention
def _brute_attention(q, k, v):
    """Triple loop, fp64 Python floats."""
    Lq, hd = q.shape
    Lk = k.shape[0]
    out = np.zeros((Lq, v.shape[1]))
    for i in range(Lq):
        s = [sum(q[i, c] * k[j, c] for c in range(hd)) / math.sqrt(hd) for j in range(Lk)]
        mx = max(s)
        p = [math.exp(x - mx) for x in s]
        tot = sum(p)
        for c in range(v.shape[1]):
            out[i, c] = sum(p[j] * v[j, c] for j in range(Lk)) / tot
    return out


def pin_attention(O):
    r = _rng(6)
    for Lq, Lk, hd in ((5, 7, 4), (9, 3, 8), (1, 1, 4), (6, 11, 16)):
        q, k, v = r.normal(size=(Lq, hd)) * 2, r.normal(size=(Lk, hd)) * 2, r.normal(size=(Lk, hd))
        _close(O.attention(q, k, v), _brute_attention(q, k, v), 1e-12, f"brute {Lq}x{Lk}x{hd}")
    q, k, v = r.normal(size=(40, 16)), r.normal(size=(70, 16)), r.normal(size=(70, 16))
    ref = TF.scaled_dot_product_attention(_t(q)[None], _t(k)[None], _t(v)[None])[0].numpy()
    _close(O.attention(q, k, v), ref, 1e-12, "attention vs torch sdpa")
    # rows of the softmax sum to one: V = 1 -> O = 1
    _close(O.attention(q * 8, k, np.ones((70, 16))), np.ones((40, 16)), 1e-12, "V = 1")
    # equal keys -> uniform weights -> mean of V
    kk = np.repeat(r.normal(size=(1, 16)), 70, axis=0)
    _close(O.attention(q, kk, v), np.broadcast_to(v.mean(axis=0), (40, 16)), 1e-12, "equal keys")
    # one dominant key -> its value row
    kd = np.zeros((70, 16)); kd[13] = 200.0
    qd = np.ones((3, 16))
    _close(O.attention(qd, kd, v), np.broadcast_to(v[13], (3, 16)), 1e-12, "dominant key")
    # L = 1 -> O = V
    _close(O.attention(q[:4], k[:1], v[:1]), np.broadcast_to(v[0], (4, 16)), 1e-14, "Lk = 1")
    # permutation equivariance of self-attention (no positional term)
    x = r.normal(size=(30, 16))
    perm = r.permutation(30)
    _close(O.attention(x[perm], x[perm], x[perm]), O.attention(x, x, x)[perm], 1e-12,
           "permutation equivariance")
    # chunking is invisible
    _close(O.attention(q, k, v, chunk=7), O.attention(q, k, v, chunk=1024), 1e-13, "chunking")


def _torch_mha(x_q, x_kv, w_in, b_in, wo, bo, heads):
    d = x_q.shape[1]
    mha = torch.nn.MultiheadAttention(d, heads, bias=True, batch_first=True, dtype=torch.float64)
    with torch.no_grad():
        mha.in_proj_weight.copy_(_t(w_in)); mha.in_proj_bias.copy_(_t(b_in))
        mha.out_proj.weight.copy_(_t(wo)); mha.out_proj.bias.copy_(_t(bo))
        y, _ = mha(_t(x_q)[None], _t(x_kv)[None], _t(x_kv)[None], need_weights=False)
    return y[0].numpy()


def pin_self_attention(O):
    r = _rng(7)
    L, d, H = 12, 16, 2
    h = r.normal(size=(L, d))
    wqkv, bqkv = r.normal(size=(3 * d, d)) * 0.5, r.normal(size=3 * d)
    wo, bo = r.normal(size=(d, d)) * 0.5, r.normal(size=d)
    ref = _torch_mha(h, h, wqkv, bqkv, wo, bo, H)
    _close(O.self_attention(h, wqkv, bqkv, wo, bo, H), ref, 1e-11, "SA vs torch MHA")
    rows = np.array([0, 5, 11])
    _close(O.self_attention(h, wqkv, bqkv, wo, bo, H, rows=rows), ref[rows], 1e-11, "SA rows")


def pin_cross_attention(O):
    r = _rng(8)
    L, Lc, Li, d, H = 10, 6, 4, 16, 4
    x, ctx, img = r.normal(size=(L, d)) * 2 + 1, r.normal(size=(Lc, d)), r.normal(size=(Li, d))
    wq, bq = r.normal(size=(d, d)) * 0.5, r.normal(size=d)
    wkv, bkv = r.normal(size=(2 * d, d)) * 0.5, r.normal(size=2 * d)
    wki, bki = r.normal(size=(2 * d, d)) * 0.5, r.normal(size=2 * d)
    wo, bo = r.normal(size=(d, d)) * 0.5, r.normal(size=d)
    xn = TF.layer_norm(_t(x), (d,), eps=1e-6).numpy()
    ref_t = _torch_mha(xn, ctx, np.concatenate([wq, wkv]), np.concatenate([bq, bkv]), wo, bo, H)
    _close(O.cross_attention(x, ctx, wq, bq, wkv, bkv, wo, bo, H), ref_t, 1e-11, "CA vs torch MHA")
    # decoupled: text part + image part share Q and the out-projection; the
    # out-projection is affine, so CA2 = CA_text + CA_img - bo
    ref_i = _torch_mha(xn, img, np.concatenate([wq, wki]), np.concatenate([bq, bki]), wo, bo, H)
    got = O.cross_attention(x, ctx, wq, bq, wkv, bkv, wo, bo, H, img=img, wkv_img=wki, bkv_img=bki)
    _close(got, ref_t + ref_i - bo, 1e-11, "decoupled CA")


def pin_ffn(O):
    r = _rng(9)
    h = r.normal(size=(7, 8))
    w1, b1, w2, b2 = r.normal(size=(20, 8)), r.normal(size=20), r.normal(size=(8, 20)), r.normal(size=8)
    lin1 = torch.nn.Linear(8, 20, dtype=torch.float64)
    lin2 = torch.nn.Linear(20, 8, dtype=torch.float64)
    with torch.no_grad():
        lin1.weight.copy_(_t(w1)); lin1.bias.copy_(_t(b1)); lin2.weight.copy_(_t(w2)); lin2.bias.copy_(_t(b2))
        ref = lin2(TF.gelu(lin1(_t(h)), approximate="tanh")).numpy()
    _close(O.ffn(h, w1, b1, w2, b2), ref, 1e-11, "FFN vs torch")


# ---------------------------------------------------------------- block
def _tiny_block_weights(r, d, F, img=False, scale=0.3):
    w = {
        "sa_wqkv": r.normal(size=(3 * d, d)) * scale, "sa_bqkv": r.normal(size=3 * d) * scale,
        "sa_wo": r.normal(size=(d, d)) * scale, "sa_bo": r.normal(size=d) * scale,
        "ca_wq": r.normal(size=(d, d)) * scale, "ca_bq": r.normal(size=d) * scale,
        "ca_wkv": r.normal(size=(2 * d, d)) * scale, "ca_bkv": r.normal(size=2 * d) * scale,
        "ca_wo": r.normal(size=(d, d)) * scale, "ca_bo": r.normal(size=d) * scale,
        "ffn_w1": r.normal(size=(F, d)) * scale, "ffn_b1": r.normal(size=F) * scale,
        "ffn_w2": r.normal(size=(d, F)) * scale, "ffn_b2": r.normal(size=d) * scale,
        "mod_bias": r.normal(size=6 * d) * scale,
    }
    if img:
        w["ca_wkv_img"] = r.normal(size=(2 * d, d)) * scale
        w["ca_bkv_img"] = r.normal(size=2 * d) * scale
    return w


def pin_block(O):
    r = _rng(10)
    B, L, Lc, d, F, H = 2, 9, 5, 16, 24, 2
    x = r.normal(size=(B, L, d))
    ctx = r.normal(size=(B, Lc, d))
    m = r.normal(size=(B, 6 * d))
    w = _tiny_block_weights(r, d, F)
    y = O.block(x, m, w, ctx, H)
    # gates zero and cross-attention out-projection zero -> identity (bitwise)
    mz = m.copy()
    wz = dict(w)
    mz[:, 2 * d:3 * d] = -w["mod_bias"][2 * d:3 * d]
    mz[:, 5 * d:6 * d] = -w["mod_bias"][5 * d:6 * d]
    wz["ca_wo"] = np.zeros_like(w["ca_wo"]); wz["ca_bo"] = np.zeros_like(w["ca_bo"])
    assert np.array_equal(O.block(x, mz, wz, ctx, H), x), "zero gates + zero CA-out -> identity"
    # gates zero alone -> x + CA(LN(x), ctx) (ungated cross-attention)
    yz = O.block(x, mz, w, ctx, H)
    for b in range(B):
        ca = O.cross_attention(x[b], ctx[b], w["ca_wq"], w["ca_bq"], w["ca_wkv"], w["ca_bkv"],
                               w["ca_wo"], w["ca_bo"], H)
        _close(yz[b], x[b] + ca, 1e-12, "zero gates -> x + CA")
    # batch independence
    _close(O.block(x[1:], m[1:], w, ctx[1:], H)[0], y[1], 1e-12, "batch independence")
    # token permutation equivariance of the whole block
    perm = r.permutation(L)
    _close(O.block(x[:, perm], m, w, ctx, H), y[:, perm], 1e-11, "block permutation equivariance")
    # rows subset
    rows = np.array([1, 4, 8])
    _close(O.block(x, m, w, ctx, H, rows=rows), y[:, rows], 1e-12, "block rows")
    # composition from torch library pieces
    for b in range(B):
        _close(y[b], _torch_block(x[b], m[b], w, ctx[b], H), 1e-10, "block vs torch composition")


def _torch_block(xb, mb, w, ctxb, H, imgb=None):
    """One sample of the block built from torch library pieces (LayerNorm,
    MultiheadAttention, Linear, GELU): x1 = x + gate1 SA(modulated LN x),
    x2 = x1 + CA(LN x1) (text part + image part sharing Q and the out-
    projection), x3 = x2 + gate2 FFN(modulated LN x2)."""
    d = xb.shape[-1]
    mb = _t(np.asarray(mb) + w["mod_bias"]).reshape(6, d)
    xb = _t(xb)
    lin = lambda a, W, bb: TF.linear(a, _t(W), _t(bb))
    h1 = TF.layer_norm(xb, (d,), eps=1e-6) * (1 + mb[1]) + mb[0]
    sa = _t(_torch_mha(h1.numpy(), h1.numpy(), w["sa_wqkv"], w["sa_bqkv"], w["sa_wo"], w["sa_bo"], H))
    x1 = xb + mb[2] * sa
    xn = TF.layer_norm(x1, (d,), eps=1e-6).numpy()
    ca = _t(_torch_mha(xn, ctxb, np.concatenate([w["ca_wq"], w["ca_wkv"]]),
                       np.concatenate([w["ca_bq"], w["ca_bkv"]]), w["ca_wo"], w["ca_bo"], H))
    if imgb is not None:
        ca = ca + _t(_torch_mha(xn, imgb, np.concatenate([w["ca_wq"], w["ca_wkv_img"]]),
                                np.concatenate([w["ca_bq"], w["ca_bkv_img"]]), w["ca_wo"],
                                w["ca_bo"], H)) - _t(w["ca_bo"])
    x2 = x1 + ca
    h2 = TF.layer_norm(x2, (d,), eps=1e-6) * (1 + mb[4]) + mb[3]
    z = lin(TF.gelu(lin(h2, w["ffn_w1"], w["ffn_b1"]), approximate="tanh"), w["ffn_w2"], w["ffn_b2"])
    return (x2 + mb[5] * z).numpy()


# ---------------------------------------------------------------- patchify
def _brute_conv3d_122(lat, w, b):
    """Direct loops: Conv3d, kernel = stride = (1,2,2), weight [d, C, 1, 2, 2]."""
    C, Fr, H8, W8 = lat.shape
    d = w.shape[0]
    w5 = w.reshape(d, C, 1, 2, 2)
    out = np.zeros((d, Fr, H8 // 2, W8 // 2))
    for o in range(d):
        for f in range(Fr):
            for i in range(H8 // 2):
                for j in range(W8 // 2):
                    s = b[o]
                    for c in range(C):
                        for a in range(2):
                            for bb in range(2):
                                s += w5[o, c, 0, a, bb] * lat[c, f, 2 * i + a, 2 * j + bb]
                    out[o, f, i, j] = s
    return out


def pin_patchify(O):
    r = _rng(11)
    C, Fr, H8, W8, d = 3, 2, 4, 6, 5
    lat = r.normal(size=(1, C, Fr, H8, W8))
    w, b = r.normal(size=(d, C * 4)), r.normal(size=d)
    x = O.patchify(lat, w, b)[0]                            # [L, d]
    ref = _brute_conv3d_122(lat[0], w, b)                    # [d, F, Hp, Wp]
    _close(x, ref.reshape(d, -1).T, 1e-12, "patchify vs brute conv3d (token order f,i,j)")
    lib = TF.conv3d(_t(lat), _t(w.reshape(d, C, 1, 2, 2)), _t(b), stride=(1, 2, 2))[0].numpy()
    _close(x, lib.reshape(d, -1).T, 1e-12, "patchify vs torch conv3d")
    # unpatchify is the transposed convolution with the same kernel layout
    o = r.normal(size=(1, x.shape[0], 4 * C))
    wh, bh = r.normal(size=(4 * C, d)), r.normal(size=4 * C)
    y = O.head_unpatchify(x[None], wh, bh, Fr, H8 // 2, W8 // 2, C)[0]
    hx = x @ wh.T + bh                                       # [L, 4C]
    # conv_transpose3d input [1, 4C -> treat head output channels as C*(1*2*2) groups]
    inp = _t(hx.T.reshape(1, 4 * C, Fr, H8 // 2, W8 // 2))
    # a per-channel scatter: weight [in=4C, out=C, 1, 2, 2] with one-hot placement
    wt = torch.zeros(4 * C, C, 1, 2, 2, dtype=torch.float64)
    for c in range(C):
        for a in range(2):
            for bb in range(2):
                wt[c * 4 + a * 2 + bb, c, 0, a, bb] = 1.0
    lib = TF.conv_transpose3d(inp, wt, stride=(1, 2, 2))[0].numpy()
    _close(y, lib, 0, "unpatchify vs torch conv_transpose3d scatter")
    # identity weights -> exact round trip of the latent
    C16 = 16
    lat16 = r.normal(size=(2, C16, 2, 4, 6)).astype(np.float32).astype(np.float64)
    dd = 64
    x16 = O.patchify(lat16, np.eye(dd), np.zeros(dd))
    back = O.head_unpatchify(x16, np.eye(dd), np.zeros(dd), 2, 2, 3, C16)
    assert np.array_equal(back, lat16), "identity round trip"
    # I2V: the 20 extra channels with a zero projection leave the noise channels' tokens
    w36 = np.zeros((d, 36 * 4)); w36[:, :64] = r.normal(size=(d, 64))
    lat36 = r.normal(size=(1, 36, 2, 4, 6))
    assert np.array_equal(O.patchify(lat36, w36, b), O.patchify(lat36[:, :16], w36[:, :64], b)), \
        "zero extra projection"


# ---------------------------------------------------------------- I2V
def pin_i2v(O):
    with open(os.path.join(GOLDEN, "i2v_mask.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        fm = np.zeros(case["frames"]); fm[case["ones"]] = 1
        m = O.i2v_mask(fm, case["lat_f"], 3, 2)
        assert m.shape == (4, case["lat_f"], 3, 2)
        nz = sorted({(int(c), int(f)) for c, f, _, _ in zip(*np.nonzero(m))})
        assert nz == [tuple(p) for p in case["nonzero_channel_frame"]], (case, nz)
        assert set(np.unique(m)) <= {0.0, 1.0}
    r = _rng(12)
    d, H = 8, 2
    clip = r.normal(size=(5, 12))
    ws = [r.normal(size=s) for s in ((d, 12), (d,), (d, d), (d,), (d, d), (d,))]
    seq = torch.nn.Sequential(torch.nn.Linear(12, d), torch.nn.GELU(approximate="tanh"),
                              torch.nn.Linear(d, d), torch.nn.GELU(approximate="tanh"),
                              torch.nn.Linear(d, d)).double()
    with torch.no_grad():
        for lin, (wi, bi) in zip((seq[0], seq[2], seq[4]), ((ws[0], ws[1]), (ws[2], ws[3]), (ws[4], ws[5]))):
            lin.weight.copy_(_t(wi)); lin.bias.copy_(_t(bi))
        ref = seq(_t(clip)).numpy()
    _close(O.image_context(clip, *ws), ref, 1e-12, "image MLP vs torch")


# ---------------------------------------------------------------- step
def pin_step(O):
    r = _rng(13)
    B, d, H, F = 2, 64, 2, 32
    Fr, H8, W8, Lc = 2, 4, 6, 3
    lat = r.normal(size=(B, 16, Fr, H8, W8))
    t = np.array([10.0, 700.0])
    ctx = r.normal(size=(B, Lc, d))
    mw = {"patch_w": np.eye(d), "patch_b": np.zeros(d), "head_w": np.eye(d), "head_b": np.zeros(d),
          "tmlp": {"w1": r.normal(size=(d, 256)) * 0.1, "b1": r.normal(size=d),
                   "w2": np.zeros((6 * d, d)), "b2": np.zeros(6 * d)}}
    # every block an identity: gate biases 0 (m = 0 because W2 = 0, b2 = 0), CA out zero
    blocks = []
    for _ in range(3):
        w = _tiny_block_weights(r, d, F)
        w["mod_bias"][2 * d:3 * d] = 0; w["mod_bias"][5 * d:6 * d] = 0
        w["ca_wo"] = np.zeros((d, d)); w["ca_bo"] = np.zeros(d)
        blocks.append(w)
    mw["blocks"] = blocks
    assert np.array_equal(O.step(lat, t, ctx, mw, H), lat), "identity step"
    # with real blocks the batch entries are independent (the composition
    # against torch pieces is pin_step_wiring)
    for w in blocks:
        w["mod_bias"] = r.normal(size=6 * d) * 0.3
        w["ca_wo"] = r.normal(size=(d, d)) * 0.3
    mw["tmlp"]["w2"] = r.normal(size=(6 * d, d)) * 0.1
    out = O.step(lat, t, ctx, mw, H)
    out1 = O.step(lat[1:], t[1:], ctx[1:], mw, H)
    _close(out1[0], out[1], 1e-9, "step batch independence")


def _torch_step(lat, t, ctx, mw, H, clip=None):
    """The denoising step built from torch library pieces and the pages' order
    ([Note, Diffusion Transformer]; [Note, I2V 架构扩展]): Conv3d patchify with
    kernel = stride = (1,2,2); the 256-wide sinusoid of the raw timestep through
    Linear-SiLU-Linear once per sample; the image features of *that* sample
    through Linear-GELU-Linear-GELU-Linear; the blocks in list order, each fed
    the same modulation and contexts; the head Linear and the transposed
    (1,2,2) scatter back to the latent grid."""
    B, Cin, Fr, H8, W8 = lat.shape
    d = mw["patch_w"].shape[0]
    Hp, Wp = H8 // 2, W8 // 2
    tw = mw["tmlp"]
    half = 128
    om = torch.exp(-math.log(10000.0) * torch.arange(half, dtype=torch.float64) / half)
    wt = torch.zeros(64, 16, 1, 2, 2, dtype=torch.float64)
    for c in range(16):
        for a in range(2):
            for bb in range(2):
                wt[c * 4 + a * 2 + bb, c, 0, a, bb] = 1.0
    outs = []
    for s in range(B):
        conv = TF.conv3d(_t(lat[s:s + 1]), _t(mw["patch_w"].reshape(d, Cin, 1, 2, 2)),
                         _t(mw["patch_b"]), stride=(1, 2, 2))[0]          # [d, F, Hp, Wp]
        x = conv.reshape(d, -1).T.numpy()
        arg = float(t[s]) * om
        e = torch.cat([torch.cos(arg), torch.sin(arg)])
        m = TF.linear(TF.silu(TF.linear(e, _t(tw["w1"]), _t(tw["b1"]))), _t(tw["w2"]), _t(tw["b2"]))
        img = None
        if clip is not None:
            iw = mw["img"]
            g = lambda a: TF.gelu(a, approximate="tanh")
            img = TF.linear(g(TF.linear(g(TF.linear(_t(clip[s]), _t(iw["w1"]), _t(iw["b1"]))),
                                        _t(iw["w2"]), _t(iw["b2"]))), _t(iw["w3"]), _t(iw["b3"])).numpy()
        for w in mw["blocks"]:
            x = _torch_block(x, m.numpy(), w, ctx[s], H, img)
        hx = TF.linear(_t(x), _t(mw["head_w"]), _t(mw["head_b"]))           # [L, 64]
        inp = hx.T.reshape(1, 64, Fr, Hp, Wp)
        outs.append(TF.conv_transpose3d(inp, wt, stride=(1, 2, 2))[0].numpy())
    return np.stack(outs)


def pin_step_wiring(O):
    """step() against the step composed from torch pieces (``_torch_step``) on
    an I2V pair whose samples differ in timestep, text context and image
    features, with three distinct blocks (their order matters) and non-zero
    extra patchify columns.  Also: swapping the two samples' clip features
    swaps the outputs, the blocks in reverse order give a different result,
    and a timestep change moves the output only through the t-MLP."""
    r = _rng(14)
    B, d, H, F = 2, 16, 2, 24
    Fr, H8, W8, Lc, Li, feat = 2, 4, 6, 5, 3, 12
    lat = r.normal(size=(B, 36, Fr, H8, W8))
    t = np.array([37.5, 810.0])
    ctx = r.normal(size=(B, Lc, d))
    clip = r.normal(size=(B, Li, feat))
    mw = {"patch_w": r.normal(size=(d, 36 * 4)) * 0.3, "patch_b": r.normal(size=d) * 0.3,
          "head_w": r.normal(size=(64, d)) * 0.3, "head_b": r.normal(size=64) * 0.3,
          "tmlp": {"w1": r.normal(size=(d, 256)) * 0.3, "b1": r.normal(size=d) * 0.3,
                   "w2": r.normal(size=(6 * d, d)) * 0.3, "b2": r.normal(size=6 * d) * 0.3},
          "img": {"w1": r.normal(size=(d, feat)) * 0.3, "b1": r.normal(size=d) * 0.3,
                  "w2": r.normal(size=(d, d)) * 0.3, "b2": r.normal(size=d) * 0.3,
                  "w3": r.normal(size=(d, d)) * 0.3, "b3": r.normal(size=d) * 0.3},
          "blocks": [_tiny_block_weights(r, d, F, img=True, scale=0.4) for _ in range(3)]}
    out = O.step(lat, t, ctx, mw, H, clip=clip)
    ref = _torch_step(lat, t, ctx, mw, H, clip=clip)
    _close(out, ref, 1e-9, "I2V step vs torch composition")
    # sample-specific image context: swapping clip features between the two
    # samples (all else equal) must change each sample's output
    lat2 = np.concatenate([lat[:1], lat[:1]])
    same = O.step(lat2, np.array([t[0], t[0]]), np.concatenate([ctx[:1], ctx[:1]]), mw, H, clip=clip)
    assert np.max(np.abs(same[0] - same[1])) > 1e-6, "samples with different clip features agree"
    # block order matters, and step follows the list order
    rev = dict(mw); rev["blocks"] = mw["blocks"][::-1]
    _close(O.step(lat, t, ctx, rev, H, clip=clip), _torch_step(lat, t, ctx, rev, H, clip=clip),
           1e-9, "reversed blocks vs torch composition")
    # T2V (16 channels, no image context) against the same composition
    mw16 = dict(mw); mw16["patch_w"] = mw["patch_w"][:, :64]
    mw16["blocks"] = [{k: v for k, v in w.items() if "img" not in k} for w in mw["blocks"]]
    _close(O.step(lat[:, :16], t, ctx, mw16, H), _torch_step(lat[:, :16], t, ctx, mw16, H),
           1e-9, "T2V step vs torch composition")


# ---------------------------------------------------------------- sampler
def pin_sampler(O):
    """Euler along the flow x_tau = tau x1 + (1 - tau) x0 ([Note, 训练方法]):
    the exact conditional velocity (x1 - x)/(1 - tau), evaluated at the model
    timestep t = 1000 tau, keeps Euler on the straight line, so N steps land
    on x1 for every N; a constant velocity c moves x0 by exactly c; the I2V
    channels beyond the first 16 never move; the guided field of a
    conditional / unconditional pair lands on x1u + s (x1c - x1u)."""
    r = _rng(40)
    for cin in (16, 36):
        x0 = r.standard_normal((1, cin, 2, 4, 6))
        x1 = r.standard_normal((1, 16, 2, 4, 6))
        vel = lambda x, t: (x1 - x[:, :16]) / (1.0 - t[:, None, None, None, None] / 1000.0)
        for n in (1, 3, 50):
            with np.errstate(divide="ignore", invalid="ignore"):   # a wrong time grid may hit tau = 1
                out = O.sample(x0, n, vel)
            _close(out[:, :16], x1, 1e-10, f"straight-path Euler, N={n}, Cin={cin}")
            assert np.array_equal(out[:, 16:], x0[:, 16:]), "I2V channels moved"
        c = r.standard_normal((1, 16, 2, 4, 6))
        out = O.sample(x0, 7, lambda x, t: np.broadcast_to(c, (1,) + c.shape[1:]))
        _close(out[:, :16], x0[:, :16] + c, 1e-12, "constant velocity")
    tau, tm = O.sampler_times(4)
    _close(tau, [0, 0.25, 0.5, 0.75, 1.0], 0, "tau grid")
    _close(tm, [0, 250, 500, 750], 0, "model timesteps")
    # guidance: closed forms of the combine, then the guided straight path
    vc, vu = r.standard_normal(5), r.standard_normal(5)
    _close(O.cfg_combine(vc, vu, 0.0), vu, 0, "guidance 0")
    _close(O.cfg_combine(vc, vu, 1.0), vc, 1e-15, "guidance 1")
    _close(O.cfg_combine(vc, vu, 5.0), 5 * vc - 4 * vu, 1e-12, "guidance 5")
    x0 = np.repeat(r.standard_normal((1, 16, 2, 4, 6)), 2, axis=0)
    x1c, x1u = r.standard_normal((16, 2, 4, 6)), r.standard_normal((16, 2, 4, 6))

    def pair(x, t):
        den = 1.0 - t[0] / 1000.0
        return np.stack([(x1c - x[0, :16]) / den, (x1u - x[1, :16]) / den])

    for s in (0.0, 1.0, 5.0):
        out = O.sample(x0, 10, pair, guidance=s)
        _close(out[0], x1u + s * (x1c - x1u), 1e-10, f"guided path, s={s}")
        assert np.array_equal(out[0], out[1]), "guided pair diverged"


def pin_text_kv(O):
    """The cached cross-attention keys / values are the K / V halves of the
    block's KV projection (torch Linear), and cross_attention with them is the
    block's cross-attention (multihead attention over those K, V)."""
    r = _rng(41)
    d, Lc, Li, L, H = 32, 6, 5, 9, 2
    w = {"ca_wkv": r.standard_normal((2 * d, d)) * 0.2, "ca_bkv": r.standard_normal(2 * d) * 0.2,
         "ca_wkv_img": r.standard_normal((2 * d, d)) * 0.2, "ca_bkv_img": r.standard_normal(2 * d) * 0.2}
    ctx, img = r.standard_normal((Lc, d)), r.standard_normal((Li, d))
    k, v, ki, vi = O.text_kv(ctx, w, img)
    kv = TF.linear(_t(ctx), _t(w["ca_wkv"]), _t(w["ca_bkv"])).numpy()
    _close(k, kv[:, :d], 1e-12, "text K")
    _close(v, kv[:, d:], 1e-12, "text V")
    kvi = TF.linear(_t(img), _t(w["ca_wkv_img"]), _t(w["ca_bkv_img"])).numpy()
    _close(ki, kvi[:, :d], 1e-12, "image K")
    _close(vi, kvi[:, d:], 1e-12, "image V")
    wq, bq = r.standard_normal((d, d)) * 0.2, r.standard_normal(d) * 0.2
    wo, bo = r.standard_normal((d, d)) * 0.2, r.standard_normal(d) * 0.2
    xq = r.standard_normal((L, d))
    ca = O.cross_attention(xq, ctx, wq, bq, w["ca_wkv"], w["ca_bkv"], wo, bo, H)
    q = O.linear(O.layer_norm(xq), wq, bq)
    _close(ca, O.linear(O.multihead(q, k, v, H), wo, bo), 1e-12, "CA from cached K/V")


# ---------------------------------------------------------------- FP8 GEMM
def pin_fp8(O):
    """OCP E4M3 value set and rounding against torch's float8_e4m3fn (decode of
    every code, conversion of random values), ties to the even code, the
    per-token / per-tensor scale mapping the largest magnitude to 448, the
    rounding error bound, and linear_fp8 on operands already on the E4M3 grid
    against the exact product."""
    vals = O.e4m3_values()
    codes = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    _close(vals, codes.numpy(), 0, "E4M3 value set")
    assert vals[-1] == 448.0 and vals[1] == 2.0 ** -9
    _close(O.e4m3_round(vals), vals, 0, "idempotent on representable values")
    _close(O.e4m3_round(-vals), -vals, 0, "sign")
    mids = (vals[:-1] + vals[1:]) / 2
    even = np.where(np.arange(len(mids)) % 2 == 0, vals[:-1], vals[1:])
    _close(O.e4m3_round(mids), even, 0, "ties to the even code")
    r = _rng(50)
    x = np.clip(r.standard_normal(20000) * 40, -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    _close(O.e4m3_round(x.astype(np.float64)), ref, 0, "vs torch float8_e4m3fn")
    # per-token quantisation: the row max maps to 448, error within half a step
    xr = (r.standard_normal((7, 300)) * np.array([1e-3, 1, 10, 100, 0.5, 3, 1e4])[:, None]).astype(np.float32)
    xr[3] = 0.0
    q, s = O.quantize_rows_fp8(xr)
    for i in range(7):
        if i == 3:
            assert s[i] == 1.0 and not q[i].any(), "zero row"
            continue
        assert np.max(np.abs(q[i])) == 448.0, ("row max", i)
        v = xr[i].astype(np.float64) / s[i]
        # half the E4M3 spacing at |v| (relative 2^-4 for normals, 2^-10 absolute below 2^-6)
        bound = np.maximum(np.abs(v) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6)
        assert np.all(np.abs(v - q[i]) <= bound), ("rounding bound", i)
    qw, sw = O.quantize_tensor_fp8(xr)
    assert np.max(np.abs(qw)) == 448.0 and np.isclose(sw, np.max(np.abs(xr)) / 448.0, rtol=1e-7)
    # operands already on the grid (q * power-of-two scales) -> the exact product
    qa = vals[r.integers(0, 127, (5, 64))] * np.sign(r.standard_normal((5, 64)))
    qa[:, 0] = 448.0                                      # each row's max is 448
    qb = vals[r.integers(0, 127, (9, 64))] * np.sign(r.standard_normal((9, 64)))
    qb[0, 0] = -448.0
    xa = (qa * 0.25).astype(np.float32)                   # scale 1/4 per row
    wb = (qb * 2.0).astype(np.float32)                    # scale 2 for the tensor
    bias = r.standard_normal(9)
    _close(O.linear_fp8(xa, wb, bias), xa.astype(np.float64) @ wb.astype(np.float64).T + bias, 1e-9,
           "linear_fp8 on grid operands")


def pin_fp8_block(O):
    """The FP8 switch of the block touches only the six Linear layers: with the
    quantisers replaced by the identity (scale 1) the FP8 block equals the
    exact block bit for bit; with real E4M3 quantisation the block update stays
    within a few percent of the exact one."""
    r = _rng(51)
    d, F, H, L, Lc = 64, 128, 2, 20, 6
    w = {"sa_wqkv": r.standard_normal((3 * d, d)) * 0.1, "sa_bqkv": r.standard_normal(3 * d) * 0.02,
         "sa_wo": r.standard_normal((d, d)) * 0.1, "sa_bo": r.standard_normal(d) * 0.02,
         "ca_wq": r.standard_normal((d, d)) * 0.1, "ca_bq": r.standard_normal(d) * 0.02,
         "ca_wkv": r.standard_normal((2 * d, d)) * 0.1, "ca_bkv": r.standard_normal(2 * d) * 0.02,
         "ca_wo": r.standard_normal((d, d)) * 0.1, "ca_bo": r.standard_normal(d) * 0.02,
         "ffn_w1": r.standard_normal((F, d)) * 0.1, "ffn_b1": r.standard_normal(F) * 0.02,
         "ffn_w2": r.standard_normal((d, F)) * 0.1, "ffn_b2": r.standard_normal(d) * 0.02,
         "mod_bias": r.standard_normal(6 * d) * 0.02}
    x, m, ctx = r.standard_normal((1, L, d)), r.standard_normal((1, 6 * d)) * 0.3, r.standard_normal((1, Lc, d))
    exact = O.block(x, m, w, ctx, H)
    qr, qt, br = O.quantize_rows_fp8, O.quantize_tensor_fp8, O.bf16_round
    seen_w, seen_x = [], []
    try:
        def fake_rows(a):
            seen_x.append(np.shape(a))
            return np.asarray(a, np.float64), np.ones(np.shape(a)[0])

        def fake_tensor(a):
            seen_w.append(np.shape(a))
            return np.asarray(a, np.float64), 1.0
        O.quantize_rows_fp8, O.quantize_tensor_fp8 = fake_rows, fake_tensor
        O.bf16_round = lambda a: np.asarray(a, np.float64)
        same = O.block(x, m, w, ctx, H, fp8=True)
    finally:
        O.quantize_rows_fp8, O.quantize_tensor_fp8, O.bf16_round = qr, qt, br
    assert np.array_equal(same, exact), "fp8 switch changed more than the Linear layers"
    # six weight tensors, each quantised whole (Wqkv as one [3d, d] tensor)
    assert sorted(seen_w) == sorted([(3 * d, d), (d, d), (d, d), (d, d), (F, d), (d, F)]), seen_w
    # activations: h1 for Q, K, V; o; LN(x) for the CA query; CA o; h2; GELU(u)
    assert sorted(seen_x) == sorted([(L, d)] * 7 + [(L, F)]), seen_x
    q8 = O.block(x, m, w, ctx, H, fp8=True)
    upd, upd8 = exact - x, q8 - x
    rel = np.abs(upd8 - upd).sum() / np.abs(upd).sum()
    assert 1e-4 < rel < 0.05, rel
    # the activation enters the quantiser as bf16 (R23): x and its bf16 rounding agree
    xa = r.standard_normal((5, d))
    assert np.array_equal(O.linear_fp8(xa, w["ffn_w1"], w["ffn_b1"]),
                          O.linear_fp8(O.bf16_round(xa), w["ffn_w1"], w["ffn_b1"]))
    assert not np.array_equal(O.linear_fp8(xa, w["ffn_w1"], w["ffn_b1"]),
                              O.linear_fp8(xa.astype(np.float32).astype(np.float64) * (1 + 2.0 ** -7),
                                           w["ffn_w1"], w["ffn_b1"]))


def pin_bf16_round(O):
    """bf16 rounding against torch's float32 -> bfloat16 conversion (a library
    routine), including exact ties, and its closed-form error bound."""
    import torch
    r = _rng(52)
    x = np.concatenate([r.standard_normal(4000) * 10.0 ** r.integers(-6, 6, 4000),
                        # ties: a bf16 value plus half its unit in the last place
                        (1.0 + np.arange(1, 200) * 2.0 ** -7) + 2.0 ** -8,
                        -(1.0 + np.arange(1, 200) * 2.0 ** -7) - 2.0 ** -8, [0.0, -0.0, 65504.0]])
    got = O.bf16_round(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, ref)
    x32 = x.astype(np.float32).astype(np.float64)
    assert np.all(np.abs(got - x32) <= np.abs(x32) * 2.0 ** -8)


def pin_fp8_step(O):
    """The step's FP8 switch reaches every block and nothing else: with the
    quantisers replaced by the identity it equals the exact step bit for bit,
    and the weight quantiser sees each block's six weights (two blocks)."""
    r = _rng(53)
    d, F, H, Lc, nb = 64, 128, 2, 5, 2
    def blk():
        return {"sa_wqkv": r.standard_normal((3 * d, d)) * 0.1, "sa_bqkv": r.standard_normal(3 * d) * 0.02,
                "sa_wo": r.standard_normal((d, d)) * 0.1, "sa_bo": r.standard_normal(d) * 0.02,
                "ca_wq": r.standard_normal((d, d)) * 0.1, "ca_bq": r.standard_normal(d) * 0.02,
                "ca_wkv": r.standard_normal((2 * d, d)) * 0.1, "ca_bkv": r.standard_normal(2 * d) * 0.02,
                "ca_wo": r.standard_normal((d, d)) * 0.1, "ca_bo": r.standard_normal(d) * 0.02,
                "ffn_w1": r.standard_normal((F, d)) * 0.1, "ffn_b1": r.standard_normal(F) * 0.02,
                "ffn_w2": r.standard_normal((d, F)) * 0.1, "ffn_b2": r.standard_normal(d) * 0.02,
                "mod_bias": r.standard_normal(6 * d) * 0.02}
    mw = {"patch_w": r.standard_normal((d, 64)) * 0.1, "patch_b": r.standard_normal(d) * 0.02,
          "tmlp": {"w1": r.standard_normal((d, 256)) * 0.05, "b1": r.standard_normal(d) * 0.02,
                   "w2": r.standard_normal((6 * d, d)) * 0.05, "b2": r.standard_normal(6 * d) * 0.02},
          "head_w": r.standard_normal((64, d)) * 0.1, "head_b": r.standard_normal(64) * 0.02,
          "blocks": [blk() for _ in range(nb)]}
    lat = r.standard_normal((1, 16, 2, 4, 6))
    t = np.array([500.0])
    ctx = r.standard_normal((1, Lc, d))
    exact = O.step(lat, t, ctx, mw, H)
    qr, qt, br = O.quantize_rows_fp8, O.quantize_tensor_fp8, O.bf16_round
    seen = []
    try:
        O.quantize_rows_fp8 = lambda a: (np.asarray(a, np.float64), np.ones(np.shape(a)[0]))

        def fake_tensor(a):
            seen.append(np.shape(a))
            return np.asarray(a, np.float64), 1.0
        O.quantize_tensor_fp8 = fake_tensor
        O.bf16_round = lambda a: np.asarray(a, np.float64)
        same = O.step(lat, t, ctx, mw, H, fp8=True)
    finally:
        O.quantize_rows_fp8, O.quantize_tensor_fp8, O.bf16_round = qr, qt, br
    assert np.array_equal(same, exact), "fp8 step switch changed more than the blocks' Linear layers"
    assert len(seen) == 6 * nb, seen
    q8 = O.step(lat, t, ctx, mw, H, fp8=True)
    assert not np.array_equal(q8, exact)



# ---------------------------------------------------------------- 8-bit attention
def pin_int8_quant(O):
    """Symmetric Int8 quantisation: hand-computed codes (ties to even), the
    group max mapping to +-127, the half-step error bound, the all-zero group,
    and the block / channel groupings of K and V (distinct magnitudes per
    block or channel, a ragged last K block)."""
    x = np.array([127.0, 0.5, 1.5, 2.5, -3.5, 126.5, -127.0, 63.25], np.float32)
    q, s = O.quantize_int8(x)                       # amax 127: inv = scale = 1
    _close(q, [127, 0, 2, 2, -4, 126, -127, 63], 0, "Int8 codes, ties to even")
    assert s == 1.0
    q, s = O.quantize_int8(np.zeros(5, np.float32))
    assert s == 1.0 and not q.any(), "zero group"
    r = _rng(60)
    for mag in (1e-3, 1.0, 37.0, 3e4):
        x = (r.standard_normal(500) * mag).astype(np.float32)
        q, s = O.quantize_int8(x)
        assert np.max(np.abs(q)) == 127 and np.all(q == np.round(q))
        assert np.isclose(s, np.max(np.abs(x)) / 127.0, rtol=1e-6)
        assert np.all(np.abs(x / s - q) <= 0.5 + 1e-5), ("half-step bound", mag)
    # per-token q
    qm = (r.standard_normal((4, 16)) * np.array([[1e-2], [1.0], [50.0], [0.0]])).astype(np.float32)
    qc, qs = O.quantize_q_int8(qm)
    for i in range(3):
        assert np.isclose(qs[i], np.max(np.abs(qm[i])) / 127.0, rtol=1e-6) and np.max(np.abs(qc[i])) == 127
    assert qs[3] == 1.0 and not qc[3].any()
    # per-64-key-block k: block b has magnitude 10^b; key 149 (ragged block 2) is the largest
    k = np.concatenate([r.standard_normal((64, 16)), r.standard_normal((64, 16)) * 10,
                        r.standard_normal((22, 16)) * 100]).astype(np.float32)
    k[149, 3] = 1e4
    kc, ks = O.quantize_k_int8(k)
    assert ks.shape == (3,)
    for b, (lo, hi) in enumerate([(0, 64), (64, 128), (128, 150)]):
        assert np.isclose(ks[b], np.max(np.abs(k[lo:hi])) / 127.0, rtol=1e-6), ("block scale", b)
        assert np.max(np.abs(kc[lo:hi])) == 127
    assert kc[149, 3] == 127
    # per-channel v: column c has magnitude 4^c
    v = (r.standard_normal((90, 6)) * 4.0 ** np.arange(6)).astype(np.float32)
    vc, vs = O.quantize_v_fp8(v)
    assert vc.shape == v.shape and vs.shape == (6,)
    for c in range(6):
        assert np.isclose(vs[c], np.max(np.abs(v[:, c])) / 448.0, rtol=1e-6) and np.max(np.abs(vc[:, c])) == 448


def _brute_attention_8bit(q, k, v, q_scaled):
    """The 8-bit attention written out with loops: Int8 by Python's round
    (half to even) of float32 products, E4M3 by torch's float8_e4m3fn."""
    f32 = np.float32
    Lq, hd = q.shape
    Lk = k.shape[0]

    def i8(vals):
        amax = max(abs(float(t)) for t in vals)
        if amax == 0:
            return [0] * len(vals), 1.0
        inv, s = f32(127) / f32(amax), f32(amax) / f32(127)
        return [round(float(min(max(f32(t) * inv, f32(-127)), f32(127)))) for t in vals], float(s)

    def e4m3(t):
        return float(torch.tensor([float(t)], dtype=torch.float64).to(torch.float8_e4m3fn).to(torch.float64)[0])

    qc, qs = [], []
    for i in range(Lq):
        c, s = i8(list(q[i]))
        qc.append(c)
        qs.append(s)
    kc, ks = [None] * Lk, [0.0] * Lk
    for b0 in range(0, Lk, 64):
        rows = list(range(b0, min(b0 + 64, Lk)))
        c, s = i8([k[j][d] for j in rows for d in range(hd)])
        for n, j in enumerate(rows):
            kc[j], ks[j] = c[n * hd:(n + 1) * hd], s
    vc, vs = [[0.0] * hd for _ in range(Lk)], [0.0] * hd
    for d in range(hd):
        amax = max(abs(float(v[j][d])) for j in range(Lk))
        inv, s = (f32(448) / f32(amax), f32(amax) / f32(448)) if amax else (f32(1), f32(1))
        for j in range(Lk):
            vc[j][d] = e4m3(min(max(f32(v[j][d]) * inv, f32(-448)), f32(448)))
        vs[d] = float(s)
    out = np.zeros((Lq, hd))
    for i in range(Lq):
        S = [sum(qc[i][d] * kc[j][d] for d in range(hd)) * qs[i] * ks[j] for j in range(Lk)]
        mx = max(S)
        if q_scaled:
            p = [e4m3(128.0 * 2.0 ** (t - mx)) for t in S]
        else:
            p = [e4m3(128.0 * math.exp((t - mx) / math.sqrt(hd))) for t in S]
        tot = sum(p)
        for d in range(hd):
            out[i, d] = vs[d] * sum(p[j] * vc[j][d] for j in range(Lk)) / tot
    return out


def pin_attention_8bit(O):
    """8-bit attention against the loop version above (two K blocks, the
    second ragged; plain and pre-scaled q), and two closed forms: equal keys
    give the mean of v; one key far above the rest gives that key's v (the
    others' probabilities round to zero).  Inputs on the Int8 / E4M3 grids
    with scale 1 make both closed forms exact."""
    r = _rng(61)
    for q_scaled, mag in ((False, 1.0), (True, 0.3)):
        q = O.bf16_round(r.standard_normal((3, 16)) * 2.0)
        k = O.bf16_round(r.standard_normal((70, 16)) * np.where(np.arange(70) < 64, 1.0, 3.0)[:, None])
        v = O.bf16_round(r.standard_normal((70, 16)))
        q = O.bf16_round(q * mag)
        _close(O.attention_8bit(q, k, v, q_scaled), _brute_attention_8bit(q, k, v, q_scaled), 1e-12,
               f"8-bit attention vs loops (q_scaled={q_scaled})")
    vals = O.e4m3_values()
    v = vals[r.integers(0, 127, (40, 8))] * np.sign(r.standard_normal((40, 8)))
    v[5] = 448.0                                          # every channel's max is 448: scale 1
    q = np.round(r.standard_normal((4, 8)) * 40)
    q[:, 0] = 127.0                                       # per-token scale 1
    k = np.tile(np.round(r.standard_normal((1, 8)) * 40), (40, 1))
    k[:, 1] = 127.0                                       # equal keys, block scale 1
    for q_scaled in (False, True):
        _close(O.attention_8bit(q, k, v, q_scaled), np.tile(v.mean(axis=0), (4, 1)), 1e-12,
               "equal keys: mean of v")
    k = np.zeros((40, 8))
    k[:, 0] = -127.0
    k[17, 0] = 127.0                                      # key 17 scores 2 * 127^2 above the rest
    for q_scaled in (False, True):
        q1 = np.zeros((4, 8))
        q1[:, 0] = 127.0
        _close(O.attention_8bit(q1, k, v, q_scaled), np.tile(v[17], (4, 1)), 0, "one dominant key")


def pin_attn8_block(O):
    """The block's 8-bit attention switch touches only the self-attention:
    with the 8-bit attention replaced by the exact one (and the bf16 rounding
    by the identity) the block equals the exact block bit for bit, with one
    call per sample (also with FP8 Linear layers).  The real 8-bit block
    update stays within a few percent of the exact one."""
    r = _rng(62)
    d, F, H, L, Lc = 256, 128, 2, 70, 6
    w = {"sa_wqkv": r.standard_normal((3 * d, d)) * 0.06, "sa_bqkv": r.standard_normal(3 * d) * 0.02,
         "sa_wo": r.standard_normal((d, d)) * 0.06, "sa_bo": r.standard_normal(d) * 0.02,
         "ca_wq": r.standard_normal((d, d)) * 0.06, "ca_bq": r.standard_normal(d) * 0.02,
         "ca_wkv": r.standard_normal((2 * d, d)) * 0.06, "ca_bkv": r.standard_normal(2 * d) * 0.02,
         "ca_wo": r.standard_normal((d, d)) * 0.06, "ca_bo": r.standard_normal(d) * 0.02,
         "ffn_w1": r.standard_normal((F, d)) * 0.06, "ffn_b1": r.standard_normal(F) * 0.02,
         "ffn_w2": r.standard_normal((d, F)) * 0.06, "ffn_b2": r.standard_normal(d) * 0.02,
         "mod_bias": r.standard_normal(6 * d) * 0.02}
    x, m, ctx = r.standard_normal((2, L, d)), r.standard_normal((2, 6 * d)) * 0.3, r.standard_normal((2, Lc, d))
    exact = O.block(x, m, w, ctx, H)
    mh8, br = O.multihead_8bit, O.bf16_round
    calls = []

    def fake(q, k, v, heads, q_scaled=False):
        calls.append((np.shape(q), np.shape(k)))
        return O.multihead(q, k, v, heads)
    try:
        O.multihead_8bit = fake
        O.bf16_round = lambda a: np.asarray(a, np.float64)
        same = O.block(x, m, w, ctx, H, attn8=True)
    finally:
        O.multihead_8bit, O.bf16_round = mh8, br
    assert np.array_equal(same, exact), "attn8 switch changed more than the self-attention"
    assert len(calls) == 2 and calls[0] == ((L, d), (L, d)), calls
    # what reaches the 8-bit attention holds bf16 values (R26)
    seen = []
    try:
        def spy(q, k, v, heads, q_scaled=False):
            seen.append(all(np.array_equal(br(a), np.asarray(a, np.float64)) for a in (q, k, v)))
            return mh8(q, k, v, heads, q_scaled)
        O.multihead_8bit = spy
        O.block(x[:1], m[:1], w, ctx[:1], H, attn8=True)
    finally:
        O.multihead_8bit = mh8
    assert seen == [True], seen
    # with FP8 Linear layers the switch reaches the self-attention too
    calls.clear()
    try:
        O.multihead_8bit = fake
        O.block(x, m, w, ctx, H, fp8=True, attn8=True)
    finally:
        O.multihead_8bit = mh8
    assert len(calls) == 2, calls
    q8 = O.block(x, m, w, ctx, H, attn8=True)
    upd, upd8 = exact - x, q8 - x
    rel = np.abs(upd8 - upd).sum() / np.abs(upd).sum()
    assert 1e-4 < rel < 0.06, rel


def pin_attn8_step(O):
    """The step's 8-bit attention switch reaches the self-attention of every
    block (two blocks, one sample) and nothing else: with the 8-bit attention
    replaced by the exact one the step equals the exact step bit for bit."""
    r = _rng(63)
    d, F, H, Lc, nb = 64, 128, 2, 5, 2

    def blk():
        return {"sa_wqkv": r.standard_normal((3 * d, d)) * 0.1, "sa_bqkv": r.standard_normal(3 * d) * 0.02,
                "sa_wo": r.standard_normal((d, d)) * 0.1, "sa_bo": r.standard_normal(d) * 0.02,
                "ca_wq": r.standard_normal((d, d)) * 0.1, "ca_bq": r.standard_normal(d) * 0.02,
                "ca_wkv": r.standard_normal((2 * d, d)) * 0.1, "ca_bkv": r.standard_normal(2 * d) * 0.02,
                "ca_wo": r.standard_normal((d, d)) * 0.1, "ca_bo": r.standard_normal(d) * 0.02,
                "ffn_w1": r.standard_normal((F, d)) * 0.1, "ffn_b1": r.standard_normal(F) * 0.02,
                "ffn_w2": r.standard_normal((d, F)) * 0.1, "ffn_b2": r.standard_normal(d) * 0.02,
                "mod_bias": r.standard_normal(6 * d) * 0.02}
    mw = {"patch_w": r.standard_normal((d, 64)) * 0.1, "patch_b": r.standard_normal(d) * 0.02,
          "tmlp": {"w1": r.standard_normal((d, 256)) * 0.05, "b1": r.standard_normal(d) * 0.02,
                   "w2": r.standard_normal((6 * d, d)) * 0.05, "b2": r.standard_normal(6 * d) * 0.02},
          "head_w": r.standard_normal((64, d)) * 0.1, "head_b": r.standard_normal(64) * 0.02,
          "blocks": [blk() for _ in range(nb)]}
    lat = r.standard_normal((1, 16, 2, 4, 6))
    t = np.array([500.0])
    ctx = r.standard_normal((1, Lc, d))
    exact = O.step(lat, t, ctx, mw, H)
    mh8, br = O.multihead_8bit, O.bf16_round
    calls = []
    try:
        def fake(q, k, v, heads, q_scaled=False):
            calls.append(np.shape(q))
            return O.multihead(q, k, v, heads)
        O.multihead_8bit = fake
        O.bf16_round = lambda a: np.asarray(a, np.float64)
        same = O.step(lat, t, ctx, mw, H, attn8=True)
    finally:
        O.multihead_8bit, O.bf16_round = mh8, br
    assert np.array_equal(same, exact), "attn8 step switch changed more than the self-attention"
    assert len(calls) == nb, calls
