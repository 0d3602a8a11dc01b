"""8-bit attention (Int8 Q K^T, E4M3 P V): the HIP quantisers against the
oracle's bit for bit, and the attention against the oracle's 8-bit attention,
through the C ABI (wan_attention_8bit_quantize / _q_fwd / _fwd).

The kernel and the oracle round the same probabilities to E4M3 against
different maxima (the kernel keeps a running max that it raises only when a
probability would pass 448; the oracle uses the row max), so their results
differ by an independent draw of the same rounding noise that separates the
oracle from exact attention.  The bar: mean |kernel - oracle| at most 1.25x
mean |oracle - exact|, and max |kernel - oracle| at most the larger of 3e-2
and max |oracle - exact|.  (A CPU replay of the kernel's algorithm gives
ratios 0.19 - 0.81 for the mean and 0.37 - 0.77 for the max on these
inputs.)  Beside it, a fixed bar that does not lean on the oracle: the
kernel's mean relative error against exact attention (float64) at most 8e-2.
E4M3 keeps 3 mantissa bits, and on these inputs the oracle's own 8-bit
rounding gives 1.8e-2 - 3.9e-2 (computed on the CPU); the bar is twice the
largest of those, where an attention that drops the softmax (mean of V)
lands at 0.5 or more."""
import numpy as np
import pytest

import oracle.wan_oracle as O
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

C_LOG2 = np.log2(np.e) / np.sqrt(128.0)
ATTN8_MEAN_REL = 8e-2    # fixed bar against exact attention (module docstring)


def _rup(v, a):
    return (v + a - 1) // a * a


def _upload(q, k, v):
    from tests.gpu_util import DEV
    B, Lq, D = q.shape
    Lk = k.shape[1]
    Lkp = _rup(Lk, 64)
    vt = np.zeros((D, B * Lkp), np.float32)
    for b in range(B):
        vt[:, b * Lkp:b * Lkp + Lk] = v[b].T
    tq = torch.from_numpy(q.reshape(B * Lq, D)).to(torch.bfloat16).to(DEV)
    tk = torch.from_numpy(k.reshape(B * Lk, D)).to(torch.bfloat16).to(DEV)
    tv = torch.from_numpy(vt).to(torch.bfloat16).to(DEV)
    return tq, tk, tv, Lkp


def _attn8_gpu(q, k, v, H, q_scaled=False):
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import DEV
    B, Lq, D = q.shape
    Lk = k.shape[1]
    tq, tk, tv, Lkp = _upload(q, k, v)
    to = torch.empty((B * Lq, D), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(W.attention_8bit_workspace_bytes(B, H, Lq, Lk), dtype=torch.uint8, device=DEV)
    W.attention_8bit_fwd(tq, D, tk, D, tv, B * Lkp, Lkp, to, D, B, H, Lq, Lk, ws, q_scaled=q_scaled)
    torch.cuda.synchronize()
    return to.float().cpu().numpy().reshape(B, Lq, D)


def _oracle8(q, k, v, H, q_scaled=False):
    return np.stack([O.multihead_8bit(q[b], k[b], v[b], H, q_scaled) for b in range(q.shape[0])])


def _exact(q, k, v, H):
    return np.stack([O.multihead(q[b], k[b], v[b], H) for b in range(q.shape[0])])


def _assert_attn8(g, o8, ex, what):
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    ek, eq = np.abs(g - o8), np.abs(o8 - ex)
    bar_max = max(3e-2, float(eq.max()))
    print(f"  {what}: |kernel - oracle| max {ek.max():.4f} mean {ek.mean():.5f}; "
          f"|oracle - exact| max {eq.max():.4f} mean {eq.mean():.5f}", flush=True)
    assert ek.max() <= bar_max, f"{what}: max {ek.max():.4f} > {bar_max:.4f}"
    assert ek.mean() <= 1.25 * eq.mean(), f"{what}: mean {ek.mean():.5f} > 1.25 x {eq.mean():.5f}"
    rel = float(np.abs(g - ex).sum() / max(float(np.abs(ex).sum()), 1e-30))
    assert rel <= ATTN8_MEAN_REL, f"{what}: mean-rel against exact {rel:.4f} > {ATTN8_MEAN_REL}"


QUANT_CASES = [  # B, H, Lq, Lk
    (1, 1, 1, 1), (2, 2, 300, 200), (1, 3, 70, 64), (2, 1, 40, 130),
]


@pytest.mark.parametrize("B,H,Lq,Lk", QUANT_CASES)
def test_attn8_quantisers_bit_exact(B, H, Lq, Lk):
    """Int8 codes of q (per token) and k (per 64-key block), E4M3 codes of
    V^T (per channel), their scales, and the zero padding of V^T: equal to
    the oracle's."""
    print(f"attn8 quantisers B={B} H={H} Lq={Lq} Lk={Lk}", flush=True)
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import DEV
    q, k, v = synth.attention_inputs(11, B, H, Lq, Lk, qk_std=1.5)
    q[0, 0, :128] = 0.0                               # an all-zero group: scale 1, codes 0
    D, nkb = H * 128, _rup(Lk, 64) // 64
    tq, tk, tv, Lkp = _upload(q, k, v)
    q8 = torch.empty((B * Lq, D), dtype=torch.int8, device=DEV)
    qs = torch.empty((B * Lq, H), dtype=torch.float32, device=DEV)
    k8 = torch.empty((B * Lk, D), dtype=torch.int8, device=DEV)
    ks = torch.empty((B, H, nkb), dtype=torch.float32, device=DEV)
    v8t = torch.full((D, B * Lkp), 0x55, dtype=torch.uint8, device=DEV)   # padding must be written
    vs = torch.empty((B, D), dtype=torch.float32, device=DEV)
    W.attention_8bit_quantize(tq, D, tk, D, tv, B * Lkp, Lkp, B, H, Lq, Lk, q8, qs, k8, ks, v8t, vs)
    torch.cuda.synchronize()
    gq8 = q8.cpu().numpy().reshape(B, Lq, D).astype(np.float64)
    gk8 = k8.cpu().numpy().reshape(B, Lk, D).astype(np.float64)
    gqs, gks, gvs = qs.cpu().numpy().reshape(B, Lq, H), ks.cpu().numpy(), vs.cpu().numpy()
    gv8 = v8t.cpu().view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(B):
        for h in range(H):
            sl = slice(h * 128, (h + 1) * 128)
            c, s = O.quantize_q_int8(q[b][:, sl])
            assert np.array_equal(gq8[b][:, sl], c) and np.array_equal(gqs[b][:, h], s.astype(np.float32))
            c, s = O.quantize_k_int8(k[b][:, sl])
            assert np.array_equal(gk8[b][:, sl], c) and np.array_equal(gks[b, h], s.astype(np.float32))
            c, s = O.quantize_v_fp8(v[b][:, sl])
            seg = gv8[sl, b * Lkp:(b + 1) * Lkp]
            assert np.array_equal(seg[:, :Lk], c.T), ("E4M3 codes of V", b, h)
            assert not seg[:, Lk:].any(), "V^T padding columns not zero"
            assert np.array_equal(gvs[b, sl], s.astype(np.float32))
    assert gqs[0, 0, 0] == 1.0 and not gq8[0, 0, :128].any()


CASES = [  # B, H, Lq, Lk
    (1, 1, 1, 1), (1, 2, 200, 64), (2, 2, 300, 100), (1, 3, 513, 257), (2, 1, 256, 600),
    (1, 2, 70, 4), (1, 1, 1000, 1000),
    # key-tile counts 2 .. 5: every tail of the pipeline (unrolled by two)
    (1, 1, 64, 128), (1, 1, 96, 150), (1, 2, 100, 250), (1, 1, 40, 320),
]


@pytest.mark.parametrize("qk_std", [1.0, 2.0])
@pytest.mark.parametrize("B,H,Lq,Lk", CASES)
def test_attn8_parity(B, H, Lq, Lk, qk_std):
    print(f"attn8 B={B} H={H} Lq={Lq} Lk={Lk} qk_std={qk_std}", flush=True)
    q, k, v = synth.attention_inputs(12, B, H, Lq, Lk, qk_std=qk_std)
    g = _attn8_gpu(q, k, v, H)
    _assert_attn8(g, _oracle8(q, k, v, H), _exact(q, k, v, H), f"attn8 {B},{H},{Lq},{Lk}")


# keys whose logits jump far above everything before them: the running max is
# raised mid-stream (2nd tile, steady-state loop, last ragged tile) or set by
# the first tile with every later tile far below it
OUTLIER_CASES = [  # Lq, Lk, first outlier key, last outlier key + 1
    (200, 150, 64, 100), (300, 600, 300, 340), (130, 600, 580, 600), (100, 500, 0, 20),
]


@pytest.mark.parametrize("q_scaled", [False, True])
@pytest.mark.parametrize("Lq,Lk,k0,k1", OUTLIER_CASES)
def test_attn8_raises_running_max(Lq, Lk, k0, k1, q_scaled):
    print(f"attn8 outlier keys {k0}..{k1} of {Lk}, Lq={Lq}, q_scaled={q_scaled}", flush=True)
    q, k, v = synth.attention_inputs(13, 1, 2, Lq, Lk)
    k[:, k0:k1] *= 4.0
    if q_scaled:   # the kernel reads q' = bf16(q c): the same attention as that of q' / c
        q = synth.bf16_round(q * np.float32(C_LOG2))
    g = _attn8_gpu(q, k, v, 2, q_scaled)
    o8 = _oracle8(q, k, v, 2, q_scaled)
    ex = _exact(q.astype(np.float64) / (C_LOG2 if q_scaled else 1.0), k, v, 2)
    _assert_attn8(g, o8, ex, f"attn8 outliers {k0}..{k1}")
    # V = 1: the normaliser adds exactly the weights the PV products use
    g1 = _attn8_gpu(q, k, np.ones_like(v), 2, q_scaled)
    assert np.max(np.abs(g1 - 1.0)) <= 4e-3


def test_attn8_full_size_sampled():
    """The 1.3B 480P self-attention shape (B = 1, 12 heads, L = 32760) in the
    launch the block uses: 24 sampled queries of two heads against the oracle
    (which needs all keys of a head but only the sampled queries)."""
    print("attn8 full size 1 x 12 x 32760, sampled rows", flush=True)
    B, H, L = 1, 12, 32760
    q, k, v = synth.attention_inputs(14, B, H, L, L, qk_std=1.0)
    g = _attn8_gpu(q, k, v, H)
    rows = np.random.default_rng(5).choice(L, 24, replace=False)
    rows[:2] = [0, L - 1]
    for h in (0, 11):
        sl = slice(h * 128, (h + 1) * 128)
        o8 = O.attention_8bit(q[0][rows][:, sl], k[0][:, sl], v[0][:, sl])
        ex = O.attention(q[0][rows][:, sl], k[0][:, sl], v[0][:, sl])
        _assert_attn8(g[0][rows][:, sl], o8, ex, f"attn8 full size head {h}")


def test_attn8_q_fwd_matches_fused():
    """The attention on quantised copies (wan_attention_8bit_q_fwd) equals
    the fused entry point bit for bit."""
    print("attn8 q_fwd vs fused", flush=True)
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import DEV
    B, H, Lq, Lk = 2, 2, 300, 200
    q, k, v = synth.attention_inputs(15, B, H, Lq, Lk)
    D, nkb = H * 128, _rup(Lk, 64) // 64
    tq, tk, tv, Lkp = _upload(q, k, v)
    q8 = torch.empty((B * Lq, D), dtype=torch.int8, device=DEV)
    qs = torch.empty((B * Lq, H), dtype=torch.float32, device=DEV)
    k8 = torch.empty((B * Lk, D), dtype=torch.int8, device=DEV)
    ks = torch.empty((B, H, nkb), dtype=torch.float32, device=DEV)
    v8t = torch.empty((D, B * Lkp), dtype=torch.uint8, device=DEV)
    vs = torch.empty((B, D), dtype=torch.float32, device=DEV)
    W.attention_8bit_quantize(tq, D, tk, D, tv, B * Lkp, Lkp, B, H, Lq, Lk, q8, qs, k8, ks, v8t, vs)
    o1 = torch.empty((B * Lq, D), dtype=torch.bfloat16, device=DEV)
    W.attention_8bit_q_fwd(q8, qs, k8, ks, v8t, vs, o1, D, B, H, Lq, Lk)
    torch.cuda.synchronize()
    g = _attn8_gpu(q, k, v, H)
    assert np.array_equal(o1.float().cpu().numpy().reshape(B, Lq, D), g)
