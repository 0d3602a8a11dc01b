"""FP8 GEMM through the C ABI against the CPU oracle's E4M3 emulation:
quantisation codes and scales bit for bit (the codes are integers decided
in float32 on both sides), the GEMM in its three output modes over ragged
shapes and K of 1, 2, 3, 4, 24 and 40 64-deep chunks (K a multiple of 256 runs
the 128-deep tiling, the rest the 64-deep one), the two tilings against each
other bit for bit, and sampled rows at the full FFN up-projection shape."""
import numpy as np
import pytest

import oracle.wan_oracle as O
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _bf16(a):
    return synth.bf16_round(np.asarray(a, np.float32))


def _decode(q):
    """E4M3 bytes (torch uint8 on the device) -> float64 numpy."""
    return q.cpu().view(torch.float8_e4m3fn).to(torch.float64).numpy()


# Accumulation bound of the FP8 GEMM, relative to the sum of |products|: the
# E4M3 products are exact; one v_mfma_scale_f32_32x32x64_f8f6f4 sums its 64
# products to about 2^-15 of their absolute sum (measured on the chip: at most
# 2.9e-5 over 600k outputs), bounded here by 2^-13; the float32 accumulation
# across the K/64 instructions adds at most K 2^-24.
def _rel_bound(K):
    return 2.0 ** -13 + K * 2.0 ** -24


def _acc_bound(x, w, K):
    qx, sx = O.quantize_rows_fp8(x)
    qw, sw = O.quantize_tensor_fp8(w)
    return _rel_bound(K) * (np.abs(qx) @ np.abs(qw).T) * sx[:, None] * sw + 1e-7


def _quant_rows(x_np):
    import video_diffusion_transformer_block_amd as W
    M, K = x_np.shape
    x = torch.from_numpy(x_np).to(torch.bfloat16).cuda()
    q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    s = torch.empty(M, dtype=torch.float32, device="cuda")
    W.quantize_rows_fp8(x, q, s)
    return q, s


def _quant_tensor(w_np):
    import video_diffusion_transformer_block_amd as W
    w = torch.from_numpy(w_np).to(torch.bfloat16).cuda()
    q = torch.empty(w.shape, dtype=torch.uint8, device="cuda")
    s = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    W.quantize_tensor_fp8(w, q, s, ws)
    return q, s


def test_quantize_rows_and_tensor_bit_exact():
    print("fp8 quantisation", flush=True)
    rng = np.random.default_rng(60)
    x = _bf16(rng.standard_normal((300, 1536)) * np.exp(rng.uniform(-6, 6, (300, 1)))).astype(np.float32)
    x[7] = 0.0
    q, s = _quant_rows(x)
    torch.cuda.synchronize()
    qo, so = O.quantize_rows_fp8(x)
    assert np.array_equal(_decode(q), qo), "per-token codes"
    assert np.array_equal(s.cpu().numpy().astype(np.float64), so), "per-token scales"
    w = _bf16(rng.standard_normal((640, 1536)) * 0.02).astype(np.float32)
    qw, sw = _quant_tensor(w)
    torch.cuda.synchronize()
    qwo, swo = O.quantize_tensor_fp8(w)
    assert np.array_equal(_decode(qw), qwo), "per-tensor codes"
    assert float(sw.cpu()[0]) == swo, "per-tensor scale"


@pytest.mark.parametrize("M,N,K", [(300, 640, 1536), (130, 270, 256), (600, 513, 2560), (1, 256, 64),
                                   (257, 300, 128), (513, 512, 192)])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_linear_fp8_vs_oracle(M, N, K, mode):
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import assert_parity
    print(f"fp8 linear M={M} N={N} K={K} mode={mode}", flush=True)
    rng = np.random.default_rng(61 + M + N + K + mode)
    x = _bf16(rng.standard_normal((M, K))).astype(np.float32)
    w = _bf16(rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    b = _bf16(rng.standard_normal(N) * 0.02).astype(np.float32)
    qx, sx = _quant_rows(x)
    qw, sw = _quant_tensor(w)
    y = torch.empty((M, N), dtype=torch.float32 if mode == 1 else torch.bfloat16, device="cuda")
    bd = torch.from_numpy(b).to(torch.bfloat16).cuda()
    W.linear_fp8_fwd(qx, sx, qw, sw, bd, y, M, N, K, mode)
    torch.cuda.synchronize()
    g = y.float().cpu().numpy()
    o = O.linear_fp8(x, w, b)
    if mode == 2:
        o = O.gelu_tanh(o)
    acc = _acc_bound(x, w, K)
    if mode == 1:     # float32 output: only the float32 accumulation order differs
        excess = np.abs(g - o) - acc
    else:
        # bf16 output: the float32 value (within acc of the exact one; GELU's
        # slope is at most 1.13, its float32 evaluation good to a few ulp)
        # rounded to nearest with 8 significant bits, |bf16(v) - v| <= 2^-8 |v|
        dv = acc if mode == 0 else 1.13 * acc + 4e-6 * np.abs(o) + 1e-6
        excess = np.abs(g - o) - dv - 2.0 ** -8 * (np.abs(o) + dv)
        assert_parity(g, o, np.inf, 4e-3, f"fp8 linear mode {mode}")
    assert np.max(excess) <= 0, np.max(np.abs(g - o))


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_linear_fp8_k_tilings_agree_bitwise(mode):
    """K = 1536 runs the 128-deep K tiling, K = 1600 (the same operands with 64
    zero columns appended) the 64-deep one.  The zero columns add exact zero
    products and change neither quantisation scale, and both kernels sum the
    64-deep chunks in the same order, so the outputs are equal element for
    element."""
    import video_diffusion_transformer_block_amd as W
    M, N, K = 700, 520, 1536
    print(f"fp8 linear tilings M={M} N={N} K={K}/{K + 64} mode={mode}", flush=True)
    rng = np.random.default_rng(70 + mode)
    x = _bf16(rng.standard_normal((M, K))).astype(np.float32)
    w = _bf16(rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    b = torch.from_numpy(_bf16(rng.standard_normal(N) * 0.02).astype(np.float32)).to(torch.bfloat16).cuda()
    outs = []
    for pad in (0, 64):
        xp = np.pad(x, ((0, 0), (0, pad)))
        wp = np.pad(w, ((0, 0), (0, pad)))
        qx, sx = _quant_rows(xp)
        qw, sw = _quant_tensor(wp)
        y = torch.empty((M, N), dtype=torch.float32 if mode == 1 else torch.bfloat16, device="cuda")
        W.linear_fp8_fwd(qx, sx, qw, sw, b, y, M, N, K + pad, mode)
        torch.cuda.synchronize()
        outs.append(y.float().cpu().numpy())
    assert np.array_equal(outs[0], outs[1]), float(np.max(np.abs(outs[0] - outs[1])))


def test_linear_fp8_full_ffn_shape_sampled_rows():
    """The FFN up-projection of the 1.3B block (M = 32760, N = 8960, K = 1536):
    the whole GEMM on the GPU, 64 sampled rows in the oracle (per-token scales
    make rows independent)."""
    import video_diffusion_transformer_block_amd as W
    M, N, K = 32760, 8960, 1536
    print(f"fp8 linear full FFN shape {M}x{N}x{K}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(62)
    x = torch.randn((M, K), generator=g).to(torch.bfloat16)
    w = (torch.randn((N, K), generator=g) * 0.02).to(torch.bfloat16)
    b = (torch.randn(N, generator=g) * 0.02).to(torch.bfloat16)
    xd, wd, bd = x.cuda(), w.cuda(), b.cuda()
    qx = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    W.quantize_rows_fp8(xd, qx, sx)
    qw = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sw = torch.empty(1, dtype=torch.float32, device="cuda")
    W.quantize_tensor_fp8(wd, qw, sw, torch.empty(256, dtype=torch.uint8, device="cuda"))
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    W.linear_fp8_fwd(qx, sx, qw, sw, bd, y, M, N, K, 1)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(63).choice(M, 64, replace=False))
    rows[-1] = M - 1
    xs = x[rows].float().numpy()
    wf = w.float().numpy()
    qwo, swo = O.quantize_tensor_fp8(wf)
    qxo, sxo = O.quantize_rows_fp8(xs)
    o = (qxo @ qwo.T) * sxo[:, None] * swo + b.float().numpy()[None, :]
    gs = y[torch.from_numpy(rows).cuda()].cpu().numpy()
    bound = _rel_bound(K) * (np.abs(qxo) @ np.abs(qwo).T) * sxo[:, None] * swo + 1e-7
    assert np.max(np.abs(gs - o) - bound) <= 0, np.max(np.abs(gs - o))


# ---- FP8 block: wan_quantize_block_fp8 + wan_dit_block_fp8_fwd against the
# oracle's block with its six Linear layers in E4M3 (same weights, inputs).
FP8_BLOCKS = {
    "bf16-ragged-b2": synth.mini(11, "bf16-ragged-b2", dim=384, heads=3, ffn=640, n_blocks=1,
                                 lat_f=3, lat_h=20, lat_w=40, batch=2, text_len=40, kind="block"),
    "bf16-i2v": synth.mini(12, "bf16-i2v", dim=256, heads=2, ffn=512, n_blocks=1, lat_f=2,
                           lat_h=16, lat_w=24, batch=1, text_len=64, img_len=257, kind="block"),
    # short samples: a GEMM wavefront's 128 rows span all three (L = 25), so the
    # gated-residual epilogue takes each row's own gate.  (The five-sample L = 6
    # case runs in the bf16 block test only: over its 30 rows the max-abs
    # comparison with the FP8 effect is decided by single E4M3 code steps.)
    "bf16-b3-short": synth.mini(13, "bf16-b3-short", dim=256, heads=2, ffn=512, n_blocks=1,
                                lat_f=1, lat_h=10, lat_w=10, batch=3, text_len=40, kind="block"),
}


def _run_block_fp8(work, rows=None):
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import cfg_of, run_tmlp, up, up_block
    m = work.model
    cfg = cfg_of(work)
    inp = synth.workload_inputs(work)
    if work.batch > 2:   # distinct timesteps, so every sample has gates of its own
        inp["t"] = np.linspace(60.0, 940.0, work.batch).astype(np.float32)
    tw = synth.tmlp_weights(work)
    bw = synth.block_weights(work, 0)
    img = None
    if m.img_len:
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([2025, work.cid, 77])))
        img = synth.bf16_round(g.standard_normal((work.batch, m.img_len, m.dim), dtype=np.float32))
    twd = {k: up(v, m.dtype) for k, v in tw.items()}
    mod = run_tmlp(cfg, work, twd, up(inp["t"], "f32"))
    x = up(inp["x"], "f32")
    bwd = up_block(bw, m.dtype)
    desc = W.block_weights(bwd)
    qbuf = torch.empty(W.block_fp8_bytes(cfg), dtype=torch.uint8, device="cuda")
    W.quantize_block_fp8(cfg, desc, qbuf)
    # the six quantised weights are not read: pass their pointers as NULL
    desc8 = W.block_weights({k: v for k, v in bwd.items()
                             if k not in ("sa_wqkv", "sa_wo", "ca_wq", "ca_wo", "ffn_w1", "ffn_w2")})
    ws = torch.empty(W.block_fp8_workspace_bytes(cfg, work.batch, work.lat_f, work.Hp, work.Wp),
                     dtype=torch.uint8, device="cuda")
    W.dit_block_fp8_fwd(cfg, x, work.batch, work.lat_f, work.Hp, work.Wp, mod, desc8, qbuf,
                        up(inp["ctx"], m.dtype), up(img, m.dtype) if img is not None else None, ws)
    torch.cuda.synchronize()
    o_mod = O.tmlp(inp["t"], tw["w1"], tw["b1"], tw["w2"], tw["b2"])
    o_x = O.block(inp["x"], o_mod, bw, inp["ctx"], m.heads, m.eps, img=img, rows=rows, fp8=True)
    e_x = O.block(inp["x"], o_mod, bw, inp["ctx"], m.heads, m.eps, img=img, rows=rows)
    return inp["x"], x.cpu().numpy(), o_x, e_x, qbuf, bw


def _check_fp8_block(x0, g_x, o_x, e_x):
    """The block output to the usual bound (max-abs 3e-2, mean-rel 1e-2).  The
    block's update (x_out - x_in) is judged against the size of the FP8 effect
    itself: an E4M3 code is an integer decided from a bf16 activation, and the
    GPU's bf16 activations (attention with bf16 probabilities, float32
    LayerNorm and GELU) differ from the oracle's in the last bf16 place often
    enough that some codes move by one E4M3 step (6-12 %) -- deviations that
    two correct FP8 implementations show between each other.  The GPU update
    must sit within half the distance between the FP8 and the exact oracle
    block, i.e. decisively on the FP8 side."""
    from tests.gpu_util import assert_parity, metrics
    du, de = g_x - x0, o_x - x0
    dev = metrics(du, de)
    eff = metrics(e_x - x0, de)
    print("output", metrics(g_x, o_x), "update", dev, "fp8 effect", eff, flush=True)
    assert_parity(g_x, o_x, 3e-2, 1e-2, "fp8 block output")
    assert dev["mean_rel"] <= 0.5 * eff["mean_rel"], (dev, eff)
    assert dev["max_abs"] <= 0.75 * eff["max_abs"], (dev, eff)


@pytest.mark.parametrize("name", list(FP8_BLOCKS))
def test_block_fp8_mini(name):
    work = FP8_BLOCKS[name]
    print(f"fp8 block {name} L={work.L} d={work.model.dim}", flush=True)
    x0, g_x, o_x, e_x, qbuf, bw = _run_block_fp8(work)
    _check_fp8_block(x0, g_x, o_x, e_x)
    # the packed weights: the scales and codes of Wqkv (quantised whole) and FFN down
    q = qbuf.cpu()
    d, F = work.model.dim, work.model.ffn
    sc = q[:24].view(torch.float32).numpy()
    qo, so = O.quantize_tensor_fp8(bw["sa_wqkv"])
    assert sc[0] == np.float32(so)
    codes = q[512:512 + 3 * d * d].view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(codes.reshape(3 * d, d), qo)
    q6, s6 = O.quantize_tensor_fp8(bw["ffn_w2"])
    assert sc[5] == np.float32(s6)
    off6 = 512 + 3 * d * d + 3 * d * d + F * d
    codes6 = q[off6:off6 + d * F].view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(codes6.reshape(d, F), q6)


def test_block_fp8_full_size_sampled_rows():
    """The 1.3B block at 480P (L = 32760) in FP8: the whole block on the GPU,
    sampled token rows in the oracle."""
    work = synth.WORKLOADS["wan1.3b-block-480p"]
    L = work.L
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, L - 1, L - 2], rng.integers(0, L, 26)]))
    print(f"fp8 block C2 full size L={L}, {len(rows)} sampled rows", flush=True)
    x0, g_x, o_x, e_x, _, _ = _run_block_fp8(work, rows=rows)
    _check_fp8_block(x0[:, rows], g_x[:, rows], o_x, e_x)
