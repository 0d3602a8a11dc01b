"""Linear layers whose token-side operand is 2 GiB or more: the launcher splits
them into launches over row slices (each operand slice below 2 GiB, the
32-bit offset range of the bf16 and FP8 kernels), and the gated residual's
slices start at batch-sample boundaries.  Sampled output rows on both sides of
every split, against the oracle.

The operands are drawn on the device from a seeded torch generator (a
2-GiB matrix drawn on the host takes far longer); the oracle reads back only
the sampled rows of the same tensors."""
import numpy as np
import pytest

import oracle.wan_oracle as O
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LIM = (1 << 31) - 1


def _split_rows(M, row_bytes, align):
    """Row offsets where the launcher starts a new slice."""
    rows = LIM // row_bytes // align * align
    return list(range(rows, M, rows))


def _sample_rows(M, cuts, seed):
    rng = np.random.default_rng(seed)
    picks = [0, 1, M - 1, M - 2] + [c + d for c in cuts for d in (-2, -1, 0, 1)]
    return np.unique(np.concatenate([picks, rng.integers(0, M, 24)]))


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_linear_bf16_operand_over_2gib(mode):
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import assert_parity
    M, N, K = 131072, 384, 8192          # A: 2 GiB of bf16
    cuts = _split_rows(M, K * 2, 256)
    assert cuts == [130816]
    print(f"bf16 linear {M}x{N}x{K} mode={mode}, split at {cuts}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(71)
    x = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
    w = (torch.randn((N, K), generator=g, device="cuda") / K ** 0.5).to(torch.bfloat16)
    b = torch.randn(N, generator=g, device="cuda").to(torch.bfloat16)
    y = torch.empty((M, N), dtype=torch.float32 if mode == 1 else torch.bfloat16, device="cuda")
    W.linear_fwd(x, w, b, y, M, N, K, mode)
    torch.cuda.synchronize()
    rows = _sample_rows(M, cuts, 72)
    idx = torch.from_numpy(rows).cuda()
    xs = x[idx].float().cpu().numpy()
    o = O.linear(xs, w.float().cpu().numpy(), b.float().cpu().numpy())
    if mode == 2:
        o = O.gelu_tanh(o)
    gs = y[idx].float().cpu().numpy()
    if mode == 1:
        assert_parity(gs, o, 1e-4, 1e-5, "bf16 linear over 2 GiB, float32 out")
    else:
        assert_parity(gs, o, 3e-2, 1e-2, f"bf16 linear over 2 GiB, mode {mode}")


def test_linear_fp8_operand_over_2gib():
    import video_diffusion_transformer_block_amd as W
    M, N, K = 266240, 256, 8192          # A: 2.03 GiB of E4M3 codes
    cuts = _split_rows(M, K, 256)
    assert cuts == [261888]
    print(f"fp8 linear {M}x{N}x{K}, split at {cuts}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(73)
    x = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
    w = (torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    b = (torch.randn(N, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    qx = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    W.quantize_rows_fp8(x, qx, sx)
    qw = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sw = torch.empty(1, dtype=torch.float32, device="cuda")
    W.quantize_tensor_fp8(w, qw, sw, torch.empty(256, dtype=torch.uint8, device="cuda"))
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    W.linear_fp8_fwd(qx, sx, qw, sw, b, y, M, N, K, 1)
    torch.cuda.synchronize()
    rows = _sample_rows(M, cuts, 74)
    idx = torch.from_numpy(rows).cuda()
    xs = x[idx].float().cpu().numpy()
    qwo, swo = O.quantize_tensor_fp8(w.float().cpu().numpy())
    qxo, sxo = O.quantize_rows_fp8(xs)
    o = (qxo @ qwo.T) * sxo[:, None] * swo + b.float().cpu().numpy()[None, :]
    gs = y[idx].cpu().numpy()
    # float32 accumulation in another order, and the scale products
    bound = (2.0 ** -13 + K * 2.0 ** -24) * (np.abs(qxo) @ np.abs(qwo).T) * sxo[:, None] * swo + 1e-7
    assert np.max(np.abs(gs - o) - bound) <= 0, np.max(np.abs(gs - o))


# eight samples of 30000 tokens, FFN 8960: the FFN hidden state is 4.3e9 bytes
# in bf16 (down-projection as launches over samples 0-2, 3-5, 6-7) and 2.15e9
# bytes of E4M3 codes (samples 0-6, 7); the gated residual's gate is per sample
SPLIT_BLOCK = synth.mini(81, "bf16-ffn-split-b8", dim=256, heads=2, ffn=8960, n_blocks=1, lat_f=3,
                         lat_h=200, lat_w=200, batch=8, text_len=40, kind="block")


@pytest.mark.parametrize("fp8", [False, True])
def test_block_ffn_down_over_2gib(fp8):
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import assert_parity, cfg_of, run_tmlp, up, up_block, workspace
    work = SPLIT_BLOCK
    m = work.model
    L, B = work.L, work.batch
    eb = 1 if fp8 else 2
    cuts = _split_rows(B * L, m.ffn * eb, L)
    assert (L, B) == (30000, 8) and cuts == ([210000] if fp8 else [90000, 180000])
    print(f"block B={B} L={L} ffn={m.ffn} fp8={fp8}: FFN down split at tokens {cuts}", flush=True)
    cfg = cfg_of(work)
    inp = synth.workload_inputs(work)
    tw = synth.tmlp_weights(work)
    bw = synth.block_weights(work, 0)
    twd = {k: up(v, m.dtype) for k, v in tw.items()}
    mod = run_tmlp(cfg, work, twd, up(inp["t"], "f32"))
    x = up(inp["x"], "f32")
    bwd = up_block(bw, m.dtype)
    ctx = up(inp["ctx"], m.dtype)
    if fp8:
        qbuf = torch.empty(W.block_fp8_bytes(cfg), dtype=torch.uint8, device="cuda")
        W.quantize_block_fp8(cfg, W.block_weights(bwd), qbuf)
        ws = torch.empty(W.block_fp8_workspace_bytes(cfg, B, work.lat_f, work.Hp, work.Wp),
                         dtype=torch.uint8, device="cuda")
        W.dit_block_fp8_fwd(cfg, x, B, work.lat_f, work.Hp, work.Wp, mod, W.block_weights(bwd), qbuf, ctx,
                            None, ws)
    else:
        ws = workspace(cfg, work)
        W.dit_block_fwd(cfg, x, B, work.lat_f, work.Hp, work.Wp, mod, W.block_weights(bwd), ctx, None, ws)
    torch.cuda.synchronize()
    g_x = x.cpu().numpy()
    del ws
    rng = np.random.default_rng(82)
    rows = np.unique(np.concatenate([[0, 1, L - 2, L - 1], rng.integers(0, L, 12)]))
    o_mod = O.tmlp(inp["t"], tw["w1"], tw["b1"], tw["w2"], tw["b2"])
    o_x = O.block(inp["x"], o_mod, bw, inp["ctx"], m.heads, m.eps, rows=rows, fp8=fp8)
    x0 = inp["x"][:, rows]
    for s in range(B):
        assert_parity(g_x[s, rows], o_x[s], 3e-2, 1e-2, f"block output, sample {s}")
        assert_parity(g_x[s, rows] - x0[s], o_x[s] - x0[s], 3e-2, 3e-2, f"block update, sample {s}")
