"""The block with its self-attention in 8 bits (cfg attn8 = 1) through the C
ABI, with bf16 and with FP8 Linear layers, against the oracle's block with
the same switch (reading R26): the 8-bit self-attention on the bf16 q, k, v,
the cross-attention exact.

Two checks.  The block output against the oracle's 8-bit block to the usual
bar (max-abs 3e-2, mean-rel 1e-2).  And the switch is engaged: the GPU's own
8-bit effect (the same block with and without attn8, same inputs) has the
size of the oracle's (8-bit minus exact block): their mean magnitudes within
a factor 4 of each other.  (The update cannot be judged against the 8-bit
effect as for the FP8 block: with bf16 Linear layers that effect is smaller
than the bf16 rounding differences of the rest of the block.)"""
import numpy as np
import pytest

import oracle.wan_oracle as O
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


BLOCKS = {
    "bf16-ragged-b2": synth.mini(21, "bf16-ragged-b2", dim=384, heads=3, ffn=640, n_blocks=1,
                                 lat_f=3, lat_h=20, lat_w=40, batch=2, text_len=40, kind="block"),
    "bf16-i2v": synth.mini(22, "bf16-i2v", dim=256, heads=2, ffn=512, n_blocks=1, lat_f=2,
                           lat_h=16, lat_w=24, batch=1, text_len=64, img_len=257, kind="block"),
}


def _run(work, fp8, rows=None):
    """GPU block with and without attn8 (same inputs), oracle block with and
    without it."""
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import cfg_of, run_tmlp, up, up_block
    m = work.model
    inp = synth.workload_inputs(work)
    tw = synth.tmlp_weights(work)
    bw = synth.block_weights(work, 0)
    img = None
    if m.img_len:
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([2025, work.cid, 77])))
        img = synth.bf16_round(g.standard_normal((work.batch, m.img_len, m.dim), dtype=np.float32))
    twd = {k: up(v, m.dtype) for k, v in tw.items()}
    bwd = up_block(bw, m.dtype)
    ctx = up(inp["ctx"], m.dtype)
    imgd = up(img, m.dtype) if img is not None else None
    outs = []
    for attn8 in (1, 0):
        cfg = cfg_of(work)
        cfg.attn8 = attn8
        mod = run_tmlp(cfg, work, twd, up(inp["t"], "f32"))
        x = up(inp["x"], "f32")
        if fp8:
            qbuf = torch.empty(W.block_fp8_bytes(cfg), dtype=torch.uint8, device="cuda")
            W.quantize_block_fp8(cfg, W.block_weights(bwd), qbuf)
            ws = torch.empty(W.block_fp8_workspace_bytes(cfg, work.batch, work.lat_f, work.Hp, work.Wp),
                             dtype=torch.uint8, device="cuda")
            W.dit_block_fp8_fwd(cfg, x, work.batch, work.lat_f, work.Hp, work.Wp, mod, W.block_weights(bwd),
                                qbuf, ctx, imgd, ws)
        else:
            ws = torch.empty(W.workspace_bytes(cfg, work.batch, work.lat_f, work.lat_h, work.lat_w),
                             dtype=torch.uint8, device="cuda")
            W.dit_block_fwd(cfg, x, work.batch, work.lat_f, work.Hp, work.Wp, mod, W.block_weights(bwd), ctx,
                            imgd, ws)
        torch.cuda.synchronize()
        outs.append(x.cpu().numpy())
        del ws
    o_mod = O.tmlp(inp["t"], tw["w1"], tw["b1"], tw["w2"], tw["b2"])
    o_x = O.block(inp["x"], o_mod, bw, inp["ctx"], m.heads, m.eps, img=img, rows=rows, fp8=fp8, attn8=True)
    e_x = O.block(inp["x"], o_mod, bw, inp["ctx"], m.heads, m.eps, img=img, rows=rows, fp8=fp8)
    return outs[0], outs[1], o_x, e_x


def _check(g8, g0, o8, o0, what):
    from tests.gpu_util import assert_parity, metrics
    gef, oef = np.abs(g8 - g0).mean(), np.abs(o8 - o0).mean()
    print(f"{what}: output", metrics(g8, o8), f"8-bit effect: GPU {gef:.3e}, oracle {oef:.3e}", flush=True)
    assert_parity(g8, o8, 3e-2, 1e-2, what)
    assert 0.25 * oef <= gef <= 4.0 * oef, (gef, oef)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("name", list(BLOCKS))
def test_attn8_block_mini(name, fp8):
    work = BLOCKS[name]
    print(f"attn8 block {name} fp8={fp8} L={work.L} d={work.model.dim}", flush=True)
    _check(*_run(work, fp8), f"attn8 block {name} fp8={fp8}")


def test_attn8_block_full_size_sampled_rows():
    """The 1.3B block at 480P (L = 32760) with FP8 Linear layers and the 8-bit
    self-attention: the whole block on the GPU, sampled token rows in the
    oracle (self-attention reads every key, so the oracle still projects all
    tokens)."""
    work = synth.WORKLOADS["wan1.3b-block-480p"]
    L = work.L
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, L - 1, L - 2], rng.integers(0, L, 18)]))
    print(f"attn8 + fp8 block full size L={L}, {len(rows)} sampled rows", flush=True)
    g8, g0, o8, o0 = _run(work, True, rows=rows)
    _check(g8[:, rows], g0[:, rows], o8, o0, "attn8 + fp8 block full size")
