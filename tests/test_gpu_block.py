"""Block-level parity through the C ABI (wan_tmlp_fwd + wan_dit_block_fwd)
against the CPU oracle, on whole outputs at small sizes and on sampled rows
at the full 1.3B / 14B sizes."""
import numpy as np
import pytest

import oracle.wan_oracle as O
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MINI_BLOCKS = {
    # ragged everywhere: L = 600 (3 query tiles, last 88), N = 384 / 640 tails, Lc = 40
    "bf16-ragged-b2": synth.mini(11, "bf16-ragged-b2", dim=384, heads=3, ffn=640, n_blocks=1,
                                 lat_f=3, lat_h=20, lat_w=40, batch=2, text_len=40, kind="block"),
    "bf16-i2v": synth.mini(12, "bf16-i2v", dim=256, heads=2, ffn=512, n_blocks=1, lat_f=2,
                           lat_h=16, lat_w=24, batch=1, text_len=64, img_len=257, kind="block"),
    "f32-tiny": synth.CONFIGS[1],
}


def _run_block(work, rows=None):
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import cfg_of, run_tmlp, up, up_block, workspace
    m = work.model
    cfg = cfg_of(work)
    inp = synth.workload_inputs(work)
    tw = synth.tmlp_weights(work)
    bw = synth.block_weights(work, 0)
    img = None
    if m.img_len:
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([2025, work.cid, 77])))
        img = synth.bf16_round(g.standard_normal((work.batch, m.img_len, m.dim), dtype=np.float32))
    # GPU
    twd = {k: up(v, m.dtype) for k, v in tw.items()}
    mod = run_tmlp(cfg, work, twd, up(inp["t"], "f32"))
    x = up(inp["x"], "f32")
    bwd = up_block(bw, m.dtype)
    ctx = up(inp["ctx"], m.dtype)
    imgd = up(img, m.dtype) if img is not None else None
    ws = workspace(cfg, work)
    W.dit_block_fwd(cfg, x, work.batch, work.lat_f, work.Hp, work.Wp, mod, W.block_weights(bwd),
                    ctx, imgd, ws)
    torch.cuda.synchronize()
    g_mod = mod.cpu().numpy()
    g_x = x.cpu().numpy()
    # oracle
    o_mod = O.tmlp(inp["t"], tw["w1"], tw["b1"], tw["w2"], tw["b2"])
    o_x = O.block(inp["x"], o_mod, bw, inp["ctx"], m.heads, m.eps, img=img, rows=rows)
    return inp["x"], g_mod, o_mod, g_x, o_x


@pytest.mark.parametrize("name", list(MINI_BLOCKS))
def test_block_mini(name):
    from tests.gpu_util import assert_parity
    work = MINI_BLOCKS[name]
    print(f"block {name} L={work.L} d={work.model.dim}", flush=True)
    x0, g_mod, o_mod, g_x, o_x = _run_block(work)
    assert_parity(g_mod, o_mod, 1e-4, 1e-5, "t-MLP")
    assert_parity(g_x, o_x, 3e-2, 1e-2, "block output")
    # the block's update alone (x_out - x_in), judged relative to its own size
    tol = 1e-4 if work.model.dtype == "f32" else 3e-2
    assert_parity(g_x - x0, o_x - x0, tol, tol, "block update")


@pytest.mark.parametrize("cid", [2, 4])
def test_block_full_size_sampled_rows(cid):
    from tests.gpu_util import assert_parity
    work = synth.CONFIGS[cid]
    L = work.L
    rng = np.random.default_rng(cid)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, L - 1, L - 2, (L // 256) * 256],
                                     rng.integers(0, L, 57)]))
    print(f"block C{cid} full size L={L}, {len(rows)} sampled rows", flush=True)
    x0, g_mod, o_mod, g_x, o_x = _run_block(work, rows=rows)
    assert_parity(g_mod, o_mod, 1e-4, 1e-5, "t-MLP")
    assert_parity(g_x[:, rows], o_x, 3e-2, 1e-2, "block output (sampled rows)")
    assert_parity(g_x[:, rows] - x0[:, rows], o_x - x0[:, rows], 3e-2, 3e-2, "block update")
