"""The allocation-free block entry point (wan_dit_block_fwd_noalloc) against
wan_dit_block_fwd: two calls in a row on the library's static scratch, the
second with a smaller input, each bit for bit equal to the workspace entry
point on the same inputs (same kernels, same order), and the smaller one also
against the CPU oracle."""
import numpy as np
import pytest

import oracle.wan_oracle as O
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# 1.3B widths; a 480x832 latent with 2 and 1 latent frames, then a smaller
# ragged one with a batch of 2 and 64 text tokens
CASES = [
    synth.mini(41, "noalloc-big", dim=1536, heads=12, ffn=8960, n_blocks=1, lat_f=2, lat_h=60,
               lat_w=104, batch=1, text_len=512, kind="block"),
    synth.mini(42, "noalloc-small", dim=1536, heads=12, ffn=8960, n_blocks=1, lat_f=1, lat_h=20,
               lat_w=30, batch=2, text_len=64, kind="block"),
]


def _inputs(work):
    from tests.gpu_util import cfg_of, run_tmlp, up, up_block
    m = work.model
    cfg = cfg_of(work)
    inp = synth.workload_inputs(work)
    tw = synth.tmlp_weights(work)
    bw = synth.block_weights(work, 0)
    twd = {k: up(v, m.dtype) for k, v in tw.items()}
    mod = run_tmlp(cfg, work, twd, up(inp["t"], "f32"))
    return cfg, inp, tw, bw, mod, up_block(bw, m.dtype), up(inp["ctx"], m.dtype)


def test_noalloc_block_equals_workspace_block_twice():
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import assert_parity, up, workspace
    for i, work in enumerate(CASES):
        cfg, inp, tw, bw, mod, bwd, ctx = _inputs(work)
        need = W.dit_block_noalloc_bytes(cfg, work.batch, work.lat_f, work.Hp, work.Wp)
        print(f"noalloc call {i}: {work.name} B={work.batch} L={work.L} scratch {need >> 20} MiB",
              flush=True)
        assert 0 < need <= W.NOALLOC_SCRATCH_BYTES
        x_ref = up(inp["x"], "f32")
        W.dit_block_fwd(cfg, x_ref, work.batch, work.lat_f, work.Hp, work.Wp, mod,
                        W.block_weights(bwd), ctx, None, workspace(cfg, work))
        x_na = up(inp["x"], "f32")
        W.dit_block_fwd_noalloc(cfg, x_na, work.batch, work.lat_f, work.Hp, work.Wp, mod,
                                W.block_weights(bwd), ctx, None)
        torch.cuda.synchronize()
        assert torch.isfinite(x_na).all()
        assert torch.equal(x_na, x_ref), f"call {i}: differs from wan_dit_block_fwd"
        if i == 1:   # the smaller input also against the oracle
            o_mod = O.tmlp(inp["t"], tw["w1"], tw["b1"], tw["w2"], tw["b2"])
            o_x = O.block(inp["x"], o_mod, bw, inp["ctx"], work.model.heads, work.model.eps)
            assert_parity(x_na.cpu().numpy(), o_x, 3e-2, 1e-2, "noalloc block vs oracle")
            assert_parity(x_na.cpu().numpy() - inp["x"], o_x - inp["x"], 3e-2, 1e-2,
                          "noalloc block update vs oracle")


def test_noalloc_block_rejects_sizes_beyond_scratch():
    import video_diffusion_transformer_block_amd as W
    work = synth.WORKLOADS["wan1.3b-block-480p"]   # the full latent needs ~1.1 GiB of temporaries
    cfg = W.make_cfg(dim=1536, heads=12, ffn=8960)
    assert W.dit_block_noalloc_bytes(cfg, 1, work.lat_f, work.Hp, work.Wp) > W.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(1, dtype=torch.float32, device="cuda")
    bw = W.binding.BlockW(*([1] * 17))
    with pytest.raises(W.WanError) as e:
        W.dit_block_fwd_noalloc(cfg, x, 1, work.lat_f, work.Hp, work.Wp, x, bw, x, None)
    assert e.value.status == -4
