"""The step with every block's self-attention in 8 bits (cfg attn8 = 1),
with bf16 and with FP8 block Linear layers, through the C ABI
(wan_dit_step_fwd, wan_dit_step_fp8_fwd), against the oracle's step with the
same switches (readings R25, R26).  Bars: the usual one on the velocity
against the oracle's 8-bit step; and the switch is engaged, the GPU's own
8-bit effect (the same step with and without attn8) at least a quarter of the
oracle's.  No upper bound here: with the mini models' near-uniform attention
almost every probability rounds to the same E4M3 value, the oracle's 8-bit
effect on the velocity falls far below the bf16 rounding of the GPU's own
bf16 attention (which the difference of the two GPU steps contains), and a
wrong 8-bit path would fail the parity bar."""
import numpy as np
import pytest

import oracle.wan_oracle as O
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MINI = {
    "bf16-t2v-b2": synth.mini(51, "bf16-t2v-b2-attn8", dim=256, heads=2, ffn=512, n_blocks=2,
                              lat_f=3, lat_h=12, lat_w=20, batch=2, text_len=40),
    "bf16-i2v": synth.mini(52, "bf16-i2v-attn8", dim=256, heads=2, ffn=512, n_blocks=2, lat_f=3,
                           lat_h=12, lat_w=20, batch=1, text_len=40, in_ch=36, img_len=257),
}


def _inputs(work):
    inp = synth.workload_inputs(work)
    if work.model.in_ch > 16:
        frames = 4 * (work.lat_f - 1) + 1
        fm = np.zeros(frames)
        fm[0] = 1
        inp["latent"][:, 32:36] = O.i2v_mask(fm, work.lat_f, work.lat_h, work.lat_w)
    return inp


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("name", list(MINI))
def test_step_attn8_vs_oracle(name, fp8):
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import assert_parity, cfg_of, metrics, up, up_block, up_model
    work = MINI[name]
    m = work.model
    print(f"attn8 step {name} fp8={fp8} L={work.L} blocks={m.n_blocks}", flush=True)
    inp = _inputs(work)
    mw = synth.model_weights(work)
    dev = up_model(mw, m.dtype)
    bdev = [up_block(b, m.dtype) for b in mw["blocks"]]
    mws, keep = W.model_weights(dev, [W.block_weights(b) for b in bdev])
    args = (up(inp["latent"], "f32"), up(inp["t"], "f32"), up(inp["ctx"], m.dtype),
            up(inp["clip"], m.dtype) if m.img_len else None)
    outs = []
    for attn8 in (1, 0):
        cfg = cfg_of(work)
        cfg.attn8 = attn8
        out = torch.empty(inp["latent"][:, :16].shape, dtype=torch.float32, device="cuda")
        if fp8:
            qbuf = torch.empty(W.model_fp8_bytes(cfg), dtype=torch.uint8, device="cuda")
            W.quantize_model_fp8(cfg, mws, qbuf)
            ws = torch.empty(W.fp8_workspace_bytes(cfg, work.batch, work.lat_f, work.lat_h, work.lat_w),
                             dtype=torch.uint8, device="cuda")
            W.dit_step_fp8_fwd(cfg, *args, mws, qbuf, out, ws)
        else:
            ws = torch.empty(W.workspace_bytes(cfg, work.batch, work.lat_f, work.lat_h, work.lat_w),
                             dtype=torch.uint8, device="cuda")
            W.dit_step_fwd(cfg, *args, mws, out, ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    g8, g0 = outs
    o8 = O.step(inp["latent"], inp["t"], inp["ctx"], mw, m.heads, m.eps, clip=inp.get("clip"), fp8=fp8,
                attn8=True)
    o0 = O.step(inp["latent"], inp["t"], inp["ctx"], mw, m.heads, m.eps, clip=inp.get("clip"), fp8=fp8)
    gef, oef = np.abs(g8 - g0).mean(), np.abs(o8 - o0).mean()
    print("velocity", metrics(g8, o8), f"8-bit effect: GPU {gef:.3e}, oracle {oef:.3e}", flush=True)
    assert_parity(g8, o8, 3e-2, 1e-2, f"attn8 step {name} fp8={fp8}")
    assert gef >= 0.25 * oef, (gef, oef)
