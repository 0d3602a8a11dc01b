"""The step and the sampler with FP8 blocks, through the C ABI
(wan_quantize_model_fp8, wan_dit_step_fp8_fwd, wan_sample_fp8_fwd), against
the CPU oracle's step with its blocks in FP8, and against their own
composition."""
import numpy as np
import pytest

import oracle.wan_oracle as O
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MINI = {
    "bf16-t2v-b2": synth.mini(41, "bf16-t2v-b2-fp8", dim=256, heads=2, ffn=512, n_blocks=2,
                              lat_f=3, lat_h=12, lat_w=20, batch=2, text_len=40),
    "bf16-i2v": synth.mini(42, "bf16-i2v-fp8", dim=256, heads=2, ffn=512, n_blocks=2, lat_f=3,
                           lat_h=12, lat_w=20, batch=1, text_len=40, in_ch=36, img_len=257),
}


def _inputs(work):
    inp = synth.workload_inputs(work)
    if work.model.in_ch > 16:
        frames = 4 * (work.lat_f - 1) + 1
        fm = np.zeros(frames); fm[0] = 1
        inp["latent"][:, 32:36] = O.i2v_mask(fm, work.lat_f, work.lat_h, work.lat_w)
    return inp


def _device(work, mw):
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import cfg_of, up_block, up_model
    m = work.model
    dev = up_model(mw, m.dtype)
    bdev = [up_block(b, m.dtype) for b in mw["blocks"]]
    mws, keep = W.model_weights(dev, [W.block_weights(b) for b in bdev])
    cfg = cfg_of(work)
    qbuf = torch.empty(W.model_fp8_bytes(cfg), dtype=torch.uint8, device="cuda")
    W.quantize_model_fp8(cfg, mws, qbuf)
    return cfg, mws, qbuf, (dev, bdev, keep)


@pytest.mark.parametrize("name", list(MINI))
def test_step_fp8_vs_oracle(name):
    """Velocity to the usual bar (max-abs 3e-2, mean-rel 1e-2) against the
    oracle's FP8 step, and decisively nearer to it than to the exact step:
    within 0.75 of the distance between the oracle's FP8 and exact steps.
    Two things separate the GPU from the oracle here. One E4M3 step of a code
    decided from slightly different bf16 activations is a legitimate
    difference between two FP8 implementations. The bf16 step's own rounding
    is of the same size as the FP8 effect on the velocity (measured: 0.24%
    against 0.54-0.59% mean-rel)."""
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import assert_parity, metrics, up
    work = MINI[name]
    m = work.model
    print(f"fp8 step {name} L={work.L} blocks={m.n_blocks}", flush=True)
    inp = _inputs(work)
    mw = synth.model_weights(work)
    cfg, mws, qbuf, keep = _device(work, mw)
    out = torch.empty(inp["latent"][:, :16].shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(W.fp8_workspace_bytes(cfg, work.batch, work.lat_f, work.lat_h, work.lat_w),
                     dtype=torch.uint8, device="cuda")
    W.dit_step_fp8_fwd(cfg, up(inp["latent"], "f32"), up(inp["t"], "f32"), up(inp["ctx"], m.dtype),
                       up(inp["clip"], m.dtype) if m.img_len else None, mws, qbuf, out, ws)
    torch.cuda.synchronize()
    g = out.cpu().numpy()
    o8 = O.step(inp["latent"], inp["t"], inp["ctx"], mw, m.heads, m.eps, clip=inp.get("clip"), fp8=True)
    oe = O.step(inp["latent"], inp["t"], inp["ctx"], mw, m.heads, m.eps, clip=inp.get("clip"))
    dev, eff = metrics(g, o8), metrics(oe, o8)
    print("velocity", dev, "fp8 effect", eff, flush=True)
    assert_parity(g, o8, 3e-2, 1e-2, f"fp8 step {name}")
    assert dev["mean_rel"] <= 0.75 * eff["mean_rel"], (dev, eff)


def test_fp8_sampler_is_the_composition_of_its_steps_bitwise():
    """wan_sample_fp8_fwd with 2 guided steps equals, bit for bit, the FP8 step
    at t = 0, Euler by 1/2 with guidance, the FP8 step at t = 500, Euler by 1/2
    (the sampler reads the text K/V from the cache, the step projects them:
    the same bf16 GEMMs)."""
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import up
    work = MINI["bf16-t2v-b2"]
    m = work.model
    print("fp8 sampler = composition of its steps", flush=True)
    inp = _inputs(work)
    inp["latent"][1] = inp["latent"][0]
    mw = synth.model_weights(work)
    cfg, mws, qbuf, keep = _device(work, mw)
    ws = torch.empty(W.fp8_workspace_bytes(cfg, 2, work.lat_f, work.lat_h, work.lat_w, True),
                     dtype=torch.uint8, device="cuda")
    ctx = up(inp["ctx"], m.dtype)
    cache = torch.empty(W.kv_cache_bytes(cfg, 2), dtype=torch.uint8, device="cuda")
    W.kv_cache_fwd(cfg, 2, ctx, None, mws, cache, ws)
    lat_a = up(inp["latent"], "f32")
    lat_b = lat_a.clone()
    W.sample_fp8_fwd(cfg, lat_a, 2, cache, mws, qbuf, ws, True, 5.0)
    vel = torch.empty(inp["latent"][:, :16].shape, dtype=torch.float32, device="cuda")
    for t in (0.0, 500.0):
        W.dit_step_fp8_fwd(cfg, lat_b, torch.full((2,), t, device="cuda"), ctx, None, mws, qbuf, vel, ws)
        W.euler_fwd(lat_b, vel, 0.5, True, 5.0)
    torch.cuda.synchronize()
    assert torch.isfinite(lat_a).all()
    assert torch.equal(lat_a, lat_b)
