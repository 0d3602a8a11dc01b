"""The sampler around the step, through the C ABI, against the CPU oracle:

* the Euler / guidance kernel (wan_euler_fwd) against its closed form;
* the step with cross-attention K/V from the cache (wan_kv_cache_fwd +
  wan_dit_step_cached_fwd) equals the plain step bit for bit;
* a short sampling run (wan_sample_fwd: guided T2V pair, I2V, fp32) against
  the oracle's Euler loop around the oracle step.
"""
import numpy as np
import pytest

import oracle.wan_oracle as O
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MINI = {
    "bf16-t2v-guided": synth.mini(31, "bf16-t2v-guided", dim=256, heads=2, ffn=512, n_blocks=2,
                                  lat_f=2, lat_h=8, lat_w=12, batch=2, text_len=40),
    "bf16-i2v": synth.mini(32, "bf16-i2v-sample", dim=256, heads=2, ffn=512, n_blocks=2, lat_f=2,
                           lat_h=8, lat_w=12, batch=1, text_len=40, in_ch=36, img_len=257),
    "f32-tiny": synth.mini(33, "f32-tiny-sample", dim=128, heads=2, ffn=512, n_blocks=1, lat_f=2,
                           lat_h=8, lat_w=8, text_len=32, dtype="f32"),
}
GUIDANCE = 5.0


def _inputs(work):
    inp = synth.workload_inputs(work)
    m = work.model
    if work.batch == 2:            # a guidance pair shares its latent and timestep
        inp["latent"][1] = inp["latent"][0]
        inp["t"][1] = inp["t"][0]
    if m.in_ch > 16:
        frames = 4 * (work.lat_f - 1) + 1
        fm = np.zeros(frames); fm[0] = 1
        inp["latent"][:, 32:36] = O.i2v_mask(fm, work.lat_f, work.lat_h, work.lat_w)
    return inp


def _device(work, mw, inp):
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import cfg_of, up, up_block, up_model
    m = work.model
    dev = up_model(mw, m.dtype)
    bdev = [up_block(b, m.dtype) for b in mw["blocks"]]
    mws, keep = W.model_weights(dev, [W.block_weights(b) for b in bdev])
    ctx = up(inp["ctx"], m.dtype)
    clip = up(inp["clip"], m.dtype) if m.img_len else None
    return cfg_of(work), mws, (dev, bdev, keep), ctx, clip


def _cache(W, cfg, work, mws, ctx, clip, ws):
    cache = torch.empty(W.kv_cache_bytes(cfg, work.batch), dtype=torch.uint8, device="cuda")
    W.kv_cache_fwd(cfg, work.batch, ctx, clip, mws, cache, ws)
    return cache


def test_euler_kernel_closed_form():
    import video_diffusion_transformer_block_amd as W
    print("euler kernel", flush=True)
    rng = np.random.default_rng(5)
    lat = rng.standard_normal((2, 36, 3, 6, 10)).astype(np.float32)
    lat[1] = lat[0]
    vel = rng.standard_normal((2, 16, 3, 6, 10)).astype(np.float32)
    dt = 0.02
    for guided, scale in ((True, GUIDANCE), (True, 0.0), (True, 1.0), (False, 1.0)):
        g = torch.from_numpy(lat.copy()).cuda()
        W.euler_fwd(g, torch.from_numpy(vel).cuda(), dt, guided, scale)
        out = g.cpu().numpy()
        if guided:
            want = lat[0, :16].astype(np.float64) + dt * O.cfg_combine(vel[0], vel[1], scale)
            for b in (0, 1):
                assert np.max(np.abs(out[b, :16] - want)) <= 1e-5, (guided, scale, b)
        else:
            assert np.max(np.abs(out[:, :16] - (lat[:, :16].astype(np.float64) + dt * vel))) <= 1e-5
        assert np.array_equal(out[:, 16:], lat[:, 16:]), "condition / mask channels moved"


@pytest.mark.parametrize("name", list(MINI))
def test_cached_step_equals_plain_step_bitwise(name):
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import up, workspace
    work = MINI[name]
    print(f"cached step {name}", flush=True)
    inp = _inputs(work)
    mw = synth.model_weights(work)
    cfg, mws, keep, ctx, clip = _device(work, mw, inp)
    ws = workspace(cfg, work)
    lat, t = up(inp["latent"], "f32"), up(inp["t"], "f32")
    out_a = torch.empty(inp["latent"][:, :16].shape, dtype=torch.float32, device="cuda")
    out_b = torch.empty_like(out_a)
    W.dit_step_fwd(cfg, lat, t, ctx, clip, mws, out_a, ws)
    cache = _cache(W, cfg, work, mws, ctx, clip, ws)
    W.dit_step_cached_fwd(cfg, lat, t, cache, mws, out_b, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out_a).all()
    assert torch.equal(out_a, out_b), "cached cross-attention K/V changed the step"


@pytest.mark.parametrize("name", list(MINI))
def test_sampler_vs_oracle(name):
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import assert_parity, up
    work = MINI[name]
    m = work.model
    n_steps = 3
    guided = work.batch == 2
    print(f"sampler {name}: {n_steps} steps, guided={guided}", flush=True)
    inp = _inputs(work)
    mw = synth.model_weights(work)
    cfg, mws, keep, ctx, clip = _device(work, mw, inp)
    ws = torch.empty(W.sample_workspace_bytes(cfg, work.batch, work.lat_f, work.lat_h, work.lat_w),
                     dtype=torch.uint8, device="cuda")
    cache = _cache(W, cfg, work, mws, ctx, clip, ws)
    lat = up(inp["latent"], "f32")
    W.sample_fwd(cfg, lat, n_steps, cache, mws, ws, guided, GUIDANCE)
    torch.cuda.synchronize()
    g = lat.cpu().numpy()
    o = O.sample(inp["latent"], n_steps,
                 lambda x, t: O.step(x, t, inp["ctx"], mw, m.heads, m.eps, clip=inp.get("clip")),
                 guidance=GUIDANCE if guided else None)
    x0 = inp["latent"].astype(np.float64)
    assert np.array_equal(g[:, 16:], inp["latent"][:, 16:]), "condition / mask channels moved"
    tol = (3e-2, 1e-2) if m.dtype == "bf16" else (1e-4, 1e-4)
    # the distance travelled from the noise, on its own scale
    assert_parity(g[:, :16] - x0[:, :16], o[:, :16] - x0[:, :16], *tol, f"sampler {name}")
    if guided:
        assert np.array_equal(g[0], g[1]), "guided pair diverged"


def test_sampler_is_the_composition_of_its_steps_bitwise():
    """wan_sample_fwd with 2 steps equals, bit for bit, the cached step at
    t = 0, Euler by 1/2, the cached step at t = 500, Euler by 1/2 (the flow
    time grid k/n and the timestep input 1000 k/n)."""
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import up
    work = MINI["bf16-t2v-guided"]
    print("sampler = composition of its steps", flush=True)
    inp = _inputs(work)
    mw = synth.model_weights(work)
    cfg, mws, keep, ctx, clip = _device(work, mw, inp)
    ws = torch.empty(W.sample_workspace_bytes(cfg, 2, work.lat_f, work.lat_h, work.lat_w),
                     dtype=torch.uint8, device="cuda")
    cache = _cache(W, cfg, work, mws, ctx, clip, ws)
    lat_a = up(inp["latent"], "f32")
    lat_b = lat_a.clone()
    W.sample_fwd(cfg, lat_a, 2, cache, mws, ws, True, GUIDANCE)
    vel = torch.empty(inp["latent"][:, :16].shape, dtype=torch.float32, device="cuda")
    for t in (0.0, 500.0):
        W.dit_step_cached_fwd(cfg, lat_b, torch.full((2,), t, device="cuda"), cache, mws, vel, ws)
        W.euler_fwd(lat_b, vel, 0.5, True, GUIDANCE)
    torch.cuda.synchronize()
    assert torch.equal(lat_a, lat_b)
