"""Full-size denoising steps (1.3B CFG batch of 2; 14B I2V), checked through
properties that hold at any size -- the oracle cannot follow 30-40 blocks at
L = 32760 (the block itself is checked against the oracle at full size on
sampled rows in test_gpu_block.py):

* batch independence, bit for bit: sample 1 of a batch-2 step equals a
  batch-1 step on sample 1's inputs;
* determinism: the same call twice gives the same bits;
* the I2V extra input channels go through a zero projection, so the
  condition latent and mask channels change nothing, bit for bit;
* identity weights (patch/head identity, zero gates, zero cross-attention
  out-projection in every block) return the latent bit for bit.
"""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _run(work, mw, latent, t, ctx, clip):
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import cfg_of
    cfg = cfg_of(work)
    B = latent.shape[0]
    mws, keep = W.model_weights(mw, [W.block_weights(b) for b in mw["blocks"]])
    out = torch.empty((B, 16) + tuple(latent.shape[2:]), dtype=torch.float32, device="cuda")
    ws = torch.empty(W.workspace_bytes(cfg, B, work.lat_f, work.lat_h, work.lat_w),
                     dtype=torch.uint8, device="cuda")
    W.dit_step_fwd(cfg, latent, t, ctx, clip, mws, out, ws)
    torch.cuda.synchronize()
    return out


def _inputs(work, B):
    m = work.model
    inp = synth.workload_inputs(work)
    dt = torch.bfloat16
    lat = torch.from_numpy(inp["latent"][:1].repeat(B, 0)).cuda()
    t = torch.from_numpy(inp["t"][:1].repeat(B)).cuda()
    ctx = torch.from_numpy(inp["ctx"]).to(dt).cuda()
    clip = torch.from_numpy(inp["clip"]).to(dt).cuda() if m.img_len else None
    return lat, t, ctx, clip


def test_c3_step_batch_independence_and_determinism():
    work = synth.WORKLOADS["wan1.3b-step-480p-cfg2"]
    print(f"C3 step: B=2, L={work.L}, {work.model.n_blocks} blocks", flush=True)
    mw = synth.device_model_weights(work)
    lat, t, ctx, _ = _inputs(work, 2)
    out2 = _run(work, mw, lat, t, ctx, None)
    assert torch.isfinite(out2).all()
    out2b = _run(work, mw, lat, t, ctx, None)
    assert torch.equal(out2, out2b), "non-deterministic step"
    out1 = _run(work, mw, lat[1:].contiguous(), t[1:].contiguous(), ctx[1:].contiguous(), None)
    assert torch.equal(out2[1], out1[0]), "sample 1 of the batch differs from the batch-1 step"
    # the two text contexts differ, so the two velocities must differ
    assert not torch.equal(out2[0], out2[1])


def test_c3_cached_step_equals_plain_step_bitwise():
    """The 30-block 1.3B guidance pair: the step with the cross-attention K/V
    from the cache equals the plain step bit for bit."""
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import cfg_of
    work = synth.WORKLOADS["wan1.3b-step-480p-cfg2"]
    print(f"C3 cached step: B=2, L={work.L}, {work.model.n_blocks} blocks", flush=True)
    cfg = cfg_of(work)
    mw = synth.device_model_weights(work)
    lat, t, ctx, _ = _inputs(work, 2)
    out = _run(work, mw, lat, t, ctx, None)
    mws, keep = W.model_weights(mw, [W.block_weights(b) for b in mw["blocks"]])
    ws = torch.empty(W.workspace_bytes(cfg, 2, work.lat_f, work.lat_h, work.lat_w),
                     dtype=torch.uint8, device="cuda")
    cache = torch.empty(W.kv_cache_bytes(cfg, 2), dtype=torch.uint8, device="cuda")
    W.kv_cache_fwd(cfg, 2, ctx, None, mws, cache, ws)
    out_c = torch.empty_like(out)
    W.dit_step_cached_fwd(cfg, lat, t, cache, mws, out_c, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out_c), "cached cross-attention K/V changed the 1.3B step"


def test_c5_step_zero_projection_and_identity():
    work = synth.WORKLOADS["wan14b-i2v-step-480p"]
    m = work.model
    print(f"C5 I2V step: L={work.L}, {m.n_blocks} blocks, {m.in_ch} channels", flush=True)
    mw = synth.device_model_weights(work)
    lat, t, ctx, clip = _inputs(work, 1)
    frames = 4 * (work.lat_f - 1) + 1
    import video_diffusion_transformer_block_amd as W
    fm = [1] + [0] * (frames - 1)
    lat[:, 32:36] = W.i2v_mask(fm, work.lat_f, work.lat_h, work.lat_w).cuda()
    out = _run(work, mw, lat, t, ctx, clip)
    assert torch.isfinite(out).all()
    lat0 = lat.clone()
    lat0[:, 16:] = 0
    out0 = _run(work, mw, lat0, t, ctx, clip)
    assert torch.equal(out, out0), "extra I2V channels leak through the zero projection"
    # identity weights: the step returns the noise latent bit for bit
    d = m.dim
    eye = torch.zeros((d, m.in_ch * 4), dtype=torch.bfloat16, device="cuda")
    eye[:64, :64] = torch.eye(64, dtype=torch.bfloat16, device="cuda")
    mw["patch_w"] = eye
    mw["patch_b"] = torch.zeros(d, dtype=torch.bfloat16, device="cuda")
    head = torch.zeros((64, d), dtype=torch.bfloat16, device="cuda")
    head[:, :64] = torch.eye(64, dtype=torch.bfloat16, device="cuda")
    mw["head_w"], mw["head_b"] = head, torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    mw["tmlp"]["w2"].zero_()
    mw["tmlp"]["b2"].zero_()
    for b in mw["blocks"]:
        b["mod_bias"][2 * d:3 * d] = 0
        b["mod_bias"][5 * d:6 * d] = 0
        b["ca_wo"].zero_()
        b["ca_bo"].zero_()
    outi = _run(work, mw, lat, t, ctx, clip)
    assert torch.equal(outi, lat[:, :16]), "identity step does not return the latent"
