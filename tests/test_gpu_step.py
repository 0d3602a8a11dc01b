"""Step-level parity through the C ABI (wan_dit_step_fwd) against the CPU
oracle: patchify -> shared t-MLP -> blocks -> head -> unpatchify, T2V and
I2V, at sizes the oracle finishes in seconds."""
import numpy as np
import pytest

import oracle.wan_oracle as O
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MINI_STEPS = {
    "bf16-t2v-b2": synth.mini(21, "bf16-t2v-b2", dim=256, heads=2, ffn=512, n_blocks=3,
                              lat_f=3, lat_h=12, lat_w=20, batch=2, text_len=40),
    "bf16-i2v": synth.mini(22, "bf16-i2v", dim=256, heads=2, ffn=512, n_blocks=2, lat_f=3,
                           lat_h=12, lat_w=20, batch=1, text_len=40, in_ch=36, img_len=257),
    "f32-tiny-step": synth.mini(1, "f32-tiny-step", dim=128, heads=2, ffn=512, n_blocks=1,
                                lat_f=2, lat_h=16, lat_w=16, text_len=32, dtype="f32"),
}


def _inputs(work):
    inp = synth.workload_inputs(work)
    m = work.model
    if m.in_ch > 16:
        frames = 4 * (work.lat_f - 1) + 1
        fm = np.zeros(frames); fm[0] = 1
        inp["latent"][:, 32:36] = O.i2v_mask(fm, work.lat_f, work.lat_h, work.lat_w)
    return inp


def run_step(work, mw=None, inp=None):
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import DEV, cfg_of, up, up_block, up_model, workspace
    m = work.model
    cfg = cfg_of(work)
    inp = inp if inp is not None else _inputs(work)
    mw = mw if mw is not None else synth.model_weights(work)
    dev = up_model(mw, m.dtype)
    bdev = [up_block(b, m.dtype) for b in mw["blocks"]]
    mws, keep = W.model_weights(dev, [W.block_weights(b) for b in bdev])
    out = torch.empty(inp["latent"][:, :16].shape, dtype=torch.float32, device=DEV)
    ws = workspace(cfg, work)
    W.dit_step_fwd(cfg, up(inp["latent"], "f32"), up(inp["t"], "f32"), up(inp["ctx"], m.dtype),
                   up(inp["clip"], m.dtype) if m.img_len else None, mws, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), inp, mw


@pytest.mark.parametrize("name", list(MINI_STEPS))
def test_step_mini(name):
    from tests.gpu_util import assert_parity
    work = MINI_STEPS[name]
    print(f"step {name} L={work.L} blocks={work.model.n_blocks}", flush=True)
    g, inp, mw = run_step(work)
    o = O.step(inp["latent"], inp["t"], inp["ctx"], mw, work.model.heads, work.model.eps,
               clip=inp.get("clip"))
    assert_parity(g, o, 3e-2, 1e-2, f"step {name}")


def test_i2v_mask_helper_matches_oracle():
    import video_diffusion_transformer_block_amd as W
    for frames, ones in ((81, [0]), (9, [0, 5]), (13, [3, 12])):
        fm = np.zeros(frames); fm[ones] = 1
        lat_f = (frames - 1) // 4 + 1
        g = W.i2v_mask(fm.astype(int).tolist(), lat_f, 4, 6).numpy()
        assert np.array_equal(g, O.i2v_mask(fm, lat_f, 4, 6)), (frames, ones)


def test_identity_step_round_trip_bitwise():
    """Identity patch/head weights and blocks whose gates and cross-attention
    out-projection are zero: the step returns its latent bit for bit."""
    work = synth.mini(23, "identity", dim=256, heads=2, ffn=512, n_blocks=2, lat_f=3, lat_h=12,
                      lat_w=20, batch=2, text_len=40)
    print("identity step round trip", flush=True)
    mw = synth.model_weights(work)
    d = work.model.dim
    mw["patch_w"] = np.zeros((d, 64), np.float32); mw["patch_w"][:64, :64] = np.eye(64)
    mw["patch_b"] = np.zeros(d, np.float32)
    mw["head_w"] = np.zeros((64, d), np.float32); mw["head_w"][:64, :64] = np.eye(64)
    mw["head_b"] = np.zeros(64, np.float32)
    mw["tmlp"]["w2"] = np.zeros_like(mw["tmlp"]["w2"]); mw["tmlp"]["b2"] = np.zeros_like(mw["tmlp"]["b2"])
    for b in mw["blocks"]:
        b["mod_bias"][2 * d:3 * d] = 0; b["mod_bias"][5 * d:6 * d] = 0
        b["ca_wo"] = np.zeros_like(b["ca_wo"]); b["ca_bo"] = np.zeros_like(b["ca_bo"])
    g, inp, _ = run_step(work, mw=mw)
    assert np.array_equal(g, inp["latent"][:, :16])
