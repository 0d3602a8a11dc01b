"""The full-size denoising steps against the CPU oracle: the 1.3B guidance
pair (30 blocks, B = 2, L = 32760; [Note] 配置表, [Guide] 工作原理), the 14B
image-to-video step (40 blocks, 36 input channels, 257 image tokens;
[Note] I2V 架构扩展, [News] 核心创新四), and the same 14B step on a short clip
(latent 21 x 8 x 8, L = 336) in bf16 and in float32.

The oracle cannot run 30-40 full-width blocks at L = 32760 inside a test (an
hour and more of float64 CPU time), so ``tests/golden/make_full_step_golden.py``
ran it once on the same seeded inputs and weights (``synth``) and stored a
seeded sample of output elements with their indices.  Here the HIP step runs
on those inputs -- weights drawn on the host with the same streams, rounded to
bf16 and uploaded block by block -- and the stored elements are compared.

The bar: outputs of unit scale (RMS at most 1: the 1.3B pair) take max-abs
3e-2 and mean-rel 1e-2 as stated.  The 14B velocity with N(0, 0.02) weights
has an RMS near 7.6; there a bf16 step's deviation is noise proportional to
that scale (rounding the head GEMM's input to bf16 alone gives an RMS of about
0.006), so the absolute 3e-2 is below what bf16 operands resolve.  Those
outputs take mean-rel 1e-2 as stated, an error RMS within 1% of the output
RMS, and no element beyond 5x the error RMS (noise, not a localized fault).
The float32 run of the short 14B step holds mean-rel 1e-4 against the
float64 oracle, which pins the wiring at full width and depth exactly."""
import dataclasses
import json
import os

import numpy as np
import pytest

import synth
from tests.golden.make_full_step_golden import WORKLOADS, golden_path, step_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _upload_model(work, dtype):
    """Model weights of ``work`` (the values synth.model_weights and
    synth.block_weights draw, bf16-representable) in the layout of the C ABI,
    on the device as ``dtype``."""
    from tests.gpu_util import up_block, up_model
    m = work.model
    mw = up_model(synth.model_weights(work, with_blocks=False), dtype)
    blocks = []
    for i, bw in enumerate(synth.block_weights_iter(work, threads=16)):
        blocks.append(up_block(bw, dtype))
        if i % 10 == 9 or i == m.n_blocks - 1:
            print(f"  uploaded block {i + 1}/{m.n_blocks}", flush=True)
    mw["blocks"] = blocks
    return mw


def _gold(cid, fp8=False):
    path = golden_path(cid, fp8)
    if not os.path.exists(path):
        pytest.skip(f"{os.path.basename(path)} not written yet "
                    f"(python -m tests.golden.make_full_step_golden --config {cid}{' --fp8' if fp8 else ''})")
    with open(path) as f:
        return json.load(f)


def _step(cid, dtype):
    """The HIP step of workload ``cid`` with operands of ``dtype`` ("bf16" or
    "f32"; the values are the same bf16-representable ones either way)."""
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import cfg_of, up
    work = WORKLOADS[cid]
    m = work.model
    lat, t, ctx, clip = step_inputs(cid)
    dlat = up(lat, "f32")
    if m.in_ch > 16:   # the mask channels from the library's own helper, as a caller builds them
        frames = 1 + 4 * (work.lat_f - 1)
        mk = W.i2v_mask([1] + [0] * (frames - 1), work.lat_f, work.lat_h, work.lat_w)
        assert np.array_equal(mk.numpy(), lat[0, 32:36])
        dlat[:, 32:36] = mk.cuda()
    mw = _upload_model(work, dtype)
    cfg = cfg_of(dataclasses.replace(work, model=dataclasses.replace(m, dtype=dtype)))
    mws, keep = W.model_weights(mw, [W.block_weights(b) for b in mw["blocks"]])
    out = torch.empty((work.batch, 16, work.lat_f, work.lat_h, work.lat_w), dtype=torch.float32,
                      device="cuda")
    ws = torch.empty(W.workspace_bytes(cfg, work.batch, work.lat_f, work.lat_h, work.lat_w),
                     dtype=torch.uint8, device="cuda")
    W.dit_step_fwd(cfg, dlat, up(t, "f32"), up(ctx, dtype), up(clip, dtype) if clip is not None else None,
                   mws, out, ws)
    torch.cuda.synchronize()
    g_all = out.cpu().numpy()
    assert np.all(np.isfinite(g_all))
    return g_all


def _noise_bar(g, o, what):
    """Outputs far above unit scale: mean-rel 1e-2, error RMS within 1% of the
    output RMS, and no element beyond 5x the error RMS."""
    from tests.gpu_util import metrics
    m = metrics(g, o)
    d = np.asarray(g, np.float64) - o
    rms_e, rms_o = float(np.sqrt(np.mean(d * d))), float(np.sqrt(np.mean(o * o)))
    m.update(rms_err=rms_e, rms_out=rms_o, max_over_rms_err=m["max_abs"] / max(rms_e, 1e-30))
    assert m["mean_rel"] <= 1e-2, f"{what}: {m}"
    assert rms_e <= 1e-2 * rms_o, f"{what}: {m}"
    assert m["max_abs"] <= 5 * rms_e, f"{what}: {m}"
    return m


@pytest.mark.parametrize("cid", [3, 5, 53])
def test_full_step_against_oracle_samples(cid):
    from tests.gpu_util import assert_parity
    work = WORKLOADS[cid]
    gold = _gold(cid)
    print(f"full step {work.name}: B={work.batch} L={work.L} blocks={work.model.n_blocks} "
          f"(oracle took {gold['oracle_seconds']:.0f}s)", flush=True)
    assert list(gold["output_shape"]) == [work.batch, 16, work.lat_f, work.lat_h, work.lat_w]
    g_all = _step(cid, work.model.dtype)
    for b, s in enumerate(gold["samples"]):
        idx = np.asarray(s["flat_index"])
        g = g_all[b].reshape(-1)[idx]
        o = np.asarray(s["value"])
        what = f"{work.name} sample {b} ({len(idx)} elements)"
        if np.sqrt(np.mean(o * o)) <= 1.0:
            met = assert_parity(g, o, 3e-2, 1e-2, what)
        else:
            met = _noise_bar(g, o, what)
        print(f"  sample {b}: {met}; mean |v| GPU {np.abs(g_all[b]).mean():.4f} "
              f"oracle {s['abs_mean_all']:.4f}", flush=True)
        # the whole output's mean magnitude matches the oracle's (a check on
        # every element, not only the stored ones)
        assert abs(np.abs(g_all[b]).mean() / s["abs_mean_all"] - 1) < 1e-2


def test_short_i2v_step_float32():
    """The 14B image-to-video step at full width and depth on the short clip,
    with float32 operands throughout: the same values as the bf16 run, so
    its distance to the float64 oracle is float32 rounding only."""
    from tests.gpu_util import assert_parity
    cid = 53
    gold = _gold(cid)
    g_all = _step(cid, "f32")
    for b, s in enumerate(gold["samples"]):
        idx = np.asarray(s["flat_index"])
        o = np.asarray(s["value"])
        met = assert_parity(g_all[b].reshape(-1)[idx], o, 1e-3 * float(np.sqrt(np.mean(o * o))), 1e-4,
                            f"float32 {WORKLOADS[cid].name} sample {b}")
        print(f"  float32 sample {b}: {met}", flush=True)
        assert abs(np.abs(g_all[b]).mean() / s["abs_mean_all"] - 1) < 1e-4


def test_full_step_fp8_against_oracle_samples():
    """The 30-block 1.3B guidance pair with every block's Linear layers in FP8
    (wan_quantize_model_fp8, wan_dit_step_fp8_fwd; [Note] Infra / 推理优化: FP8
    GEMM) against the oracle's FP8 step on the stored elements (reading R28).

    An E4M3 code is an integer decided from a bf16 activation; where two
    correct implementations differ in a bf16 activation's last place, codes
    move by a whole E4M3 step (6 - 12 %), and over 30 full-width blocks those
    flips compound.  Two FP8 runs of the oracle itself at this width (d = 1536,
    FFN 8960, a short clip), one with bf16-level noise added after every block,
    drift apart by 0.67x the FP8 effect after one block and 0.84 - 0.87x from
    10 to 30 blocks, while each keeps an FP8 effect (distance from the exact
    step) of the same size (tests/golden/fp8_drift.py, on the CPU).  So the bar, on the stored elements, is:
    the GPU's FP8 step no farther from the oracle's FP8 step than the exact
    step is (1.0x the FP8 effect); the GPU's own FP8 effect (its distance from
    the exact step, the bf16 golden's values at the same seeded indices)
    between 0.8x and 1.25x the oracle's -- an FP8 switch that does nothing
    lands near 0.05x (bf16 noise), a wrong scale far above; and the mean
    magnitude within 1 % of the oracle's."""
    import video_diffusion_transformer_block_amd as W
    from tests.gpu_util import cfg_of, metrics, up
    cid = 3
    work = WORKLOADS[cid]
    m = work.model
    g8, ge = _gold(cid, fp8=True), _gold(cid)
    lat, t, ctx, clip = step_inputs(cid)
    mw = _upload_model(work, m.dtype)
    cfg = cfg_of(work)
    mws, keep = W.model_weights(mw, [W.block_weights(b) for b in mw["blocks"]])
    qbuf = torch.empty(W.model_fp8_bytes(cfg), dtype=torch.uint8, device="cuda")
    W.quantize_model_fp8(cfg, mws, qbuf)
    out = torch.empty((work.batch, 16, work.lat_f, work.lat_h, work.lat_w), dtype=torch.float32,
                      device="cuda")
    ws = torch.empty(W.fp8_workspace_bytes(cfg, work.batch, work.lat_f, work.lat_h, work.lat_w),
                     dtype=torch.uint8, device="cuda")
    W.dit_step_fp8_fwd(cfg, up(lat, "f32"), up(t, "f32"), up(ctx, m.dtype), None, mws, qbuf, out, ws)
    torch.cuda.synchronize()
    g_all = out.cpu().numpy()
    assert np.all(np.isfinite(g_all))
    for b, (s8, se) in enumerate(zip(g8["samples"], ge["samples"])):
        assert s8["flat_index"] == se["flat_index"]
        idx = np.asarray(s8["flat_index"])
        g = g_all[b].reshape(-1)[idx]
        o8, oe = np.asarray(s8["value"]), np.asarray(se["value"])
        dev, eff, own = metrics(g, o8), metrics(oe, o8), metrics(g, oe)
        print(f"  fp8 sample {b}: GPU vs FP8 oracle {dev}; FP8 effect {eff}; GPU vs exact {own}; "
              f"ratios {dev['mean_rel'] / eff['mean_rel']:.2f}, {own['mean_rel'] / eff['mean_rel']:.2f}",
              flush=True)
        assert dev["mean_rel"] <= 1.0 * eff["mean_rel"], (dev, eff)
        assert 0.8 * eff["mean_rel"] <= own["mean_rel"] <= 1.25 * eff["mean_rel"], (own, eff)
        assert abs(np.abs(g_all[b]).mean() / s8["abs_mean_all"] - 1) < 1e-2
