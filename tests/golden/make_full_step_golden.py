"""Write sampled velocity elements of the two full-size denoising steps.

Runs the CPU oracle (``oracle/wan_oracle.py``, float64) on the seeded inputs
of ``synth`` and stores, for each workload, a seeded sample of output
elements with their indices.  It calls only ``oracle/`` and ``synth/``; no
value here comes from the HIP path.

Workloads:
  * ``wan1.3b-step-480p-cfg2``: the 1.3B-shaped step, 30 blocks, a pair of
    samples with the same latent and timestep and two text contexts
    ([Note, 配置表] for the widths; [Guide, 工作原理] for the guidance pair);
  * ``wan14b-i2v-step-480p``: the 14B-shaped image-to-video step, 40 blocks,
    36 input channels (noise, condition latent, the 4 mask channels of a video
    whose first frame is given), 257 image tokens through the image MLP
    ([Note, I2V 架构扩展]; [News, 核心创新四]).

  * ``wan14b-i2v-step-short``: the same 14B image-to-video step on a short
    clip (latent 21 x 8 x 8, L = 336 tokens), full width and depth.

Usage (hours of CPU time at float64 for 3 and 5, minutes for 53; each
workload is independent):

    python -m tests.golden.make_full_step_golden --config 3
    python -m tests.golden.make_full_step_golden --config 5
    python -m tests.golden.make_full_step_golden --config 53
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

import oracle.wan_oracle as O
import synth

HERE = os.path.dirname(os.path.abspath(__file__))
N_SAMPLED = 4096          # output elements stored per batch sample


# the 14B image-to-video model at its full width and depth on a short clip
# (latent 21 x 8 x 8, L = 336 tokens): small enough for the oracle to take
# minutes, so the step can also be compared in float32
SHORT_I2V = synth.mini(53, "wan14b-i2v-step-short", dim=5120, heads=40, ffn=13824, n_blocks=40,
                       lat_f=21, lat_h=8, lat_w=8, batch=1, text_len=512, in_ch=36, img_len=257)
WORKLOADS = {3: synth.by_id(3), 5: synth.by_id(5), 53: SHORT_I2V}


def golden_path(cid: int, fp8: bool = False) -> str:
    return os.path.join(HERE, f"step_{WORKLOADS[cid].name}{'-fp8' if fp8 else ''}.json")


def step_inputs(cid: int):
    """The latent, timestep, text context and image features of a full-size
    step workload, exactly as the GPU test builds them.  The I2V mask
    channels are the expansion of a binary mask over the 81 video frames with
    only frame 0 given."""
    w = WORKLOADS[cid]
    inp = synth.workload_inputs(w)
    lat = inp["latent"]
    if w.model.in_ch > 16:
        frames = 1 + 4 * (w.lat_f - 1)
        fm = np.zeros(frames)
        fm[0] = 1
        lat[:, 32:36] = O.i2v_mask(fm, w.lat_f, w.lat_h, w.lat_w)
    return lat, inp["t"], inp["ctx"], inp.get("clip")


def sample_index(cid: int, shape):
    """Seeded flat indices (without replacement) of the stored elements of
    each batch sample of an output [B, C, F, H8, W8]."""
    g = np.random.default_rng([2025, cid, 777])
    per = int(np.prod(shape[1:]))
    return [np.sort(g.choice(per, size=N_SAMPLED, replace=False)) for _ in range(shape[0])]


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, choices=tuple(WORKLOADS), required=True)
    ap.add_argument("--head-threads", type=int, default=os.cpu_count() or 1)
    ap.add_argument("--fp8", action="store_true",
                    help="every block's six Linear layers in FP8 (E4M3, the oracle's emulation)")
    a = ap.parse_args(argv)
    cid = a.config
    w = WORKLOADS[cid]
    m = w.model
    O.HEAD_THREADS = a.head_threads
    t0 = time.perf_counter()
    lat, t, ctx, clip = step_inputs(cid)
    mw = synth.model_weights(w, with_blocks=False)
    print(f"[golden C{cid}] inputs drawn in {time.perf_counter() - t0:.1f}s", flush=True)

    def blocks():
        for i in range(m.n_blocks):
            tb = time.perf_counter()
            yield synth.block_weights(w, i)
            print(f"[golden C{cid}] block {i + 1}/{m.n_blocks} done "
                  f"({time.perf_counter() - tb:.0f}s, {time.perf_counter() - t0:.0f}s total)",
                  flush=True)

    out = O.step(lat, t, ctx, mw, m.heads, eps=m.eps, clip=clip, blocks=blocks(), fp8=a.fp8)
    idx = sample_index(cid, out.shape)
    per = out.shape[1:]
    samples = []
    for b in range(out.shape[0]):
        flat = out[b].reshape(-1)
        samples.append({
            "flat_index": idx[b].tolist(),
            "value": [float(v) for v in flat[idx[b]]],
            "abs_mean_all": float(np.mean(np.abs(flat))),
            "abs_max_all": float(np.max(np.abs(flat))),
        })
    rec = {
        "what": f"velocity of the {w.name} denoising step{' with FP8 blocks' if a.fp8 else ''}, "
                "sampled elements (float64 oracle)",
        "workload": w.name, "config_id": cid,
        "output_shape": list(out.shape), "per_sample_shape": list(per),
        "index_order": "flat index into one sample's [C, F, H8, W8] velocity (row-major)",
        "writer": "python -m tests.golden.make_full_step_golden --config %d%s" % (cid, " --fp8" if a.fp8 else ""),
        "oracle_seconds": round(time.perf_counter() - t0, 1),
        "samples": samples,
    }
    with open(golden_path(cid, a.fp8), "w") as f:
        json.dump(rec, f)
    print(f"[golden C{cid}] wrote {golden_path(cid, a.fp8)} after {time.perf_counter() - t0:.0f}s", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
