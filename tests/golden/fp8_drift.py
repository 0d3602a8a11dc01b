"""How far two correct FP8 runs of a deep DiT drift apart (CPU, float64 oracle).

Runs the oracle's step blocks at the 1.3B width (d = 1536, 12 heads, FFN
8960; [Note, 配置表]) on a short clip (latent 3 x 16 x 32, L = 384, 30
blocks) three ways: exact, with every block's Linear layers in FP8 (E4M3,
[Note] Infra / 推理优化), and in FP8 with bf16-level noise (relative 2^-9)
added to the hidden state after every block -- the size of the last-place
differences two correct implementations of the bf16 block show.  At chosen
depths it prints, for the head's velocity: the FP8 effect (FP8 vs exact),
the drift between the two FP8 runs, their ratio, and the perturbed run's own
FP8 effect relative to the unperturbed one.  It calls only ``oracle/`` and
``synth/``; the full-size FP8 step test's bar rests on these ratios.

Measured (about 10 minutes on 8 cores): drift / effect 0.67 after 1 block,
0.83 after 5, 0.84 - 0.87 from 10 to 30 blocks (0.86 at 30); each FP8 run's own effect
0.99 - 1.00 of the other's.

Usage: python -m tests.golden.fp8_drift
"""
import numpy as np

import oracle.wan_oracle as O
import synth

DEPTHS = (1, 2, 5, 10, 15, 20, 25, 30)


def _mean_rel(a, b):
    return float(np.abs(a - b).sum() / np.abs(b).sum())


def main():
    w = synth.mini(78, "fp8-drift-1536", dim=1536, heads=12, ffn=8960, n_blocks=30, lat_f=3,
                   lat_h=16, lat_w=32, batch=1, text_len=64)
    inp = synth.workload_inputs(w)
    mw = synth.model_weights(w)
    x = O.patchify(inp["latent"], mw["patch_w"], mw["patch_b"])
    tw = mw["tmlp"]
    m = O.tmlp(inp["t"], tw["w1"], tw["b1"], tw["w2"], tw["b2"])
    rng = np.random.default_rng(0)

    def perturb(a):
        return a * (1 + 2.0 ** -9 * rng.standard_normal(a.shape))

    def head(a):
        return O.head_unpatchify(a, mw["head_w"], mw["head_b"], w.lat_f, w.Hp, w.Wp, 16)

    xe, x8, x8p = x.copy(), x.copy(), perturb(x)
    print(f"L = {w.L}, {w.model.n_blocks} blocks at d = {w.model.dim}", flush=True)
    for i, wts in enumerate(mw["blocks"]):
        xe = O.block(xe, m, wts, inp["ctx"], w.model.heads, w.model.eps)
        x8 = O.block(x8, m, wts, inp["ctx"], w.model.heads, w.model.eps, fp8=True)
        x8p = perturb(O.block(x8p, m, wts, inp["ctx"], w.model.heads, w.model.eps, fp8=True))
        if i + 1 in DEPTHS:
            ve, v8, v8p = head(xe), head(x8), head(x8p)
            eff, drift = _mean_rel(ve, v8), _mean_rel(v8p, v8)
            print(f"depth {i + 1:2d}: FP8 effect {eff:.4f}, drift between the FP8 runs {drift:.4f} "
                  f"(ratio {drift / eff:.2f}); perturbed run's own effect "
                  f"{_mean_rel(v8p, ve) / eff:.2f} x", flush=True)


if __name__ == "__main__":
    main()
