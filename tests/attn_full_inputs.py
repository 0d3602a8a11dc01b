"""Seeded inputs of the full-length attention stress tests (shared by the GPU
parity tests and the CPU check that their bar rejects a wrong softmax)."""
import numpy as np

import synth


def outlier_ranges(L):
    """Key runs whose logits are raised: in the first tile, mid-stream, and
    in the last (ragged) tile."""
    return [(3, 19), (L // 2 + 7, L // 2 + 23), (L - 21, L - 5)]


def sampled_rows(L, n=1024, seed=0):
    fixed = [0, 1, 31, 32, 255, 256, 511, L // 2, L - 256, L - 2, L - 1, (L // 256) * 256,
             (L // 256) * 256 - 1]
    rng = np.random.default_rng([seed, L])
    return np.unique(np.concatenate([fixed, rng.integers(0, L, n - len(fixed))]))


def full_inputs(H, L, threads=16):
    q, k, v = synth.attention_inputs_full(5, H, L, qk_std=2.0, threads=threads)
    for a, b in outlier_ranges(L):
        k[a:b] = synth.bf16_round(k[a:b] * np.float32(2.5))
    return q, k, v


def cross_inputs(H, Lq, Lk, threads=16):
    """Cross-attention stress inputs at the block's real shapes: queries of the
    full token sequence (q ~ N(0, 4)) against Lk context keys (k ~ N(0, 4),
    v ~ N(0, 1)), with the same raised key runs scaled to the short context."""
    q, _, _ = synth.attention_inputs_full(7, H, Lq, qk_std=2.0, threads=threads)
    _, k, v = synth.attention_inputs_full(8, H, Lk, qk_std=2.0, threads=threads)
    for a, b in [(3, 11), (Lk // 2, Lk // 2 + 8), (Lk - 9, Lk - 1)]:
        k[a:b] = synth.bf16_round(k[a:b] * np.float32(2.5))
    return q, k, v
