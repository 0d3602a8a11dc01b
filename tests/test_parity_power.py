"""CPU check that the attention parity bar can see a wrong softmax: on the
stress inputs, replacing softmax attention by the plain mean of V (or by a
softmax without the 1/sqrt(hd) scale) must fail the comparison used by the
GPU tests."""
import numpy as np

import oracle.wan_oracle as O
import synth
from tests.gpu_util_cpu import metrics


def test_stress_inputs_reject_mean_of_v():
    q, k, v = synth.attention_inputs(1, 1, 2, 300, 100)
    ref = np.stack([O.multihead(q[0], k[0], v[0], 2)])
    mean_v = np.broadcast_to(v.mean(axis=1, keepdims=True), ref.shape)
    m = metrics(mean_v, ref)
    assert m["max_abs"] > 3e-2 and m["mean_rel"] > 1e-2, m


def test_stress_inputs_reject_unscaled_softmax():
    q, k, v = synth.attention_inputs(1, 1, 2, 300, 100)
    ref = O.multihead(q[0], k[0], v[0], 2)
    bad = O.multihead(q[0] * np.sqrt(128.0), k[0], v[0], 2)   # drops the 1/sqrt(hd)
    m = metrics(bad, ref)
    assert m["max_abs"] > 3e-2 and m["mean_rel"] > 1e-2, m


def test_full_length_inputs_reject_mean_of_v_and_unscaled_softmax():
    """The full-length stress inputs (12 heads x 32760 tokens, peaked logits
    with raised key runs) on 64 sampled query rows: the plain mean of V and a
    softmax without the 1/sqrt(hd) scale both fail the GPU tests' bar."""
    from tests.attn_full_inputs import full_inputs, sampled_rows
    H, L = 12, 32760
    q, k, v = full_inputs(H, L, threads=8)
    rows = sampled_rows(L, n=64)
    ref = O.multihead(q[rows], k, v, H)
    mean_v = np.broadcast_to(v.astype(np.float64).mean(axis=0, keepdims=True), ref.shape)
    m = metrics(mean_v, ref)
    assert m["max_abs"] > 3e-2 and m["mean_rel"] > 1e-2, m
    bad = O.multihead(q[rows] * np.sqrt(128.0), k, v, H)
    m = metrics(bad, ref)
    assert m["max_abs"] > 3e-2 and m["mean_rel"] > 1e-2, m


def test_cross_inputs_reject_mean_of_v_and_unscaled_softmax():
    """The cross-attention stress inputs (512 text keys, 257 image keys; the
    rows are independent, so 256 query rows show it): the plain mean of V and
    a softmax without the 1/sqrt(hd) scale both fail the GPU tests' bar."""
    from tests.attn_full_inputs import cross_inputs
    for H, Lk in [(12, 512), (40, 257)]:
        q, k, v = cross_inputs(H, 256, Lk, threads=8)
        ref = O.multihead(q, k, v, H)
        mean_v = np.broadcast_to(v.astype(np.float64).mean(axis=0, keepdims=True), ref.shape)
        m = metrics(mean_v, ref)
        assert m["max_abs"] > 3e-2 and m["mean_rel"] > 1e-2, m
        m = metrics(O.multihead(q * np.sqrt(128.0), k, v, H), ref)
        assert m["max_abs"] > 3e-2 and m["mean_rel"] > 1e-2, m


def test_attn8_fixed_bar_rejects_mean_of_v_and_passes_the_oracle():
    """The 8-bit attention tests' fixed bar (mean relative error against exact
    attention): the oracle's own 8-bit attention passes it on every parity
    input, and the plain mean of V fails it on each of them."""
    from tests.test_gpu_attn8 import ATTN8_MEAN_REL, CASES
    for qk_std in (1.0, 2.0):
        for B, H, Lq, Lk in CASES:
            if Lk == 1:   # one key: every attention is V itself
                continue
            q, k, v = synth.attention_inputs(12, B, H, Lq, Lk, qk_std=qk_std)
            ex = np.stack([O.multihead(q[b], k[b], v[b], H) for b in range(B)])
            o8 = np.stack([O.multihead_8bit(q[b], k[b], v[b], H) for b in range(B)])
            assert metrics(o8, ex)["mean_rel"] <= ATTN8_MEAN_REL / 2, (B, H, Lq, Lk, qk_std)
            mean_v = np.broadcast_to(v.astype(np.float64).mean(axis=1, keepdims=True), ex.shape)
            assert metrics(mean_v, ex)["mean_rel"] > 5 * ATTN8_MEAN_REL, (B, H, Lq, Lk, qk_std)
