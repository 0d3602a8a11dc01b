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
