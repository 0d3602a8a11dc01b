"""The oracle against its pins (closed forms, library routines, brute force,
invariants).  CPU only."""
import json
import os

import numpy as np
import pytest

import oracle.wan_oracle as O
from tests import oracle_pins as P

PINS = [getattr(P, n) for n in dir(P) if n.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(O)


def test_param_counts_match_model_names():
    """Block = 4d^2 (SA) + 4d^2 (CA) + 2dF (FFN) plus biases, a shared t-MLP
    256->d->6d, a per-block 6d bias: the totals must come out near the model
    names, and a per-block (unshared) d->6d AdaLN layer must cost about the
    quoted 25%."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "model_table.json")) as f:
        g = json.load(f)
    for m in g["models"]:
        d, F, n = m["dim"], m["ffn"], m["layers"]
        blk = (3 * d * d + 3 * d) + (d * d + d) + (d * d + d) + (2 * d * d + 2 * d) + (d * d + d) \
            + (F * d + F) + (d * F + d) + 6 * d
        shared = (256 * d + d) + (6 * d * d + 6 * d)
        io = (16 * 4 * d + d) + (d * 16 * 4 + 16 * 4)
        total = n * blk + shared + io
        assert abs(total / m["total_params"] - 1) < 0.10, (m["name"], total)
        unshared_extra = n * 6 * d * d
        assert abs(unshared_extra / (total + unshared_extra) - g["adaln_sharing_saving"]) < 0.06


def test_threaded_heads_match_sequential():
    """The optional head thread pool changes no arithmetic."""
    r = np.random.default_rng(3)
    q, k, v = (r.normal(size=(70, 4 * 32)) for _ in range(3))
    ref = O.multihead(q, k, v, 4)
    old = O.HEAD_THREADS
    try:
        O.HEAD_THREADS = 3
        got = O.multihead(q, k, v, 4)
    finally:
        O.HEAD_THREADS = old
    assert np.max(np.abs(got - ref)) <= 1e-12
