"""Integrity of the stored full-step goldens (CPU only): each file belongs to
its workload, its indices are the writer's seeded sample (regenerated here
without running the oracle), its values are finite and within the recorded
extremes, and it names the command that wrote it.  A golden that is not
written yet is skipped."""
import json
import os

import numpy as np
import pytest

from tests.golden.make_full_step_golden import N_SAMPLED, WORKLOADS, golden_path, sample_index

# every workload exactly; the 1.3B guidance pair also with FP8 blocks
CASES = [(cid, False) for cid in sorted(WORKLOADS)] + [(3, True)]


@pytest.mark.parametrize("cid,fp8", CASES)
def test_step_golden_integrity(cid, fp8):
    path = golden_path(cid, fp8)
    if not os.path.exists(path):
        pytest.skip(f"{os.path.basename(path)} not written")
    with open(path) as f:
        g = json.load(f)
    w = WORKLOADS[cid]
    shape = [w.batch, 16, w.lat_f, w.lat_h, w.lat_w]
    assert g["config_id"] == cid and g["workload"] == w.name
    assert g["output_shape"] == shape and g["per_sample_shape"] == shape[1:]
    assert g["writer"] == f"python -m tests.golden.make_full_step_golden --config {cid}" + (" --fp8" if fp8 else "")
    assert ("FP8" in g["what"]) == fp8
    idx = sample_index(cid, shape)
    assert len(g["samples"]) == w.batch
    for b, s in enumerate(g["samples"]):
        assert s["flat_index"] == idx[b].tolist()
        v = np.asarray(s["value"])
        assert v.shape == (N_SAMPLED,) and np.all(np.isfinite(v))
        assert np.max(np.abs(v)) <= s["abs_max_all"] and 0 < s["abs_mean_all"] <= s["abs_max_all"]
