"""Consistency of the stored oracle values (tests/golden/oracle_*.npz, written by
tests/golden/make_oracle_fixtures.py from the oracle alone): the configuration they were written
for is the one the tests use, every array has its shape, the recorded maxima are maxima of what
is stored, and the losses start near ln V (random weights of std 0.02 give almost uniform
next-token distributions) and stay finite."""
import json
import math
import os

import numpy as np
import pytest

from tests.cfgs import M125, M3B
from tests.golden import make_oracle_fixtures as fx


@pytest.mark.parametrize("name,cfg", [("125m", M125), ("3b", M3B)])
def test_fixture_consistent(name, cfg):
    path = fx.fixture_path(name)
    if not os.path.exists(path):
        pytest.skip(f"{os.path.basename(path)} not generated yet")
    with np.load(path, allow_pickle=False) as z:
        d = {k: z[k] for k in z.files}
    meta = json.loads(str(d["meta"]))
    assert meta["config"] == dict(cfg)
    assert meta["chunks"] == fx.WORKLOADS[name]["chunks"] and meta["tokens"] == meta["chunks"] * cfg["chunk"]
    assert meta["samples"] == fx.SAMPLES and meta["sample_seed"] == fx.SAMPLE_SEED
    nt = 3 * cfg["n_fast"]
    assert d["losses"].shape == (meta["chunks"],) and np.all(np.isfinite(d["losses"]))
    for k in ("phi_absmax", "dw_absmax", "dw_argmax", "dw_at_argmax"):
        assert d[k].shape == (nt,), k
    assert d["dw_samples"].shape == (nt, fx.SAMPLES)
    sizes = fx.fast_tensor_sizes(cfg)
    assert np.all(d["dw_argmax"] >= 0) and np.all(d["dw_argmax"] < np.array(sizes))
    np.testing.assert_array_equal(np.abs(d["dw_at_argmax"]), d["dw_absmax"])
    assert np.all(np.max(np.abs(d["dw_samples"]), axis=1) <= d["dw_absmax"])
    assert np.all(d["dw_absmax"] > 0) and np.all(d["phi_absmax"] > d["dw_absmax"])
    lnv = math.log(cfg["vocab"])
    assert abs(d["losses"][0] - lnv) < 0.05 * lnv
