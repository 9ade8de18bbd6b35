"""The stored oracle results (tests/golden/oracle_*.npz) on the CPU: each
file belongs to the case tests/golden/make_goldens.py names for it, holds the
full last-row logits and the K and V rows of every KV-owning layer at the
sampled positions (the first and the last included), and those rows are
finite fp16 values of the config's KV width.  The GPU parity tests read these
files; this checks that none of them is stale or partial."""
import json
import os
import sys

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(HERE, "golden"))

import make_goldens  # noqa: E402
import synth  # noqa: E402


@pytest.mark.parametrize("name", sorted(make_goldens.CASES))
def test_golden_file_matches_its_case(name):
    path = make_goldens.path_of(name)
    if not os.path.exists(path):
        pytest.skip(f"{path} not written")
    cfg_name, n = make_goldens.CASES[name]
    c = synth.CONFIGS[cfg_name]
    g = np.load(path)
    meta = json.loads(str(g["meta"]))
    assert meta["config"] == cfg_name and meta["n"] == n and meta["model_seed"] == c.seed
    assert g["logits"].shape == (c.n_vocab,) and np.isfinite(g["logits"]).all()
    assert np.array_equal(g["kv_layers"], np.arange(c.n_layer_kv_from_start))
    pos = g["kv_pos"]
    assert pos[0] == 0 and pos[-1] == n - 1 and np.all(np.diff(pos) > 0) and len(pos) == min(32, n)
    kvd = c.n_kv_head * c.head_dim
    for key in ("K", "V"):
        a = g[key]
        assert a.dtype == np.float16 and a.shape == (c.n_layer_kv_from_start, len(pos), kvd)
        assert np.isfinite(a).all()
