"""Write oracle results for the large configs to tests/golden/.

Calls only the fp64 oracle (oracle/) on the seeded inputs of `synth`; the
GPU parity tests compare the HIP path against these files instead of
re-running the oracle (minutes to hours at these sizes) inside the test.
Each file holds the last-row logits
(fp32, all n_vocab), the fp16 K and V rows of 32 sampled positions (first
and last included) in every KV-owning layer, and the run's metadata.

    python tests/golden/make_goldens.py [name ...]      (names below)
"""
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synth  # noqa: E402

CASES = {
    "tinyllama_512": ("tinyllama", 512),
    "e2b_512": ("e2b", 512),
    "e2b_2048": ("e2b", 2048),
    "e4b_512": ("e4b", 512),
    "e2b_8192": ("e2b", 8192),
    "e4b_2048": ("e4b", 2048),
    "e2b_ctrl_8192": ("e2b_ctrl", 8192),
    "e2b_long_16384": ("e2b_long", 16384),
    "e4b_8192": ("e4b", 8192),
    "e2b_long_32768": ("e2b_long", 32768),
}


def path_of(name):
    return os.path.join(HERE, f"oracle_{name}.npz")


def make(name):
    cfg, n = CASES[name]
    c = synth.CONFIGS[cfg]
    m = oracle.parse_model(synth.build_model(c))
    toks = synth.prompt(c, n)
    kv = oracle.KVState(m, n)
    t = time.time()
    logits = oracle.prefill(m, kv, toks, prune=0 < c.n_layer_kv_from_start < c.n_layer)
    dt = time.time() - t
    rng = np.random.default_rng([7, n])
    pos = np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=min(30, n), replace=False)]))
    layers = np.arange(c.n_layer_kv_from_start, dtype=np.int64)
    meta = {"config": cfg, "n": n, "model_seed": c.seed, "oracle_seconds": round(dt, 1),
            "numpy": np.__version__, "source": "oracle.prefill (fp64) on synth.build_model / synth.prompt"}
    np.savez(path_of(name), logits=logits.astype(np.float32), kv_pos=pos.astype(np.int64),
             kv_layers=layers, K=kv.K[layers][:, pos], V=kv.V[layers][:, pos], meta=np.array(json.dumps(meta)))
    print(f"{name}: {dt:.1f} s", flush=True)


if __name__ == "__main__":
    names = sys.argv[1:] or list(CASES)
    for nm in names:
        if os.path.exists(path_of(nm)) and "--force" not in sys.argv:
            print(f"{nm}: exists", flush=True)
            continue
        if nm.startswith("--"):
            continue
        make(nm)
