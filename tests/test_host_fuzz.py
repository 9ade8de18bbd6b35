"""Sanitizer fuzz of the host parsers that read untrusted files (CPU only).

The model container parser and the KVCP snapshot check are built with
AddressSanitizer and UndefinedBehaviorSanitizer on the host side
(prompt_prefill_cross_amd/build.py, build_fuzz) and driven with thousands of
mutated inputs derived from a valid container and a valid snapshot (a token
section included): header fields set to boundary values, bit flips,
truncation, extension.  Every input must come back with a status; any
out-of-bounds access, integer overflow or leak aborts the driver with a
sanitizer report, which fails the test.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import synth


@pytest.fixture(scope="module")
def driver():
    if not os.path.exists(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")) and not shutil.which("hipcc"):
        pytest.skip("hipcc is not available")
    from prompt_prefill_cross_amd import build as b
    return b.build_fuzz(verbose=False)


@pytest.mark.parametrize("seed", [11, 12])
def test_parsers_survive_mutated_inputs(driver, tmp_path, seed):
    model = tmp_path / "tiny.ppxm"
    model.write_bytes(synth.build_model("tiny").tobytes())
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((2, 24, 64)).astype(np.float16)
    snap = tmp_path / "seed.kvc"
    snap.write_bytes(oracle.kvcp.dump_tokens(K, K, 24, list(range(100, 124))))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=87")
    r = subprocess.run([driver, str(model), str(snap), str(tmp_path / "scratch.kvc"), "2000", str(seed)],
                       capture_output=True, text=True, timeout=600, env=env)
    print(r.stdout)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "container: 2000 mutated inputs" in r.stdout and "snapshot: 2000 mutated inputs" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
