"""Host-side checks of libppx that need no GPU: the library loads, exports
every function include/ppx.h declares, and its host logic (prune predicate,
KVCP file validation) agrees with the pages' rules and with the oracle."""
import json
import os
import re

import numpy as np
import pytest

import oracle
import prompt_prefill_cross_amd as ppx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLD = os.path.join(ROOT, "tests", "golden")


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(ppx.LIB_PATH):
        from prompt_prefill_cross_amd import build
        build.build(verbose=False)
    return ppx.lib()


def header_functions():
    src = open(os.path.join(ROOT, "include", "ppx.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ppx_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 20
    lib = ppx.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_binding_covers_the_header():
    bound = {n for n, _, _ in ppx.SIGNATURES}
    assert set(header_functions()) == bound


def test_status_strings():
    for st in ppx.STATUS:
        assert ppx.lib().ppx_status_str(st)


def test_prune_predicate_truth_table_via_c_abi():
    g = json.load(open(os.path.join(GOLD, "prune_predicate.json")))
    for c in g["cases"]:
        L = c["n_layer"]
        inp = np.zeros(L + 1, np.uint8)
        inp[c["layer_inp_true"]] = 1
        got = ppx.prune_predicate(L, c["n_layer_kv_from_start"], c["embeddings"], c["n_seq_max"], inp,
                                  c["crop_before_nextn"])
        assert got == c["expected"], c["note"]


def _statuses(path, nl, kvd, n_pos, n_ctx):
    st, fpos = ppx.kvfile_validate(path, nl, kvd, n_pos, n_ctx)
    try:
        oracle.kvcp.load(open(path, "rb").read(), nl, kvd, n_pos, n_ctx)
        ok = True
    except oracle.kvcp.SnapshotError:
        ok = False
    return st, ok, fpos


def test_kvfile_validation_matches_oracle(tmp_path):
    rng = np.random.default_rng(7)
    K = rng.standard_normal((3, 10, 64)).astype(np.float16)
    V = rng.standard_normal((3, 10, 64)).astype(np.float16)
    good = tmp_path / "good.kvc"
    good.write_bytes(oracle.kvcp.dump(K, V, 10))
    st, ok, fpos = _statuses(str(good), 3, 64, 10, 32)
    assert st == 0 and ok and fpos == 10
    assert _statuses(str(good), 3, 64, 4, 32)[:2] == (0, True)  # a prefix of the file
    cases = {
        "bad_magic": (b"KVCX" + good.read_bytes()[4:], 3, 64, 4, 32, -5),
        "truncated": (good.read_bytes()[:-2], 3, 64, 4, 32, -5),
        "layers": (good.read_bytes(), 2, 64, 4, 32, -6),
        "kv_dim": (good.read_bytes(), 3, 32, 4, 32, -6),
        "too_many_pos": (good.read_bytes(), 3, 64, 11, 32, -5),
        "over_n_ctx": (good.read_bytes(), 3, 64, 10, 8, -3),
        "header_only": (good.read_bytes()[:10], 3, 64, 1, 32, -5),
    }
    for name, (data, nl, kvd, n, nctx, want) in cases.items():
        p = tmp_path / f"{name}.kvc"
        p.write_bytes(data)
        st, ok, _ = _statuses(str(p), nl, kvd, n, nctx)
        assert st == want and not ok, name
    assert ppx.kvfile_validate(str(tmp_path / "missing.kvc"), 3, 64, 1, 32)[0] == -4


def test_kvcp_size_pin_via_engine_rule(tmp_path):
    # the engine accepts exactly 16 + 563,200 bytes for TinyLlama's 22 layers x 25 positions x 256
    g = json.load(open(os.path.join(GOLD, "kvcp_tinyllama_25.json")))
    K = np.zeros((22, 25, 256), np.float16)
    p = tmp_path / "t.kvc"
    p.write_bytes(oracle.kvcp.dump(K, K, 25))
    assert os.path.getsize(p) - 16 == g["payload_bytes"]
    assert ppx.kvfile_validate(str(p), 22, 256, 25, 2048)[0] == 0


def test_kvfile_with_token_section_matches_oracle(tmp_path):
    """A snapshot may end with a token section ("KVTK", int32 count = n_pos,
    the ids); the engine's check and the oracle's reader accept and reject
    the same files."""
    rng = np.random.default_rng(11)
    K = rng.standard_normal((3, 6, 64)).astype(np.float16)
    V = rng.standard_normal((3, 6, 64)).astype(np.float16)
    ids = [5, 9, 9, 2, 7, 1]
    good = tmp_path / "tok.kvc"
    good.write_bytes(oracle.kvcp.dump_tokens(K, V, 6, ids))
    st, ok, fpos = _statuses(str(good), 3, 64, 6, 32)
    assert st == 0 and ok and fpos == 6
    assert oracle.kvcp.stored_tokens(good.read_bytes()) == ids
    body = len(oracle.kvcp.dump(K, V, 6))
    data = good.read_bytes()
    cases = {
        "bad_token_magic": data[:body] + b"KVTX" + data[body + 4:],
        "count_mismatch": data[:body + 4] + np.int32(5).tobytes() + data[body + 8:],
        "missing_id": data[:-4],
        "extra_bytes": data + b"\0\0\0\0",
    }
    for name, d in cases.items():
        p = tmp_path / f"{name}.kvc"
        p.write_bytes(d)
        st, ok, _ = _statuses(str(p), 3, 64, 6, 32)
        assert st == -5 and not ok, name


def test_reusable_prefix_rule_brute_force():
    """oracle.kvcp.reusable_prefix against a direct search: the longest l with
    equal first l ids, at most len(prompt) - 1 and n_ctx."""
    rng = np.random.default_rng(3)
    for _ in range(2000):
        stored = list(rng.integers(0, 3, rng.integers(0, 7)))
        prompt = list(rng.integers(0, 3, rng.integers(1, 8)))
        n_ctx = int(rng.integers(1, 9))
        cap = min(len(stored), len(prompt) - 1, n_ctx)
        want = max(l for l in range(cap + 1) if stored[:l] == prompt[:l])
        assert oracle.kvcp.reusable_prefix(stored, prompt, n_ctx) == want


def test_model_weight_bytes_host_only():
    """ppx_model_weight_bytes lays a container out without a GPU: the repacked
    weights take the container's tensor bytes (Q4_0 18 B per 32 weights, fp32
    gains and the raw per-layer-embedding table) plus 256-byte alignment per
    array; a damaged container gives 0."""
    import ctypes
    import synth
    L = ppx.lib()
    for name in ("tiny", "tinyllama"):
        buf = synth.build_model(name)
        m = oracle.parse_model(buf)
        tensor_bytes = sum(t.rows * t.cols * (4 if t.ttype == 0 else 18 // 2) // (1 if t.ttype == 0 else 16)
                           for t in m.tensors.values())
        need = L.ppx_model_weight_bytes(ctypes.c_void_p(buf.ctypes.data), buf.nbytes)
        assert tensor_bytes <= need <= tensor_bytes + 2 * 256 * (len(m.tensors) + 1), (name, need, tensor_bytes)
        assert need == L.ppx_model_weight_bytes(ctypes.c_void_p(buf.ctypes.data), buf.nbytes)
    bad = buf.copy()
    bad[:4] = 0
    assert L.ppx_model_weight_bytes(ctypes.c_void_p(bad.ctypes.data), bad.nbytes) == 0
    assert L.ppx_model_weight_bytes(ctypes.c_void_p(buf.ctypes.data), 100) == 0
    assert L.ppx_model_weight_bytes(None, 0) == 0

