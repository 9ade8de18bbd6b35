"""Token-verified prefix reuse: a snapshot with the token ids of its cached
positions, from which ppx_kv_load_prefix loads the longest common prefix with
a new prompt (leaving at least one token to run).  The resumed prefill must
equal a full prefill of the new prompt -- against the fp64 oracle on the tiny
model (with a prompt that diverges midway) and against the stored oracle
result of the E2B-like 2048-token prompt (reusing 2047 positions)."""
import os

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import container, kv_within, logits_ok, oracle_model

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def ppx():
    import prompt_prefill_cross_amd as p
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    p.lib()
    return p


_models = {}


def engine_model(ppx, name):
    if name not in _models:
        _models.clear()
        torch.cuda.synchronize()
        _models[name] = ppx.Model(container(name))
    return _models[name]


def test_prefix_reuse_vs_oracle_tiny(ppx, tmp_path):
    cfg, n0, keep = "tiny", 48, 30
    a = synth.prompt(cfg, n0)
    mm = engine_model(ppx, cfg)
    V = mm.info["n_vocab"]
    b = np.concatenate([a[:keep], (a[keep:keep + 16] + 1) % V]).astype(np.int32)
    kv = ppx.KVCache(mm, 64)
    # exact precision: every owning layer's cache is compared with the oracle's
    # (the fp16-operand path cannot hold this model's layer 1 to the bound)
    mm.prefill(a, kv, n_ubatch=16, precision="exact")
    snap = str(tmp_path / "a.kvc")
    kv.save_tokens(snap, a)
    kv2 = ppx.KVCache(mm, 64)
    L = kv2.load_prefix(snap, b)
    assert L == keep and kv2.n_pos == keep
    got = mm.prefill(b[L:], kv2, n_ubatch=16, precision="exact").cpu().numpy().astype(np.float64)
    om = oracle_model(cfg)
    okv = oracle.KVState(om, len(b))
    ref = oracle.prefill(om, okv, b, prune=True).astype(np.float64)
    ok, d = logits_ok(got, ref)
    print(f"tiny reuse {L} of {len(b)}: logits max-abs {d:.3e}")
    assert ok, d
    K, Vc = kv2.kv_tensors()
    for g, want in ((K[:, :len(b)], okv.K[:, :len(b)]), (Vc[:, :len(b)], okv.V[:, :len(b)])):
        okk, dk = kv_within(g.cpu().numpy(), want)
        assert okk, dk


def test_prefix_reuse_identical_prompt_e2b_2048(ppx, tmp_path):
    import json
    path = os.path.join(GOLD, "oracle_e2b_2048.npz")
    if not os.path.exists(path):
        pytest.skip(f"no stored oracle result {path}")
    g = np.load(path)
    meta = json.loads(str(g["meta"]))
    cfg, n = meta["config"], meta["n"]
    toks = synth.prompt(cfg, n)
    mm = engine_model(ppx, cfg)
    kv = ppx.KVCache(mm, n)
    mm.prefill(toks, kv, n_ubatch=512)
    snap = str(tmp_path / "e2b.kvc")
    kv.save_tokens(snap, toks)
    del kv
    kv2 = ppx.KVCache(mm, n)
    L = kv2.load_prefix(snap, toks)
    assert L == n - 1
    lg = mm.prefill(toks[L:], kv2, n_ubatch=512).cpu().numpy().astype(np.float64)
    ok, d = logits_ok(lg, g["logits"])
    print(f"e2b 2048 reusing {L}: logits max-abs {d:.3e}")
    assert ok, d


def test_prefix_reuse_edges(ppx, tmp_path):
    cfg = "tiny"
    mm = engine_model(ppx, cfg)
    V = mm.info["n_vocab"]
    a = synth.prompt(cfg, 20)
    kv = ppx.KVCache(mm, 32)
    mm.prefill(a, kv, n_ubatch=16)
    tok_snap, plain = str(tmp_path / "t.kvc"), str(tmp_path / "p.kvc")
    kv.save_tokens(tok_snap, a)
    kv.save(plain)
    kv2 = ppx.KVCache(mm, 32)
    # diverging at the first token: nothing reused
    assert kv2.load_prefix(tok_snap, np.r_[(a[0] + 1) % V, a[1:]]) == 0 and kv2.n_pos == 0
    # a one-token prompt leaves that token to run
    assert kv2.load_prefix(tok_snap, a[:1]) == 0
    # a prompt shorter than the snapshot: all but its last token
    assert kv2.load_prefix(tok_snap, a[:12]) == 11 and kv2.n_pos == 11
    # a prompt longer than the snapshot: the whole snapshot
    assert kv2.load_prefix(tok_snap, np.r_[a, a[:5]]) == 20 and kv2.n_pos == 20
    # a snapshot without token ids cannot be verified: an error, cache empty
    with pytest.raises(ppx.PPXError) as e:
        kv2.load_prefix(plain, a)
    assert e.value.status == -5 and kv2.n_pos == 0
    # the plain loader still reads a snapshot that carries a token section
    kv2.load(tok_snap, 20)
    assert kv2.n_pos == 20
    K1, V1 = kv.kv_tensors()
    K2, V2 = kv2.kv_tensors()
    assert torch.equal(K1[:, :20], K2[:, :20]) and torch.equal(V1[:, :20], V2[:, :20])
