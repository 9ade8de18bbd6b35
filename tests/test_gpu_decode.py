"""The decode step (ppx_decode): one generated token after a prefill, on the
single-row path, appending K/V in the owning layers.  Its result is defined
as the prefill of that one token at position n_pos (the pages' generation
runs reuse the prefill's cache), so the checks are:
  * logits of every decoded token vs the fp64 oracle resumed one token at a
    time from the same cache (max-abs 2e-2, same top-1);
  * every owning layer's K/V vs the oracle's (|d| <= 1e-2 + one fp16 ulp),
    the appended rows and the prefilled ones (the tiny model's prefill runs
    at exact precision: its fp16-operand path cannot hold layer 1 to the
    bound, see test_conditioning.py);
  * at the E2B-like shape, decode == ppx_prefill of the one token from the
    same snapshot;
  * errors leave n_pos unchanged.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import container, kv_within, logits_ok, oracle_model

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


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


@pytest.mark.parametrize("cfg,n0,steps", [("tiny", 40, 4), ("tinyllama", 100, 2)])
def test_decode_vs_oracle(ppx, cfg, n0, steps):
    toks = synth.prompt(cfg, n0 + steps)
    om = oracle_model(cfg)
    okv = oracle.KVState(om, n0 + steps)
    oracle.prefill(om, okv, toks[:n0], prune=True)
    mm = engine_model(ppx, cfg)
    kv = ppx.KVCache(mm, n0 + steps)
    mm.prefill(toks[:n0], kv, n_ubatch=512, precision="exact" if cfg == "tiny" else "fast")
    for k in range(steps):
        pos = n0 + k
        ref = oracle.prefill(om, okv, toks[pos:pos + 1], prune=True).astype(np.float64)
        got = mm.decode(int(toks[pos]), kv).cpu().numpy().astype(np.float64)
        torch.cuda.synchronize()
        assert kv.n_pos == pos + 1
        ok, d = logits_ok(got, ref)
        print(f"{cfg} decode at {pos}: logits max-abs {d:.3e}")
        assert ok, (pos, d)
        K, V = kv.kv_tensors()
        for g, want in ((K[:, :pos + 1], okv.K[:, :pos + 1]), (V[:, :pos + 1], okv.V[:, :pos + 1])):
            okk, dk = kv_within(g.cpu().numpy(), want)
            assert okk, (pos, dk)


def test_e2b_decode_equals_one_token_prefill(ppx, tmp_path):
    """At the E2B-like shape: decode(t) after a 512-token prefill gives the
    logits and cache rows of ppx_prefill([t]) from the same snapshot."""
    cfg, n = "e2b", 512
    toks = synth.prompt(cfg, n + 1)
    mm = engine_model(ppx, cfg)
    kv = ppx.KVCache(mm, n + 1)
    mm.prefill(toks[:n], kv, n_ubatch=512)
    snap = str(tmp_path / "p.kvc")
    kv.save(snap, n)
    la = mm.decode(int(toks[n]), kv).cpu().numpy()
    Ka, Va = (t[:, n].cpu().numpy() for t in kv.kv_tensors())
    kv2 = ppx.KVCache(mm, n + 1)
    kv2.load(snap, n)
    lb = mm.prefill(toks[n:n + 1], kv2, n_ubatch=512).cpu().numpy()
    Kb, Vb = (t[:, n].cpu().numpy() for t in kv2.kv_tensors())
    torch.cuda.synchronize()
    ok, d = logits_ok(la.astype(np.float64), lb.astype(np.float64))
    print(f"e2b decode vs one-token prefill: logits max-abs {d:.3e}")
    assert ok, d
    for g, w in ((Ka, Kb), (Va, Vb)):
        okk, dk = kv_within(g, w.astype(np.float64))
        assert okk, dk


def test_decode_errors_leave_cache(ppx):
    mm = engine_model(ppx, "tiny")
    kv = ppx.KVCache(mm, 8)
    mm.prefill(synth.prompt("tiny", 8), kv, n_ubatch=64)
    with pytest.raises(ppx.PPXError):
        mm.decode(5, kv)  # the cache is full
    assert kv.n_pos == 8
    kv2 = ppx.KVCache(mm, 16)
    mm.prefill(synth.prompt("tiny", 8), kv2, n_ubatch=64)
    with pytest.raises(ppx.PPXError):
        mm.decode(mm.info["n_vocab"], kv2)  # token out of range
    assert kv2.n_pos == 8
