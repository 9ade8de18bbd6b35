"""Extraction through ppx_prefill: every row's input to flagged layers
(embeddings_layer_inp, index n_layer = the final hidden state) and every
row's output-normed final state (embeddings), with the prune predicate of
the llama.cpp Gemma 4 prefill page (section 1) evaluated on those flags.

Checks:
  * vs the fp64 oracle's extraction: layer 0's input (the embedding gather)
    to fp32 rounding; later rows within max-abs 2e-2 of the reference rows'
    scale (rms), the bound the logits are held to, since the logits are the
    head matrix times the last normed row;
  * consistency: the extracted inputs are the engine's own layer inputs
    (debug_rows) bit for bit, and the head of the last extracted embedding
    reproduces the logits;
  * the predicate: flags below the first KV-shared layer keep the prune (the
    logits equal a plain pruned prefill bit for bit); a flag at or above it,
    or the embeddings, turn it off (the logits equal a plain unpruned prefill
    bit for bit); prune ON then fails.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import container, logits_ok, oracle_model

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


def rows_ok(got, ref, rel=2e-2):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = max(float(np.sqrt(np.mean(ref * ref))), 1e-30)
    d = float(np.abs(got - ref).max()) / scale
    return d <= rel, d


@pytest.mark.parametrize("cfg,n,ub", [("tiny", 64, 16), ("e2b", 40, 512)])
def test_extraction_vs_oracle(ppx, cfg, n, ub):
    om = oracle_model(cfg)
    L, ls = om.n_layer, om.n_layer_kv_from_start
    layers = sorted({0, 1, ls - 1, ls, L - 1, L})
    toks = synth.prompt(cfg, n)
    inp = {il: None for il in layers}
    emb = []
    ref = oracle.prefill(om, oracle.KVState(om, n), toks, prune=False, layer_inp=inp, embeddings=emb)
    mm = engine_model(ppx, cfg)
    kv = ppx.KVCache(mm, n)
    lg, got, ge = mm.extract(toks, kv, layers=layers, embeddings=True, n_ubatch=ub)
    torch.cuda.synchronize()
    ok, d = logits_ok(lg.cpu().numpy(), ref)
    assert ok, d
    g0 = got[0].cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(g0, inp[0], rtol=2 ** -23, atol=1e-30)
    for il in layers[1:]:
        ok, d = rows_ok(got[il].cpu().numpy(), inp[il])
        print(f"{cfg}: input of layer {il}: max-abs / rms {d:.3e}")
        assert ok, (il, d)
    ok, d = rows_ok(ge.cpu().numpy(), emb[0])
    print(f"{cfg}: embeddings: max-abs / rms {d:.3e}")
    assert ok, d
    # the head of the last embedding is the logits
    name, V = ("tok_embd" if om.tied else "output"), om.n_vocab
    e_last = ge[-1].cpu().numpy().astype(np.float64)
    head = np.concatenate([om.q4(name, rows=np.arange(s, min(V, s + 16384))) @ e_last
                           for s in range(0, V, 16384)])
    ok, d = logits_ok(lg.cpu().numpy(), head, atol=1e-3)
    assert ok, d


def test_extraction_is_the_layer_input_and_keeps_the_prune(ppx):
    cfg, n, ub = "tiny", 48, 16
    om = oracle_model(cfg)
    L, ls, d = om.n_layer, om.n_layer_kv_from_start, om.d_model
    toks = synth.prompt(cfg, n)
    mm = engine_model(ppx, cfg)
    # flags below the first shared layer: the prune stays on
    kva = ppx.KVCache(mm, n)
    la, got, _ = mm.extract(toks, kva, layers=range(ls), n_ubatch=ub)
    kvb = ppx.KVCache(mm, n)
    rows = torch.zeros((L, n, d), dtype=torch.float32, device="cuda")
    lb = mm.prefill(toks, kvb, n_ubatch=ub, prune="on", debug_rows=rows)
    torch.cuda.synchronize()
    assert torch.equal(la, lb)
    for il in range(ls):
        assert torch.equal(got[il], rows[il])
    # a flag at the first shared layer, or the embeddings: every row runs every layer
    kvc = ppx.KVCache(mm, n)
    lc = mm.prefill(toks, kvc, n_ubatch=ub, prune="off", debug_rows=rows)
    for kw in ({"layers": [ls]}, {"layers": [L]}, {"embeddings": True}):
        kvd = ppx.KVCache(mm, n)
        ld, got, emb = mm.extract(toks, kvd, n_ubatch=ub, **kw)
        torch.cuda.synchronize()
        assert torch.equal(ld, lc), kw
        if "layers" in kw and kw["layers"][0] < L:
            assert torch.equal(got[kw["layers"][0]], rows[kw["layers"][0]])
        with pytest.raises(ppx.PPXError) as e:
            mm.extract(toks, ppx.KVCache(mm, n), n_ubatch=ub, prune="on", **kw)
        assert e.value.status == -7
