"""Several prompts over one unified KV cache (ppx_prefill_unified).

One buffer holds every sequence; cells go out in pages of 64 positions of one
sequence, and a row attends only to the cells of its own sequence (the
llama.cpp Gemma 4 prefill page, section 5, sets such a unified cache against
one cache per sequence).  Checks:
  * per-sequence logits vs the oracle's unified pass (one buffer, attention
    masked by each cell's sequence): max-abs 2e-2, same top-1; each
    sequence's (position -> K/V) of every owning layer vs the oracle's
    (|d| <= 1e-2 + one fp16 ulp), the tiny model at exact precision;
  * sequences grown over several calls hold scattered pages, and a removed
    sequence's pages are reused: call by call against the oracle;
  * the E2B-like model: unified equals split caches bit for bit (the same
    kernels read the same values at other addresses), both against the
    oracle, a one-token step per sequence included, and a recorded launch
    sequence replays onto another cache;
  * argument errors change no sequence and no page.
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


def check_seq(cache, u, sid, what):
    """Sequence sid's K/V, in position order, against the oracle's cells."""
    K, V = cache.seq_kv(sid)
    cells = u.cells_of(sid)
    assert K.shape[1] == cells.shape[0] == cache.n_pos(sid)
    for got, want in ((K, u.K[:, cells]), (V, u.V[:, cells])):
        okk, dk = kv_within(got.cpu().numpy(), want)
        assert okk, (what, sid, dk)


@pytest.mark.parametrize("ub,prune", [(16, "auto"), (7, "off"), (64, "auto")])
def test_tiny_unified_vs_oracle(ppx, ub, prune):
    n_cells = 320
    ids = [4, 0, 2, 9]
    lens = (13, 1, 30, 7)
    base = synth.prompt("tiny", sum(lens) + 8)
    offs = np.cumsum((0,) + lens)
    prompts = [base[offs[i]:offs[i + 1]] for i in range(len(lens))]
    om = oracle_model("tiny")
    u = oracle.UnifiedKV(om, n_cells)
    ref = oracle.prefill_unified(om, u, ids, prompts, prune=prune != "off", n_ubatch=ub)
    mm = engine_model(ppx, "tiny")
    cache = ppx.UnifiedCache(mm, n_cells, 16)
    lg = mm.prefill_unified(prompts, ids, cache, n_ubatch=ub, prune=prune, precision="exact").cpu().numpy()
    torch.cuda.synchronize()
    for i, sid in enumerate(ids):
        ok, d = logits_ok(lg[i], ref[i])
        print(f"tiny unified ub={ub} prune={prune} seq {sid}: logits max-abs {d:.3e}")
        assert ok, (sid, d)
        assert cache.n_pos(sid) == lens[i]
        check_seq(cache, u, sid, "tiny")
    assert cache.free_cells() == n_cells - 64 * len(ids)


def test_tiny_unified_interleaved_calls_and_page_reuse(ppx):
    """Sequence 0 grows over two calls past two page boundaries while
    sequence 1 takes the pages between, so its pages are scattered; removing
    sequence 1 frees its pages, which a new sequence then takes."""
    n_cells = 320
    toks = synth.prompt("tiny", 340)
    a, b, c = toks[:150], toks[150:250], toks[250:330]
    om = oracle_model("tiny")
    u = oracle.UnifiedKV(om, n_cells)
    mm = engine_model(ppx, "tiny")
    cache = ppx.UnifiedCache(mm, n_cells, 8)
    steps = [([0, 1], [a[:70], b[:40]], "auto"), ([1, 0], [b[40:], a[70:]], "off")]
    for n_step, (ids, ps, prune) in enumerate(steps):
        ref = oracle.prefill_unified(om, u, ids, ps, prune=prune != "off", n_ubatch=32)
        lg = mm.prefill_unified(ps, ids, cache, n_ubatch=32, prune=prune, precision="exact").cpu().numpy()
        torch.cuda.synchronize()
        for i, sid in enumerate(ids):
            ok, d = logits_ok(lg[i], ref[i])
            print(f"tiny unified step {n_step} seq {sid}: logits max-abs {d:.3e}")
            assert ok, (n_step, sid, d)
    pages0 = sorted(set((cache.cells(0) // 64).tolist()))
    pages1 = sorted(set((cache.cells(1) // 64).tolist()))
    assert pages0 == [0, 1, 4] and pages1 == [2, 3], (pages0, pages1)
    for sid in (0, 1):
        check_seq(cache, u, sid, "grown")
    cache.seq_rm(1)
    u.seq_rm(1)
    assert cache.n_pos(1) == 0 and cache.free_cells() == n_cells - 3 * 64
    ids, ps = [5, 0], [c, b[:3]]
    ref = oracle.prefill_unified(om, u, ids, ps, prune=True, n_ubatch=32)
    lg = mm.prefill_unified(ps, ids, cache, n_ubatch=32, precision="exact").cpu().numpy()
    torch.cuda.synchronize()
    for i, sid in enumerate(ids):
        ok, d = logits_ok(lg[i], ref[i])
        print(f"tiny unified after reuse seq {sid}: logits max-abs {d:.3e}")
        assert ok, (sid, d)
        check_seq(cache, u, sid, "reused")
    assert sorted(set((cache.cells(5) // 64).tolist())) == [2, 3]


def test_e2b_unified_equals_split_and_oracle(ppx):
    """Four prompts (one of a single token) in one call, then one token per
    sequence: unified and split caches give the same bits, and both match
    the oracle; the same call shape recorded once replays onto a second
    unified cache."""
    cfg = "e2b"
    lens = (300, 77, 129, 1)
    ids = [3, 0, 7, 1]
    base = synth.prompt(cfg, sum(lens) + 16)
    offs = np.cumsum((0,) + lens)
    prompts = [base[offs[i]:offs[i + 1]] for i in range(len(lens))]
    steps = [[int(base[sum(lens) + i])] for i in range(len(lens))]
    om = oracle_model(cfg)
    okvs = [oracle.KVState(om, 512) for _ in lens]
    ref = oracle.prefill_multi(om, okvs, prompts, prune=True)
    ref2 = oracle.prefill_multi(om, okvs, steps, prune=True)
    mm = engine_model(ppx, cfg)
    kvs = [ppx.KVCache(mm, 512) for _ in lens]
    ls = mm.prefill_multi(prompts, kvs, n_ubatch=128).cpu().numpy()
    ls2 = mm.prefill_multi(steps, kvs, n_ubatch=128).cpu().numpy()
    outs = []
    for rep in range(2):
        cache = ppx.UnifiedCache(mm, 1024, 8)
        lu = mm.prefill_unified(prompts, ids, cache, n_ubatch=128).cpu().numpy()
        lu2 = mm.prefill_unified(steps, ids, cache, n_ubatch=128).cpu().numpy()
        torch.cuda.synchronize()
        outs.append((lu, lu2, cache))
    lu, lu2, cache = outs[0]
    assert np.array_equal(outs[1][0], lu) and np.array_equal(outs[1][1], lu2)
    assert np.array_equal(lu, ls) and np.array_equal(lu2, ls2)
    for i, sid in enumerate(ids):
        for got, want, what in ((lu[i], ref[i], "prompt"), (lu2[i], ref2[i], "step")):
            ok, d = logits_ok(got, want)
            print(f"e2b unified seq {sid} {what}: logits max-abs {d:.3e}")
            assert ok, (sid, what, d)
        n = lens[i] + 1
        K, V = cache.seq_kv(sid)
        Ks, Vs = kvs[i].kv_tensors()
        assert torch.equal(K, Ks[:, :n]) and torch.equal(V, Vs[:, :n])
        for got, want in ((K, okvs[i].K[:, :n]), (V, okvs[i].V[:, :n])):
            okk, dk = kv_within(got.cpu().numpy(), want)
            assert okk, (sid, dk)
        K2, V2 = outs[1][2].seq_kv(sid)
        assert torch.equal(K, K2) and torch.equal(V, V2)


def test_unified_errors_change_nothing(ppx):
    mm = engine_model(ppx, "tiny")
    cache = ppx.UnifiedCache(mm, 128, 4)
    mm.prefill_unified([synth.prompt("tiny", 100)], [0], cache, n_ubatch=64)
    torch.cuda.synchronize()
    before = (cache.n_pos(0), cache.free_cells(), cache.cells(0).copy())
    cases = [
        (([[1, 2], [3]], [1, 1]), -1),      # one sequence twice
        (([[1, 2]], [4]), -1),              # sequence id out of range
        (([[1, 2]], [-1]), -1),
        (([[1, 2]], [1]), -3),              # no free page left
        (([[1] * 29], [0]), -3),            # past n_cells positions
        (([[]], [2]), -10),                 # empty prompt
        (([[5000]], [2]), -2),              # token out of range
    ]
    for (ps, ids), status in cases:
        with pytest.raises(ppx.PPXError) as e:
            mm.prefill_unified(ps, ids, cache, n_ubatch=64)
        assert e.value.status == status, (ps, ids, e.value.status)
    with pytest.raises(ppx.PPXError) as e:
        mm.prefill_unified([[1, 2]], [1], cache, n_ubatch=64, prune="on", n_seq_max=0)
    assert e.value.status == -1
    assert (cache.n_pos(0), cache.free_cells()) == before[:2] and np.array_equal(cache.cells(0), before[2])
    assert cache.n_pos(1) == 0
    # the remaining 28 cells of sequence 0's second page still take its tokens
    mm.prefill_unified([[1] * 28], [0], cache, n_ubatch=64)
    torch.cuda.synchronize()
    assert cache.n_pos(0) == 128 and cache.free_cells() == 0
    with pytest.raises(ValueError):
        ppx.UnifiedCache(mm, 100, 4)
