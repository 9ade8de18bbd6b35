"""End-to-end parity of ppx_prefill against the fp64 oracle, and the pages'
invariants on the GPU:
  * last-row logits: max-abs <= 2e-2 and the same top-1 token;
  * KV cache entries: |d| <= 1e-2 + one fp16 ulp of the oracle value (the
    configs' keys reach |k| ~ 30-60 where one fp16 ulp exceeds 1e-2);
  * pruned == unpruned (llama.cpp Gemma 4 prefill page, section 3);
  * KV-shared layers leave the cache unchanged: the cache after a pruned and
    after an unpruned prefill are bit-identical (section 1);
  * resume from a saved snapshot == full prefill (PicoLM page, resume
    section), at N = 25 and N = 500 for the TinyLlama-shaped model;
  * ubatch size does not change the result.
"""
import dataclasses
import os

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import container, kv_within, logits_ok, oracle_kv_from_rows, oracle_model

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ppx():
    import prompt_prefill_cross_amd as p
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    p.lib()
    return p


_cache = {}


def run_oracle(cfg, n, prune=True):
    key = (cfg, n, prune)
    if key not in _cache:
        m = oracle_model(cfg)
        kv = oracle.KVState(m, n)
        lg = oracle.prefill(m, kv, synth.prompt(cfg, n), prune=prune)
        _cache[key] = (lg, kv)
    return _cache[key]


_models = {}


def engine_model(ppx, name):
    if name not in _models:
        _models.clear()
        torch.cuda.synchronize()
        _models[name] = ppx.Model(container(name))
    return _models[name]


def gpu_prefill(ppx, cfg, toks, n_ctx, ub, prune="auto", kv=None):
    mm = engine_model(ppx, cfg)
    if kv is None:
        kv = ppx.KVCache(mm, n_ctx)
    lg = mm.prefill(toks, kv, n_ubatch=ub, prune=prune)
    torch.cuda.synchronize()
    return lg.cpu().numpy(), kv


def check_kv(ppx, cfg, n, kv, rkv, rows, unconditional_layers):
    """KV parity.  Unconditional: the engine's cache vs the oracle's, for the
    listed owning layers.  Conditional, every owning layer: the oracle's K/V
    projection applied to the engine's own layer-input rows (debug_rows) must
    reproduce the engine's cache -- this isolates the engine's K/V arithmetic
    from upstream fp16 rounding amplified through earlier layers' attention."""
    om = oracle_model(cfg)
    K, V = kv.kv_tensors()
    K = K[:, :n].cpu().numpy()
    V = V[:, :n].cpu().numpy()
    for il in unconditional_layers:
        for got, want in ((K[il], rkv.K[il, :n]), (V[il], rkv.V[il, :n])):
            okk, dk = kv_within(got, want)
            assert okk, ("unconditional", il, dk)
    for il in range(om.n_layer_kv_from_start):
        kc, vc = oracle_kv_from_rows(om, il, rows[il], np.arange(n))
        for got, want in ((K[il], kc), (V[il], vc)):
            okk, dk = kv_within(got, want)
            assert okk, ("conditional", il, dk)


TINY_RUNS = [(64, "auto"), (16, "auto"), (64, "off"), (7, "off")]


@pytest.mark.parametrize("ub,prune", TINY_RUNS)
def test_tiny_vs_oracle_exact(ppx, ub, prune):
    """Exact precision: logits and every owning layer's K/V against the
    oracle's cache, unconditionally, to the KV bound."""
    n = 64
    ref, rkv = run_oracle("tiny", n)
    mm = engine_model(ppx, "tiny")
    kv = ppx.KVCache(mm, n)
    lg = mm.prefill(synth.prompt("tiny", n), kv, n_ubatch=ub, prune=prune, precision="exact").cpu().numpy()
    ok, d = logits_ok(lg, ref)
    assert ok, d
    K, V = kv.kv_tensors()
    for il in range(mm.info["n_layer_kv_from_start"]):
        for got, want in ((K[il, :n], rkv.K[il, :n]), (V[il, :n], rkv.V[il, :n])):
            okk, dk = kv_within(got.cpu().numpy(), want)
            print(f"exact ub={ub} prune={prune} layer {il}: KV max-abs {dk:.2e}")
            assert okk, (il, dk)


@pytest.mark.parametrize("ub,prune", TINY_RUNS)
def test_tiny_vs_oracle(ppx, ub, prune):
    """Fast precision: logits against the oracle; layer 0's K/V against the
    oracle's cache (they depend on the embedding only), every owning layer's
    K/V against the oracle's projection of the engine's own layer inputs."""
    n = 64
    ref, rkv = run_oracle("tiny", n)
    mm = engine_model(ppx, "tiny")
    rows = torch.zeros((mm.info["n_layer"], n, mm.info["d_model"]), dtype=torch.float32, device="cuda")
    kv = ppx.KVCache(mm, n)
    lg = mm.prefill(synth.prompt("tiny", n), kv, n_ubatch=ub, prune=prune, debug_rows=rows).cpu().numpy()
    ok, d = logits_ok(lg, ref)
    assert ok, d
    check_kv(ppx, "tiny", n, kv, rkv, rows.cpu().numpy().astype(np.float64), [0])


@pytest.mark.xfail(reason="fp16 MFMA operands cannot hold the tiny model's layer-1 K/V to 1e-2: its layer-1 "
                          "values reach |v| ~ 12 and layer 0 amplifies fp16 rounding of the query and the "
                          "attention output alone past the bound (tests/test_conditioning.py shows it on the "
                          "CPU); the exact precision holds every layer (test_tiny_vs_oracle_exact)",
                   strict=True)
def test_tiny_fast_every_layer_kv_unconditional(ppx):
    n = 64
    ref, rkv = run_oracle("tiny", n)
    mm = engine_model(ppx, "tiny")
    kv = ppx.KVCache(mm, n)
    mm.prefill(synth.prompt("tiny", n), kv, n_ubatch=64)
    K, V = kv.kv_tensors()
    for il in range(mm.info["n_layer_kv_from_start"]):
        for got, want in ((K[il, :n], rkv.K[il, :n]), (V[il, :n], rkv.V[il, :n])):
            okk, dk = kv_within(got.cpu().numpy(), want)
            assert okk, (il, dk)


def test_tiny_invariants(ppx):
    n = 64
    toks = synth.prompt("tiny", n)
    la, kva = gpu_prefill(ppx, "tiny", toks, n, 64, "on")
    lb, kvb = gpu_prefill(ppx, "tiny", toks, n, 64, "off")
    lc, kvc = gpu_prefill(ppx, "tiny", toks, n, 16, "on")
    assert logits_ok(la, lb)[0]
    # shared layers never write: the cache is the same bytes either way
    assert torch.equal(kva.buf, kvb.buf) and torch.equal(kva.buf, kvc.buf)
    # ubatch-independent and deterministic
    assert np.array_equal(la, lc)
    ld, _ = gpu_prefill(ppx, "tiny", toks, n, 64, "on")
    assert np.array_equal(la, ld)


def test_recorded_launches_replay_with_new_tokens(ppx):
    """A prefill of a shape seen before replays its recorded launch sequence;
    the replay must read the new prompt's tokens (embedding, per-layer
    embedding of every row, and the pruned tail's row) and give exactly the
    result of the direct launches (the timing mode never records)."""
    mm = engine_model(ppx, "e2b")
    n, ub = 96, 64
    logits = torch.empty(mm.info["n_vocab"], dtype=torch.float32, device="cuda")
    kv = ppx.KVCache(mm, n)
    rng = np.random.default_rng(77)
    prompts = [rng.integers(0, mm.info["n_vocab"], n).astype(np.int32) for _ in range(3)]
    replayed = []
    for toks in prompts:  # the first call records, the others replay
        kv.clear()
        replayed.append(mm.prefill(toks, kv, n_ubatch=ub, logits=logits).clone())
    torch.cuda.synchronize()
    for toks, got in zip(prompts, replayed):
        kv.clear()
        direct = mm.prefill(toks, kv, n_ubatch=ub, timing=ppx.Timing())
        torch.cuda.synchronize()
        assert torch.equal(got, direct)
    assert not torch.equal(replayed[1], replayed[2])


@pytest.mark.parametrize("cfg,n,ub,prune", [("e2b", 2048, 512, "auto"), ("e2b", 1000, 128, "off"),
                                          ("tinyllama", 512, 64, "auto")])
def test_pipelined_ubatches_equal_the_serial_order(ppx, cfg, n, ub, prune):
    """Ubatches run through the row-batched layers together (one launch per
    operation over the ubatches in flight); asking for the last row's hidden
    states runs them one at a time instead, the serial order.  The long-K
    down projection splits K over workgroups only when few ubatches share
    the launch, so the two orders differ only in the order of fp32 sums:
    logits within 1e-3 with the same top-1, the cache within the KV bound."""
    mm = engine_model(ppx, cfg)
    toks = synth.prompt(cfg, n)
    kva = ppx.KVCache(mm, n)
    la = mm.prefill(toks, kva, n_ubatch=ub, prune=prune).clone()
    kvb = ppx.KVCache(mm, n)
    hid = torch.empty((mm.info["n_layer"], mm.info["d_model"]), dtype=torch.float32, device="cuda")
    lb = mm.prefill(toks, kvb, n_ubatch=ub, prune=prune, debug_hidden=hid)
    torch.cuda.synchronize()
    ok, d = logits_ok(la.cpu().numpy(), lb.cpu().numpy(), atol=1e-3)
    print(f"{cfg} n={n} ub={ub} prune={prune}: grouped vs serial logits max-abs {d:.2e}")
    assert ok, d
    Ka, Va = kva.kv_tensors()
    Kb, Vb = kvb.kv_tensors()
    for got, want in ((Ka[:, :n], Kb[:, :n]), (Va[:, :n], Vb[:, :n])):
        okk, dk = kv_within(got.cpu().numpy(), want.cpu().numpy())
        assert okk, dk


def test_replay_after_the_rope_table_grows(ppx):
    """A recorded launch sequence holds the RoPE table's address.  Creating a
    cache with a longer context replaces the table; a later prefill of a shape
    recorded before must not replay against the freed one.  Order: record on
    cache A, create the longer cache B, prefill A again with the same shape
    (and a new prompt), check against the oracle and the direct launches."""
    mm = ppx.Model(container("tiny"))  # a fresh model: its table covers only what this test creates
    n = 48
    kva = ppx.KVCache(mm, 64)
    t1 = synth.prompt("tiny", n)
    first = mm.prefill(t1, kva, n_ubatch=16).clone()
    kvb = ppx.KVCache(mm, 4096)  # grows the table
    scratch = torch.full((1 << 22,), float("nan"), device="cuda")  # reuses freed memory, if any
    rng = np.random.default_rng(48)
    t2 = rng.integers(0, mm.info["n_vocab"], n).astype(np.int32)
    kva.clear()
    again = mm.prefill(t2, kva, n_ubatch=16).clone()
    kva.clear()
    direct = mm.prefill(t2, kva, n_ubatch=16, timing=ppx.Timing())
    torch.cuda.synchronize()
    assert torch.equal(again, direct)
    om = oracle_model("tiny")
    ref = oracle.prefill(om, oracle.KVState(om, 64), t2, prune=True)
    ok, d = logits_ok(again.cpu().numpy(), ref)
    assert ok, d
    ok, d = logits_ok(first.cpu().numpy(), oracle.prefill(om, oracle.KVState(om, 64), t1, prune=True))
    assert ok, d
    del scratch, kvb
    kva.close()
    mm.close()


def test_tiny_error_paths(ppx):
    mm = engine_model(ppx, "tiny")
    kv = ppx.KVCache(mm, 32)
    with pytest.raises(ppx.PPXError) as e:
        mm.prefill([], kv)
    assert e.value.status == -10
    with pytest.raises(ppx.PPXError) as e:
        mm.prefill([0, 2048], kv)
    assert e.value.status == -2
    with pytest.raises(ppx.PPXError) as e:
        mm.prefill(np.zeros(33, np.int32), kv)
    assert e.value.status == -3
    with pytest.raises(ppx.PPXError) as e:
        mm.prefill([1, 2], kv, embeddings=1)  # no output buffer for the embeddings
    assert e.value.status == -1
    with pytest.raises(ppx.PPXError) as e:
        mm.prefill([1, 2], kv, embeddings=1, prune="on",
                   embd_out=torch.empty((2, mm.info["d_model"]), device="cuda"))  # predicate false
    assert e.value.status == -7
    with pytest.raises(ppx.PPXError) as e:
        mm.prefill([1, 2], kv, n_seq_max=2)
    assert e.value.status == -7
    assert kv.n_pos == 0
    mm.prefill([1, 2, 3], kv)
    assert kv.n_pos == 3


# (config, prompt length, ubatch, precision); in the second and the last case
# the two rows the next-n head reads sit in different ubatches
NEXTN_RUNS = [("tiny", 64, 64, "exact"), ("tiny", 33, 16, "exact"), ("tiny", 64, 16, "fast"),
              ("e2b", 129, 64, "fast")]


@pytest.mark.parametrize("cfg,n,ub,precision", NEXTN_RUNS)
def test_nextn_head_vs_oracle(ppx, cfg, n, ub, precision):
    """A next-n head reads the second-to-last row, which makes the
    predicate's crop_before_nextn false: prune auto runs every row through
    every layer, and the head's logits and the last row's both match the
    oracle -- on the recorded launch sequence and on the one-ubatch-at-a-time
    debug path."""
    om = oracle_model(cfg)
    toks = synth.prompt(cfg, n)
    want = []
    ref = oracle.prefill(om, oracle.KVState(om, n), toks, nextn=want)
    mm = engine_model(ppx, cfg)
    assert mm.info["has_nextn"] == 1
    L, d, Ls = mm.info["n_layer"], mm.info["d_model"], mm.info["n_layer_kv_from_start"]
    rows = torch.full((L, n, d), float("nan"), dtype=torch.float32, device="cuda")
    for debug in (False, True, False):
        kv = ppx.KVCache(mm, n)
        nx = torch.empty(mm.info["n_vocab"], dtype=torch.float32, device="cuda")
        lg = mm.prefill(toks, kv, n_ubatch=ub, precision=precision, nextn_logits=nx,
                        debug_rows=rows if debug else None)
        torch.cuda.synchronize()
        for what, got, r in (("last row", lg, ref), ("next-n", nx, want[0])):
            ok, dd = logits_ok(got.cpu().numpy(), r)
            print(f"{cfg} n={n} ub={ub} {precision} debug={debug} {what}: max-abs {dd:.2e}")
            assert ok, (what, dd)
    # every KV-shared layer saw every row: the prune was off
    assert bool(torch.isfinite(rows[Ls:]).all())


def test_nextn_head_error_paths(ppx):
    mm = engine_model(ppx, "tiny")
    kv = ppx.KVCache(mm, 32)
    nx = torch.empty(mm.info["n_vocab"], dtype=torch.float32, device="cuda")
    with pytest.raises(ppx.PPXError) as e:
        mm.prefill([1, 2, 3], kv, prune="on", nextn_logits=nx)  # the predicate is false
    assert e.value.status == -7
    with pytest.raises(ppx.PPXError) as e:
        mm.prefill([1], kv, nextn_logits=nx)  # no second-to-last row
    assert e.value.status == -1
    plain = ppx.Model(synth.build_model(dataclasses.replace(synth.CONFIGS["tiny"], nextn=False)))
    assert plain.info["has_nextn"] == 0
    kp = ppx.KVCache(plain, 32)
    with pytest.raises(ppx.PPXError) as e:
        plain.prefill([1, 2, 3], kp, nextn_logits=nx)
    assert e.value.status == -7
    assert kv.n_pos == 0 and kp.n_pos == 0
    torch.cuda.synchronize()


def test_tinyllama_full_and_resume(ppx, tmp_path):
    cfg, n = "tinyllama", 512
    toks = synth.prompt(cfg, n)
    ref, rkv = run_oracle(cfg, n, prune=False)
    mm = engine_model(ppx, cfg)
    rows = torch.zeros((mm.info["n_layer"], n, mm.info["d_model"]), dtype=torch.float32, device="cuda")
    kv = ppx.KVCache(mm, n)
    lg = mm.prefill(toks, kv, n_ubatch=512, debug_rows=rows).cpu().numpy()
    ok, d = logits_ok(lg, ref)
    assert ok, d
    check_kv(ppx, cfg, n, kv, rkv, rows.cpu().numpy().astype(np.float64), range(22))
    del rows
    path = tmp_path / "prompt.kvc"
    kv.save(str(path), n)
    assert os.path.getsize(path) == 16 + 2 * 22 * n * 256 * 2
    # the PicoLM page's order: magic, positions (512 = 0x200), layers (22),
    # KV dim (256 = 0x100), typed out byte by byte; then K, then V, each
    # [layer][position][dim] fp16 (offsets computed by hand)
    raw = path.read_bytes()
    assert raw[:16] == bytes([0x4B, 0x56, 0x43, 0x50, 0, 2, 0, 0, 22, 0, 0, 0, 0, 1, 0, 0])
    K1, V1 = kv.kv_tensors()
    for il, p_, c in ((0, 0, 0), (5, 17, 3), (21, 511, 255)):
        ko = 16 + 2 * ((il * n + p_) * 256 + c)
        vo = 16 + 2 * 22 * n * 256 + 2 * ((il * n + p_) * 256 + c)
        assert np.frombuffer(raw[ko:ko + 2], "<f2")[0] == K1[il, p_, c].item()
        assert np.frombuffer(raw[vo:vo + 2], "<f2")[0] == V1[il, p_, c].item()
    mm = engine_model(ppx, cfg)
    for N in (25, 500):
        kv2 = ppx.KVCache(mm, n)
        kv2.load(str(path), N)
        assert kv2.n_pos == N
        lr, _ = gpu_prefill(ppx, cfg, toks[N:], n, 512, kv=kv2)
        assert kv2.n_pos == n
        ok, d = logits_ok(lr, ref)
        assert ok, (N, d)
        ok, d = logits_ok(lr, lg, atol=1e-3)
        assert ok, (N, d)
        # The loaded prefix is the snapshot, bit for bit; positions computed
        # after the resume match the uninterrupted run to rounding (the
        # attention's key split follows the ubatch shape) and the oracle
        # to the KV bound.
        K1, V1 = kv.kv_tensors()
        K2, V2 = kv2.kv_tensors()
        assert torch.equal(K2[:, :N], K1[:, :N]) and torch.equal(V2[:, :N], V1[:, :N])
        for got, want in ((K2, rkv.K), (V2, rkv.V)):
            okk, dk = kv_within(got[:, :n].cpu().numpy(), want[:, :n])
            assert okk, (N, dk)


GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# (golden file, ubatch, prune): the configs' full shapes against stored oracle results
GOLDEN_RUNS = [
    ("e2b_512", 512, "auto"), ("e2b_512", 512, "off"), ("e2b_512", 128, "auto"),
    ("e2b_2048", 512, "auto"), ("e2b_2048", 512, "off"),
    ("e4b_512", 512, "auto"), ("e4b_512", 512, "off"),
    ("e2b_8192", 512, "auto"), ("e4b_2048", 512, "auto"),
    ("e2b_ctrl_8192", 1024, "auto"), ("e2b_long_16384", 1024, "auto"),
    ("e4b_8192", 512, "auto"), ("e2b_long_32768", 1024, "auto"),
    # unpruned at the larger sizes: the stored results serve both modes, since
    # the oracle's pruned and unpruned passes are bit-identical
    ("e2b_8192", 512, "off"), ("e4b_2048", 512, "off"), ("e4b_8192", 512, "off"),
    ("e2b_long_16384", 1024, "off"),
]


def load_golden(name):
    import json
    path = os.path.join(GOLD, f"oracle_{name}.npz")
    if not os.path.exists(path):
        pytest.skip(f"no stored oracle result {path} (tests/golden/make_goldens.py writes it)")
    g = np.load(path)
    return g, json.loads(str(g["meta"]))


@pytest.mark.parametrize("name,ub,prune", GOLDEN_RUNS, ids=[f"{a}-ub{b}-{c}" for a, b, c in GOLDEN_RUNS])
def test_full_size_vs_stored_oracle(ppx, name, ub, prune):
    check_golden(ppx, name, ub, prune, "fast")


EXACT_GOLDEN_RUNS = [("e2b_512", 512, "auto"), ("e4b_512", 512, "off"), ("e2b_2048", 512, "auto")]


@pytest.mark.parametrize("name,ub,prune", EXACT_GOLDEN_RUNS, ids=[f"{a}-ub{b}-{c}" for a, b, c in EXACT_GOLDEN_RUNS])
def test_full_size_exact_vs_stored_oracle(ppx, name, ub, prune):
    check_golden(ppx, name, ub, prune, "exact")


def check_golden(ppx, name, ub, prune, precision):
    g, meta = load_golden(name)
    cfg, n = meta["config"], meta["n"]
    mm = engine_model(ppx, cfg)
    kv = ppx.KVCache(mm, n)
    lg = mm.prefill(synth.prompt(cfg, n), kv, n_ubatch=ub, prune=prune, precision=precision).cpu().numpy()
    ok, d = logits_ok(lg, g["logits"])
    print(f"{name} ub={ub} prune={prune} {precision}: logits max-abs {d:.3e}")
    assert ok, d
    K, V = kv.kv_tensors()
    layers = torch.from_numpy(g["kv_layers"]).cuda()
    pos = torch.from_numpy(g["kv_pos"]).cuda()
    for got, want in ((K, g["K"]), (V, g["V"])):
        sel = got[layers][:, pos].cpu().numpy()
        okk, dk = kv_within(sel, want)
        assert okk, dk


def test_e2b_prune_invariants_full_size(ppx):
    """KV-shared layers write nothing: pruned and unpruned prefills leave
    bit-identical caches; their logits agree within the logit tolerance."""
    cfg, n = "e2b", 1024
    toks = synth.prompt(cfg, n)
    la, kva = gpu_prefill(ppx, cfg, toks, n, 512, "on")
    buf_a = kva.buf.clone()
    del kva
    lb, kvb = gpu_prefill(ppx, cfg, toks, n, 512, "off")
    assert torch.equal(buf_a, kvb.buf)
    ok, d = logits_ok(la, lb)
    assert ok, d


def test_snapshot_rejections_leave_cache_empty(ppx, tmp_path):
    mm = engine_model(ppx, "tiny")
    kv = ppx.KVCache(mm, 64)
    mm.prefill(synth.prompt("tiny", 10), kv)
    good = tmp_path / "g.kvc"
    kv.save(str(good), 10)
    bad = tmp_path / "b.kvc"
    bad.write_bytes(b"XXXX" + good.read_bytes()[4:])
    for path, n, want in ((bad, 5, -5), (good, 11, -5), (tmp_path / "none.kvc", 1, -4)):
        kv2 = ppx.KVCache(mm, 64)
        with pytest.raises(ppx.PPXError) as e:
            kv2.load(str(path), n)
        assert e.value.status == want
        assert kv2.n_pos == 0


def test_torch_owned_weights(ppx):
    """ppx_model_load_into: the repacked weights in a torch tensor give the
    same bits as the library's own allocation; the tensor outlives the model
    and is not freed with it; a short or misaligned buffer is refused."""
    import ctypes
    buf = container("tiny")
    toks = synth.prompt("tiny", 40)
    ma = ppx.Model(buf)
    mb = ppx.Model(buf, torch_weights=True)
    need = ppx.lib().ppx_model_weight_bytes(ctypes.c_void_p(buf.ctypes.data), buf.nbytes)
    assert mb._weights.numel() == need == mb.device_bytes == ma.device_bytes
    la = ma.prefill(toks, ppx.KVCache(ma, 64), n_ubatch=16).clone()
    kvb = ppx.KVCache(mb, 64)
    lb = mb.prefill(toks, kvb, n_ubatch=16)
    torch.cuda.synchronize()
    assert torch.equal(la, lb)
    w = mb._weights
    kvb.close()
    mb.close()
    w.zero_()  # still the caller's memory
    torch.cuda.synchronize()
    L = ppx.lib()
    h = ctypes.c_void_p()
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    st = L.ppx_model_load_into(ctypes.c_void_p(buf.ctypes.data), buf.nbytes, ctypes.c_void_p(small.data_ptr()),
                               small.numel(), None, ctypes.byref(h))
    assert st == -9 and not h.value
    big = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    st = L.ppx_model_load_into(ctypes.c_void_p(buf.ctypes.data), buf.nbytes, ctypes.c_void_p(big.data_ptr() + 1),
                               need, None, ctypes.byref(h))
    assert st == -1 and not h.value

