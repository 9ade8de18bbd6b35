"""Pins of the fp64 oracle against things other than itself.

Closed forms, library special cases, hand-built fixtures under
tests/golden/ (each with its citation), a scalar brute-force implementation
(tests/brute.py) on micro shapes, and the invariants the pages fix:
pruned == unpruned (llama.cpp Gemma 4 prefill page, section 3: identical
outputs), KV-shared layers leave the cache untouched (section 1), and
resuming after N cached positions equals a full prefill (PicoLM page,
resume section).  Several prompts in one pass are pinned to the same brute
force run on each prompt alone.
"""
import dataclasses
import json
import math
import os
import struct

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import forward as F
from tests import brute

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


MICRO = synth.Config("micro", 90, n_layer=4, n_layer_kv_from_start=2, d_model=32, n_head=2,
                     n_kv_head=1, head_dim=16, n_ff=64, n_vocab=40, ple_dim=32, act="geglu",
                     tied=True, n_ubatch=2, seed=9090)
MICRO_SW = synth.Config("micro_sw", 91, n_layer=3, n_layer_kv_from_start=3, d_model=32, n_head=4,
                        n_kv_head=2, head_dim=8, n_ff=64, n_vocab=48, ple_dim=0, act="swiglu",
                        tied=False, n_ubatch=3, seed=9191)


# ------------------------------------------------------------------ Q4_0

def test_deq_hand_built_blocks():
    g = _gold("q4_0_blocks.json")
    for blk in g["blocks"]:
        raw = np.array(blk["bytes"], dtype=np.uint8).reshape(1, 18)
        got = oracle.deq_q4_0(raw)[0]
        assert got.tolist() == blk["values"], blk["what"]


def test_deq_exhaustive_codes_and_scale_sweep():
    # every code in both nibble positions, against scales decoded by struct
    rng = np.random.default_rng(5)
    bits = np.concatenate([np.arange(0, 0x7C00, 97), rng.integers(0x8000, 0xFC00, 200)]).astype(np.uint16)
    for b in bits:
        for c in range(16):
            raw = np.zeros((1, 18), np.uint8)
            raw[0, 0:2] = np.frombuffer(struct.pack("<H", int(b)), np.uint8)
            raw[0, 2:] = c | ((15 - c) << 4)
            (d,) = struct.unpack("<e", struct.pack("<H", int(b)))
            got = oracle.deq_q4_0(raw)[0]
            assert got[0] == d * (c - 8) and got[16] == d * (7 - c)


def test_fp16_store_is_round_to_nearest_even():
    # ties between fp16 neighbours of 1.0 (spacing 2^-10) round to the even one
    one = 1.0
    cases = {one + 2 ** -11: 1.0, one + 3 * 2 ** -11: 1.0 + 2 ** -9,
             one + 2 ** -11 + 2 ** -30: 1.0 + 2 ** -10, -(one + 2 ** -11): -1.0,
             65519.0: 65504.0, 2 ** -25: 0.0, 3 * 2 ** -26: 2 ** -24}
    for v, want in cases.items():
        assert float(np.float64(v).astype(np.float16)) == want, v


# ------------------------------------------------------------------ elementwise

def test_rms_norm_closed_form():
    x = np.array([[3.0, 4.0]])
    g = np.array([1.0, 2.0])
    got = F.rms_norm(x, g, 0.0)
    np.testing.assert_allclose(got, [[3 / math.sqrt(12.5), 8 / math.sqrt(12.5)]], rtol=1e-15)
    # scale invariance and unit mean square when eps = 0 and g = 1
    z = np.random.default_rng(1).standard_normal((5, 64))
    np.testing.assert_allclose(F.rms_norm(7.5 * z, np.ones(64), 0.0), F.rms_norm(z, np.ones(64), 0.0),
                               rtol=1e-13)
    np.testing.assert_allclose((F.rms_norm(z, np.ones(64), 0.0) ** 2).mean(axis=1), 1.0, rtol=1e-13)
    # eps enters under the root: a zero row stays zero, a constant row c gives c/sqrt(c^2+eps)
    np.testing.assert_allclose(F.rms_norm(np.full((1, 4), 1e-3), np.ones(4), 1e-6),
                               1e-3 / math.sqrt(1e-6 + 1e-6), rtol=1e-13)


def test_gelu_tanh_against_library_and_identities():
    z = np.linspace(-8, 8, 4001)
    ref = torch.nn.functional.gelu(torch.from_numpy(z), approximate="tanh").numpy()
    np.testing.assert_allclose(F.gelu_tanh(z), ref, rtol=1e-13, atol=1e-15)
    # odd-part identity of x*Phi-like gates: g(z) - g(-z) = z
    np.testing.assert_allclose(F.gelu_tanh(z) - F.gelu_tanh(-z), z, atol=1e-12)
    # close to the erf form (within the approximation's known few-1e-4 error)
    erf = torch.nn.functional.gelu(torch.from_numpy(z)).numpy()
    assert np.abs(F.gelu_tanh(z) - erf).max() < 5e-4


def test_silu_against_library_and_identity():
    z = np.linspace(-30, 30, 3001)
    np.testing.assert_allclose(F.silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(),
                               rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(F.silu(z) - F.silu(-z), z, atol=1e-12)


def test_rope_special_cases():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((3, 2, 16))
    # position 0 is the identity
    np.testing.assert_array_equal(F.rope(v, np.zeros(3, int), 10000.0), v)
    # each (i, i + hd/2) pair keeps its norm
    r = F.rope(v, np.array([5, 77, 32767]), 10000.0)
    n0 = v[..., :8] ** 2 + v[..., 8:] ** 2
    n1 = r[..., :8] ** 2 + r[..., 8:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-12)
    # explicit rotation: hd = 4, base 10000: pair (0,2) turns by p rad, pair (1,3) by p/100 rad
    e = np.array([[[1.0, 1.0, 0.0, 0.0]]])
    got = F.rope(e, np.array([1]), 10000.0)[0, 0]
    np.testing.assert_allclose(got, [math.cos(1), math.cos(0.01), math.sin(1), math.sin(0.01)], rtol=1e-15)
    # relative-position property: <rope(q,m), rope(k,n)> depends only on m - n
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    dots = [float((F.rope(q, np.array([m]), 1e4) * F.rope(k, np.array([m - 9]), 1e4)).sum())
            for m in (9, 100, 4000)]
    np.testing.assert_allclose(dots, dots[0], rtol=1e-10)


# ------------------------------------------------------------------ attention

def _attn_loops(q, K, V, pos):
    rows, H, hd = q.shape
    KVH = K.shape[1]
    out = np.zeros((rows, H, hd))
    for t in range(rows):
        for h in range(H):
            g = h * KVH // H
            s = [sum(q[t, h, i] * float(K[j, g, i]) for i in range(hd)) / math.sqrt(hd)
                 for j in range(pos[t] + 1)]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            tot = sum(w)
            for i in range(hd):
                out[t, h, i] = sum(w[j] / tot * float(V[j, g, i]) for j in range(pos[t] + 1))
    return out.reshape(rows, H * hd)


def test_attention_brute_force_gqa_causal_prefix():
    rng = np.random.default_rng(3)
    H, KVH, hd, P = 4, 2, 8, 9
    K = rng.standard_normal((P, KVH, hd)).astype(np.float16)
    V = rng.standard_normal((P, KVH, hd)).astype(np.float16)
    pos = np.array([3, 4, 5, 8])  # queries after a 3-position prefix
    q = rng.standard_normal((4, H, hd)) * 2
    np.testing.assert_allclose(F.attention(q, K, V, pos), _attn_loops(q, K, V, pos), rtol=1e-12, atol=1e-13)


def test_attention_special_cases():
    rng = np.random.default_rng(4)
    K = rng.standard_normal((6, 1, 8))
    V = rng.standard_normal((6, 1, 8))
    q = rng.standard_normal((1, 2, 8))
    # one visible key -> its value
    np.testing.assert_allclose(F.attention(q, K, V, np.array([0])).reshape(2, 8), np.repeat(V[0], 2, 0),
                               rtol=1e-14)
    # identical keys -> the mean of the visible values
    Kc = np.repeat(K[:1], 6, 0)
    np.testing.assert_allclose(F.attention(q, Kc, V, np.array([5])).reshape(2, 8),
                               np.repeat(V.mean(0), 2, 0), rtol=1e-12)
    # a far future key is masked out
    K2 = K.copy(); V2 = V.copy()
    K2[5] = 100 * q[0, 0]; V2[5] = 1e6
    np.testing.assert_allclose(F.attention(q, K2, V2, np.array([4])), F.attention(q, K, V, np.array([4])),
                               rtol=1e-14)


# ------------------------------------------------------------------ whole model

@pytest.mark.parametrize("cfg", [MICRO, MICRO_SW], ids=lambda c: c.name)
def test_oracle_matches_scalar_brute_force(cfg):
    buf = synth.build_model(cfg)
    n = 5
    toks = synth.prompt(cfg, n)
    m = oracle.parse_model(buf)
    kv = oracle.KVState(m, n)
    lg = oracle.prefill(m, kv, toks)
    bm = brute.BruteModel(buf.tobytes())
    blg, bK, bV = brute.brute_prefill(bm, [int(t) for t in toks], n)
    np.testing.assert_allclose(lg, np.array(blg, dtype=np.float32), rtol=2e-6, atol=1e-5)
    np.testing.assert_array_equal(kv.K.astype(np.float64), brute.as_arrays(bK, n))
    np.testing.assert_array_equal(kv.V.astype(np.float64), brute.as_arrays(bV, n))


@pytest.fixture(scope="module")
def tiny():
    buf = synth.build_model("tiny")
    return oracle.parse_model(buf), synth.prompt("tiny", 64)


@pytest.mark.parametrize("cfg", ["tiny", MICRO], ids=["tiny", "micro"])
def test_pruned_equals_unpruned(cfg):
    buf = synth.build_model(cfg)
    m = oracle.parse_model(buf)
    c = synth.CONFIGS[cfg] if isinstance(cfg, str) else cfg
    toks = synth.prompt(c, 48)
    a, b = oracle.KVState(m, 64), oracle.KVState(m, 64)
    la = oracle.prefill(m, a, toks, prune=False)
    lb = oracle.prefill(m, b, toks, prune=True, n_ubatch=16)
    np.testing.assert_allclose(la, lb, rtol=1e-12, atol=1e-12)
    assert np.array_equal(a.K, b.K) and np.array_equal(a.V, b.V)


def test_shared_layers_leave_cache_unchanged(tiny):
    m, toks = tiny
    full = oracle.KVState(m, 64)
    oracle.prefill(m, full, toks)
    # the same model cut after the owning layers writes the same cache
    import copy
    cut = copy.copy(m)
    cut.n_layer = m.n_layer_kv_from_start
    k2 = oracle.KVState(cut, 64)
    oracle.prefill(cut, k2, toks)
    assert np.array_equal(full.K, k2.K) and np.array_equal(full.V, k2.V)


def test_resume_equals_full_prefill(tiny):
    m, toks = tiny
    full = oracle.KVState(m, 64)
    lf = oracle.prefill(m, full, toks)
    for N in (1, 25, 63):
        kv = oracle.KVState(m, 64)
        oracle.prefill(m, kv, toks[:N])
        lr = oracle.prefill(m, kv, toks[N:], prune=True)
        np.testing.assert_allclose(lr, lf, rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(kv.K, full.K)
        np.testing.assert_array_equal(kv.V, full.V)


def test_token_by_token_equals_prefill(tiny):
    m, toks = tiny
    full = oracle.KVState(m, 64)
    lf = oracle.prefill(m, full, toks[:20])
    kv = oracle.KVState(m, 64)
    for t in toks[:20]:
        lt = oracle.prefill(m, kv, [t])
    np.testing.assert_allclose(lt, lf, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(kv.K[:, :20], full.K[:, :20])


def test_ubatch_independence(tiny):
    m, toks = tiny
    outs = []
    for ub in (None, 7, 16, 64):
        kv = oracle.KVState(m, 64)
        outs.append((oracle.prefill(m, kv, toks, n_ubatch=ub), kv.K.copy()))
    for lg, K in outs[1:]:
        np.testing.assert_allclose(lg, outs[0][0], rtol=1e-12, atol=1e-12)
        assert np.array_equal(K, outs[0][1])


def test_prefill_rejects_bad_input(tiny):
    m, toks = tiny
    kv = oracle.KVState(m, 16)
    with pytest.raises(ValueError):
        oracle.prefill(m, kv, [])
    with pytest.raises(ValueError):
        oracle.prefill(m, kv, [m.n_vocab])
    with pytest.raises(ValueError):
        oracle.prefill(m, kv, toks[:17])
    assert kv.n_pos == 0


# ------------------------------------------------------------------ extraction

@pytest.mark.parametrize("cfg", [MICRO, MICRO_SW], ids=lambda c: c.name)
def test_extraction_matches_scalar_brute_force(cfg):
    """Every row's input to every layer (index L: the final rows) and every
    row's output-normed final state, against the scalar brute force."""
    buf = synth.build_model(cfg)
    m = oracle.parse_model(buf)
    n = 5
    toks = synth.prompt(cfg, n)
    inp = {il: None for il in range(m.n_layer + 1)}
    emb = []
    oracle.prefill(m, oracle.KVState(m, n), toks, n_ubatch=2, layer_inp=inp, embeddings=emb)
    hb = {}
    brute.brute_prefill(brute.BruteModel(buf.tobytes()), [int(t) for t in toks], n, hidden=hb)
    for il in range(m.n_layer + 1):
        np.testing.assert_allclose(inp[il], np.array(hb["inp"][il]), rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(emb[0], np.array(hb["embd"]), rtol=1e-9, atol=1e-9)


def test_extraction_invariants(tiny):
    """Layer 0's input is the embedding; row r's final state is the last row
    of the prompt's first r + 1 tokens (causality); the logits are the head
    matrix times the last embedding; a pruned run extracts the owning layers'
    inputs unchanged and refuses layers from the first shared one on."""
    m, toks = tiny
    n, L, ls = 24, m.n_layer, m.n_layer_kv_from_start
    inp = {0: None, 1: None, L: None}
    emb = []
    lg = oracle.prefill(m, oracle.KVState(m, n), toks[:n], layer_inp=inp, embeddings=emb)
    np.testing.assert_array_equal(inp[0], m.embd_scale * m.q4("tok_embd", rows=toks[:n]))
    for r in (0, 9, n - 1):
        tr = {}
        oracle.prefill(m, oracle.KVState(m, n), toks[:r + 1], trace=tr)
        np.testing.assert_allclose(inp[L][r], tr[L - 1], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(emb[0][r], F.rms_norm(tr[L - 1], m.f32("output_norm"), m.rms_eps),
                                   rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lg, (m.q4("tok_embd") @ emb[0][-1]).astype(np.float32), rtol=1e-6, atol=1e-6)
    own = {il: None for il in range(ls)}
    oracle.prefill(m, oracle.KVState(m, n), toks[:n], prune=True, layer_inp=own)
    assert ls == 2
    np.testing.assert_array_equal(own[0], inp[0])
    np.testing.assert_array_equal(own[1], inp[1])
    with pytest.raises(ValueError):
        oracle.prefill(m, oracle.KVState(m, n), toks[:n], prune=True, layer_inp={ls: None})
    with pytest.raises(ValueError):
        oracle.prefill(m, oracle.KVState(m, n), toks[:n], prune=True, embeddings=[])


# ------------------------------------------------------------------ several sequences

@pytest.mark.parametrize("prune", [False, True])
def test_multi_sequence_matches_scalar_brute_force(prune):
    """Two prompts in one pass (rows laid end to end, n_ubatch 3 cuts inside
    both) against the scalar brute force run on each prompt alone."""
    buf = synth.build_model(MICRO)
    m = oracle.parse_model(buf)
    bm = brute.BruteModel(buf.tobytes())
    prompts = [synth.prompt(MICRO, 5), synth.prompt(MICRO, 9)[4:8]]
    kvs = [oracle.KVState(m, 5), oracle.KVState(m, 6)]
    lg = oracle.prefill_multi(m, kvs, prompts, prune=prune, n_ubatch=3)
    assert lg.shape == (2, m.n_vocab) and lg.dtype == np.float32
    for s, t in enumerate(prompts):
        blg, bK, bV = brute.brute_prefill(bm, [int(v) for v in t], kvs[s].n_ctx)
        np.testing.assert_allclose(lg[s], np.array(blg, dtype=np.float32), rtol=2e-6, atol=1e-5)
        n = len(t)
        np.testing.assert_array_equal(kvs[s].K[:, :n].astype(np.float64), brute.as_arrays(bK, n)[:, :n])
        np.testing.assert_array_equal(kvs[s].V[:, :n].astype(np.float64), brute.as_arrays(bV, n)[:, :n])
        assert kvs[s].n_pos == n


def test_multi_sequence_equals_separate_prefills(tiny):
    """Prompts of different lengths, one resuming from cached positions, cut
    into ubatches that straddle sequences: each sequence's logits and cache
    equal those of its own prefill (sequences are independent), pruned or
    not."""
    m, toks = tiny
    lens, starts = (13, 1, 30, 7), (0, 5, 0, 20)
    prompts = [toks[3 * s:3 * s + n] for s, n in enumerate(lens)]

    def fresh():
        kvs = []
        for s, p0 in enumerate(starts):
            kv = oracle.KVState(m, 64)
            if p0:
                oracle.prefill(m, kv, toks[40:40 + p0])
            kvs.append(kv)
        return kvs

    ref_kvs = fresh()
    ref = [oracle.prefill(m, kv, p, prune=False) for kv, p in zip(ref_kvs, prompts)]
    for prune, ub in ((False, None), (True, 8), (True, 64), (False, 5)):
        kvs = fresh()
        lg = oracle.prefill_multi(m, kvs, prompts, prune=prune, n_ubatch=ub)
        for s in range(len(lens)):
            np.testing.assert_allclose(lg[s], ref[s], rtol=1e-12, atol=1e-12)
            np.testing.assert_array_equal(kvs[s].K, ref_kvs[s].K)
            np.testing.assert_array_equal(kvs[s].V, ref_kvs[s].V)
            assert kvs[s].n_pos == starts[s] + lens[s]


def test_multi_sequence_identical_prompts_and_rejections(tiny):
    m, toks = tiny
    kvs = [oracle.KVState(m, 32) for _ in range(3)]
    lg = oracle.prefill_multi(m, kvs, [toks[:11]] * 3, prune=True, n_ubatch=4)
    assert np.array_equal(lg[0], lg[1]) and np.array_equal(lg[1], lg[2])
    kv = oracle.KVState(m, 32)
    with pytest.raises(ValueError):
        oracle.prefill_multi(m, [kv, kv], [toks[:3], toks[:4]])  # one cache for two sequences
    with pytest.raises(ValueError):
        oracle.prefill_multi(m, [kv], [toks[:3], toks[:4]])
    with pytest.raises(ValueError):
        oracle.prefill_multi(m, [kv, oracle.KVState(m, 32)], [toks[:3], []])
    with pytest.raises(ValueError):
        oracle.prefill_multi(m, [kv, oracle.KVState(m, 2)], [toks[:3], toks[:3]])
    assert kv.n_pos == 0


# ------------------------------------------------------------------ unified cache

def test_masked_cell_attention_reduces_to_causal_attention():
    """One sequence in position order is plain causal attention; shuffling
    the cells and adding another sequence's cells (huge values) between
    them changes nothing."""
    rng = np.random.default_rng(21)
    P, H, KVH, hd = 11, 4, 2, 8
    q = rng.standard_normal((P, H, hd))
    K = rng.standard_normal((P, KVH, hd)).astype(np.float16)
    V = rng.standard_normal((P, KVH, hd)).astype(np.float16)
    pos = np.arange(P)
    ref = F.attention(q, K, V, pos)
    got = F.attention_cells(q, K, V, np.zeros(P, np.int64), pos, np.zeros(P, np.int64), pos)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)
    n = 2 * P + 3
    cells = rng.permutation(n)[:P]
    Ku = np.full((n, KVH, hd), 1e4, np.float16)
    Vu = np.full((n, KVH, hd), -1e4, np.float16)
    cs = np.full(n, 7, np.int64)
    cp = np.arange(n) % 5
    cs[-1] = -1
    Ku[cells], Vu[cells], cs[cells], cp[cells] = K, V, 3, pos
    got = F.attention_cells(q, Ku, Vu, cs, cp, np.full(P, 3, np.int64), pos)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def _seq_kv(u, s):
    c = u.cells_of(s)
    return u.K[:, c], u.V[:, c]


@pytest.mark.parametrize("prune", [False, True])
def test_unified_cache_matches_scalar_brute_force(prune):
    """Three prompts in one buffer, ubatches straddling them: each prompt's
    logits and (position -> K/V) against the brute force on that prompt alone."""
    buf = synth.build_model(MICRO)
    m = oracle.parse_model(buf)
    bm = brute.BruteModel(buf.tobytes())
    prompts = [synth.prompt(MICRO, 5), synth.prompt(MICRO, 9)[4:7], synth.prompt(MICRO, 12)[8:12]]
    u = oracle.UnifiedKV(m, 16)
    lg = oracle.prefill_unified(m, u, [4, 0, 2], prompts, prune=prune, n_ubatch=2)
    for i, (sid, t) in enumerate(zip([4, 0, 2], prompts)):
        blg, bK, bV = brute.brute_prefill(bm, [int(v) for v in t], len(t))
        np.testing.assert_allclose(lg[i], np.array(blg, dtype=np.float32), rtol=2e-6, atol=1e-5)
        K, V = _seq_kv(u, sid)
        np.testing.assert_array_equal(K.astype(np.float64), brute.as_arrays(bK, len(t)))
        np.testing.assert_array_equal(V.astype(np.float64), brute.as_arrays(bV, len(t)))
        assert u.n_pos(sid) == len(t)
    assert np.count_nonzero(u.cell_seq == -1) == 16 - 12


def test_unified_cache_interleaved_calls_and_reuse(tiny):
    """Sequences that grow over several calls hold cells scattered through
    the buffer; a removed sequence's cells are reused by a new one.  Each
    sequence matches its own split cache, call by call."""
    m, toks = tiny
    a, b, c = toks[:20], toks[20:45], toks[45:64]
    u = oracle.UnifiedKV(m, 64)
    ka, kb, kc = oracle.KVState(m, 64), oracle.KVState(m, 64), oracle.KVState(m, 64)
    steps = [([0, 1], [a[:7], b[:10]], [ka, kb]), ([1, 0], [b[10:], a[7:]], [kb, ka])]
    for ids, ps, kvs in steps:
        got = oracle.prefill_unified(m, u, ids, ps, n_ubatch=8)
        want = oracle.prefill_multi(m, kvs, ps, n_ubatch=8)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    assert not np.all(np.diff(u.cells_of(0)) == 1)  # sequence 0's cells are not one run
    u.seq_rm(1)
    assert u.n_pos(1) == 0
    lg = oracle.prefill_unified(m, u, [5, 0], [c, b[:3]], prune=True, n_ubatch=16)
    np.testing.assert_allclose(lg[0], oracle.prefill(m, kc, c), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lg[1], oracle.prefill(m, ka, b[:3]), rtol=1e-12, atol=1e-12)
    for sid, kv in ((5, kc), (0, ka)):
        K, V = _seq_kv(u, sid)
        assert np.array_equal(K, kv.K[:, :kv.n_pos]) and np.array_equal(V, kv.V[:, :kv.n_pos])
    with pytest.raises(ValueError):
        oracle.prefill_unified(m, u, [0, 0], [c[:1], c[:1]])
    with pytest.raises(ValueError):
        oracle.prefill_unified(m, u, [9], [toks[:u.n_cells]])


# ------------------------------------------------------------------ next-n head

@pytest.mark.parametrize("cfg", [MICRO, MICRO_SW], ids=lambda c: c.name)
def test_nextn_head_matches_scalar_brute_force(cfg):
    """The head reads the second-to-last row's final state: against the
    scalar brute force, with the two rows in different ubatches; requesting
    it changes nothing else."""
    c = dataclasses.replace(cfg, nextn=True)
    buf = synth.build_model(c)
    m = oracle.parse_model(buf)
    toks = synth.prompt(c, 5)
    out = []
    kv = oracle.KVState(m, 5)
    lg = oracle.prefill(m, kv, toks, n_ubatch=2, nextn=out)
    ref = brute.brute_nextn(brute.BruteModel(buf.tobytes()), [int(t) for t in toks], 5)
    np.testing.assert_allclose(out[0], np.array(ref, dtype=np.float32), rtol=2e-6, atol=1e-5)
    kv2 = oracle.KVState(m, 5)
    assert np.array_equal(lg, oracle.prefill(m, kv2, toks, n_ubatch=2))
    assert np.array_equal(kv.K, kv2.K) and np.array_equal(kv.V, kv2.V)
    assert not np.allclose(out[0], lg, atol=1e-3)


def test_nextn_head_resumes_and_refuses_the_prune(tiny):
    """Rows before the call come from the cache: a call after N cached
    positions gives the head of the full prompt (its second-to-last row sees
    the same keys).  The head needs a row the prune drops, a second row, and
    a model that has it."""
    m, toks = tiny
    full = []
    oracle.prefill(m, oracle.KVState(m, 64), toks, nextn=full)
    for N in (1, 40, 62):
        kv = oracle.KVState(m, 64)
        oracle.prefill(m, kv, toks[:N])
        got = []
        oracle.prefill(m, kv, toks[N:], nextn=got)
        np.testing.assert_allclose(got[0], full[0], rtol=1e-6, atol=1e-6)
    with pytest.raises(ValueError):
        oracle.prefill(m, oracle.KVState(m, 64), toks, prune=True, nextn=[])
    with pytest.raises(ValueError):
        oracle.prefill(m, oracle.KVState(m, 64), toks[:1], nextn=[])
    plain = oracle.parse_model(synth.build_model(dataclasses.replace(MICRO, nextn=False)))
    with pytest.raises(ValueError):
        oracle.prefill(plain, oracle.KVState(plain, 4), synth.prompt(MICRO, 4), nextn=[])
    assert not oracle.prune_shared(m.n_layer, m.n_layer_kv_from_start, False, 1, [0] * (m.n_layer + 1),
                                   crop_before_nextn=False)


# ------------------------------------------------------------------ predicate and snapshot

def test_prune_predicate_truth_table():
    g = _gold("prune_predicate.json")
    for c in g["cases"]:
        L = c["n_layer"]
        inp = [False] * (L + 1)
        for i in c["layer_inp_true"]:
            inp[i] = True
        got = oracle.prune_shared(L, c["n_layer_kv_from_start"], c["embeddings"], c["n_seq_max"], inp,
                                  c["crop_before_nextn"])
        assert got == c["expected"], c["note"]


def test_kvcp_size_pin():
    g = _gold("kvcp_tinyllama_25.json")
    K = np.zeros((g["n_layers"], g["n_pos"], g["kv_dim"]), np.float16)
    data = oracle.kvcp.dump(K, K, g["n_pos"])
    assert len(data) - oracle.kvcp.HEADER == g["payload_bytes"] == 563200
    assert round((len(data) - oracle.kvcp.HEADER) / 1024) == g["approx_kib"]


def test_kvcp_round_trip_and_rejections():
    rng = np.random.default_rng(6)
    K = rng.standard_normal((3, 10, 16)).astype(np.float16)
    V = rng.standard_normal((3, 10, 16)).astype(np.float16)
    data = oracle.kvcp.dump(K, V, 10)
    k2, v2 = oracle.kvcp.load(data, 3, 16, 4, 100)
    assert np.array_equal(k2, K[:, :4]) and np.array_equal(v2, V[:, :4])
    bad = [(b"XXXX" + data[4:], 3, 16, 4, 100), (data, 2, 16, 4, 100), (data, 3, 8, 4, 100),
           (data[:-2], 3, 16, 4, 100), (data, 3, 16, 11, 100), (data, 3, 16, 4, 3), (data[:10], 3, 16, 1, 10)]
    for args in bad:
        with pytest.raises(oracle.kvcp.SnapshotError):
            oracle.kvcp.load(*args)


def test_kvcp_header_and_body_order_against_hand_written_bytes():
    """The PicoLM page's file contents, in its order: the magic, then the
    cached positions, the layer count and the KV dimension, then K, then V.
    The expected header is typed out byte by byte here (25 positions, 22
    layers, KV dim 256 -- the page's TinyLlama example), so a swap of two
    header fields in both the writer and the reader fails; the body offsets
    are computed by hand from [layer][position][dim] order."""
    nl, npos, kvd = 22, 25, 256
    K = np.zeros((nl, npos, kvd), np.float16)
    V = np.zeros((nl, npos, kvd), np.float16)
    K[3, 7, 5] = 1.5     # fp16 0x3E00
    V[21, 24, 255] = -2.0  # fp16 0xC000
    data = oracle.kvcp.dump(K, V, npos)
    assert data[:16] == bytes([0x4B, 0x56, 0x43, 0x50, 25, 0, 0, 0, 22, 0, 0, 0, 0, 1, 0, 0])
    k_off = 16 + 2 * ((3 * npos + 7) * kvd + 5)
    assert data[k_off:k_off + 2] == bytes([0x00, 0x3E])
    v_off = 16 + 2 * nl * npos * kvd + 2 * ((21 * npos + 24) * kvd + 255)
    assert data[v_off:v_off + 2] == bytes([0x00, 0xC0])
    assert v_off + 2 == len(data)
    assert sum(1 for b in data[16:] if b) == 2  # the two high bytes above; nothing else is set
    # a header typed with the layer count and the position count swapped is
    # refused by the reader (the layer count no longer matches the model)
    swapped = bytes([0x4B, 0x56, 0x43, 0x50, 22, 0, 0, 0, 25, 0, 0, 0, 0, 1, 0, 0]) + data[16:]
    with pytest.raises(oracle.kvcp.SnapshotError):
        oracle.kvcp.load(swapped, nl, kvd, 1, 100)
    k2, v2 = oracle.kvcp.load(data, nl, kvd, npos, 100)
    assert k2[3, 7, 5] == 1.5 and v2[21, 24, 255] == -2.0
