"""Conditioning of the tiny synthetic model for very short prompts (CPU).

The engine's fast path rounds GEMM activations and weights (d * (q - 8)) to
fp16 and the query to fp16 before attention.  Applying exactly those
roundings to the fp64 oracle's own pass shows how far any implementation with
fp16 operands must land from the exact logits.  On the tiny model the residual
grows about 15x per layer and the last layer's scores reach ~60, so for the
2-token prompt below the roundings alone move the logits by more than the
2e-2 bound, while for a 64-token prompt (the GPU parity test's) they stay
well inside it.  This is a property of that synthetic model; the E2B-like
model is held to the bound at every prompt length the GPU tests run.
"""
import math

import numpy as np

import oracle
import synth
from oracle import forward as F


def _pass(m, toks, rounded):
    f16 = (lambda a: a.astype(np.float16).astype(np.float64)) if rounded else (lambda a: a)
    H, KVH, hd, L, ls = m.n_head, m.n_kv_head, m.head_dim, m.n_layer, m.n_layer_kv_from_start
    n = len(toks)
    pos = np.arange(n)
    K = np.zeros((ls, n, m.kv_dim))
    V = np.zeros((ls, n, m.kv_dim))
    x = F.embed_rows(m, np.asarray(toks))
    W = lambda name: f16(m.q4(name))  # noqa: E731  fast-mode weights
    for il in range(L):
        p = f"blk.{il}."
        src = il if il < ls else m.kv_src[il]
        a = F.rms_norm(x, m.f32(p + "attn_norm"), m.rms_eps)
        q = f16(F.rope((f16(a) @ W(p + "wq").T).reshape(n, H, hd), pos, m.rope_base))
        if il < ls:  # the K|V projection is exact in the engine: only the fp16 store rounds
            K[il] = F.rope((a @ m.q4(p + "wk").T).reshape(n, KVH, hd), pos, m.rope_base).reshape(n, -1)
            V[il] = a @ m.q4(p + "wv").T
            K[il], V[il] = K[il].astype(np.float16), V[il].astype(np.float16)
        o = F.attention(q, K[src].reshape(n, KVH, hd), V[src].reshape(n, KVH, hd), pos)
        x = x + f16(o) @ W(p + "wo").T
        b = f16(F.rms_norm(x, m.f32(p + "ffn_norm"), m.rms_eps))
        h = F.gelu_tanh(b @ W(p + "ffn_gate").T) * (b @ W(p + "ffn_up").T)
        x = x + f16(h) @ W(p + "ffn_down").T
    return F.head(m, x[-1]).astype(np.float64)


def test_fp16_operands_alone_exceed_the_bound_on_a_two_token_tiny_prompt():
    m = oracle.parse_model(synth.build_model("tiny"))
    assert m.ple_dim == 0 and m.act == 0
    base = synth.prompt("tiny", 64)
    exact = _pass(m, base[:2], False)
    ref = oracle.prefill(m, oracle.KVState(m, 2), base[:2]).astype(np.float64)
    np.testing.assert_allclose(exact, ref, rtol=1e-6, atol=1e-5)  # the helper is the oracle's pass
    rng = np.random.default_rng(64)
    lens = [int(v) for v in rng.integers(1, 6, 64)]
    off = sum(lens[:26])
    toks = synth.prompt("tiny", sum(lens) + 8)[off:off + lens[26]]
    assert len(toks) == 2
    d_short = np.abs(_pass(m, toks, True) - _pass(m, toks, False)).max()
    d_long = np.abs(_pass(m, base, True) - _pass(m, base, False)).max()
    print(f"fp16-operand deviation: 2 tokens {d_short:.4f}, 64 tokens {d_long:.4f}")
    assert d_short > 2e-2 and d_long < 1e-2
    assert math.isfinite(d_short)


def _layer_kv(m, toks, w16, a16, q16, o16):
    """The owning layers' fp16 K/V of the oracle's pass with chosen operands
    rounded to fp16: weights d * (q - 8) (w16), GEMM activations (a16), the
    attention query (q16) and the attention output (o16).  The K/V
    projection itself stays exact, as in the engine."""
    f16 = lambda a: a.astype(np.float16).astype(np.float64)  # noqa: E731
    same = lambda a: a  # noqa: E731
    H, KVH, hd, L, ls = m.n_head, m.n_kv_head, m.head_dim, m.n_layer, m.n_layer_kv_from_start
    n = len(toks)
    pos = np.arange(n)
    K = np.zeros((ls, n, m.kv_dim))
    V = np.zeros((ls, n, m.kv_dim))
    x = F.embed_rows(m, np.asarray(toks))
    W = lambda name: (f16 if w16 else same)(m.q4(name))  # noqa: E731
    A = f16 if a16 else same
    for il in range(L):
        p = f"blk.{il}."
        src = il if il < ls else m.kv_src[il]
        a = F.rms_norm(x, m.f32(p + "attn_norm"), m.rms_eps)
        q = (f16 if q16 else same)(F.rope((A(a) @ W(p + "wq").T).reshape(n, H, hd), pos, m.rope_base))
        if il < ls:
            K[il] = F.rope((a @ m.q4(p + "wk").T).reshape(n, KVH, hd), pos, m.rope_base).reshape(n, -1)
            V[il] = a @ m.q4(p + "wv").T
            K[il], V[il] = K[il].astype(np.float16), V[il].astype(np.float16)
        o = F.attention(q, K[src].reshape(n, KVH, hd), V[src].reshape(n, KVH, hd), pos)
        x = x + (f16 if o16 else same)(o) @ W(p + "wo").T
        b = A(F.rms_norm(x, m.f32(p + "ffn_norm"), m.rms_eps))
        h = F.gelu_tanh(b @ W(p + "ffn_gate").T) * (b @ W(p + "ffn_up").T)
        x = x + A(h) @ W(p + "ffn_down").T
    return K, V


def _within(got, ref):
    """The GPU tests' KV bound: |d| <= 1e-2 + one fp16 ulp of the reference."""
    ax = np.maximum(np.abs(ref), 2.0 ** -14)
    return bool(np.all(np.abs(got - ref) <= 1e-2 + 2.0 ** (np.floor(np.log2(ax)) - 10)))


def test_fp16_query_and_attention_output_alone_break_the_tiny_layer1_kv_bound():
    """Why the fast path's every-layer KV check on the tiny model is an
    expected failure and the exact precision exists: applied to the oracle's
    own 64-token pass, the fast path's roundings put layer 1's K/V outside the
    1e-2 bound, and so do fp16 rounding of the attention query and output
    alone, with exact weights and activations -- any fp16-operand attention
    does.  Layer 0 (embedding only) stays inside; with nothing rounded the
    pass is the oracle itself."""
    m = oracle.parse_model(synth.build_model("tiny"))
    toks = synth.prompt("tiny", 64)
    K0, V0 = _layer_kv(m, toks, False, False, False, False)
    kv = oracle.KVState(m, 64)
    oracle.prefill(m, kv, toks)
    assert np.array_equal(K0.astype(np.float16), kv.K) and np.array_equal(V0.astype(np.float16), kv.V)
    Kf, Vf = _layer_kv(m, toks, True, True, True, True)        # the fast path's roundings
    Kq, Vq = _layer_kv(m, toks, False, False, True, True)      # fp16 query and attention output only
    assert _within(Kf[0], K0[0]) and _within(Vf[0], V0[0])
    assert not (_within(Kf[1], K0[1]) and _within(Vf[1], V0[1]))
    assert not (_within(Kq[1], K0[1]) and _within(Vq[1], V0[1]))
