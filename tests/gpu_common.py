"""Helpers for the GPU parity tests: model caching, tolerances, and the
engine's documented row orders of fused weights (used to lay the oracle's
dequantised tensors out the way the kernel-level entry points return them)."""
import functools
import os

import numpy as np

import oracle
import synth

MODEL_DIR = os.environ.get("PPX_MODEL_DIR", "/tmp/ppx_models")


@functools.lru_cache(maxsize=2)
def container(name):
    return synth.build_model(name)


@functools.lru_cache(maxsize=2)
def oracle_model(name):
    return oracle.parse_model(container(name))


def rope_pair_rows(n_rows, hd):
    """Row order of a Q or K weight in the engine: 16-row blocks alternate the
    first and second half of each head, so rope partners share a lane."""
    out = []
    for r in range(n_rows):
        h, rr = divmod(r, hd)
        blk, c = divmod(rr, 16)
        out.append(h * hd + (blk & 1) * (hd // 2) + (blk >> 1) * 16 + c)
    return np.array(out)


def fused_reference(m, name):
    """fp64 [rows, cols] of an engine tensor as the kernel entry points see it."""
    if name in ("tok_embd", "output"):
        return m.q4(name)
    il = int(name.split(".")[1])
    kind = name.split(".", 2)[2]
    p = f"blk.{il}."
    hd = m.head_dim
    if kind == "wq":
        return m.q4(p + "wq")[rope_pair_rows(m.n_head * hd, hd)]
    if kind == "wk":
        return np.concatenate([m.q4(p + "wk")[rope_pair_rows(m.kv_dim, hd)], m.q4(p + "wv")], 0)
    if kind == "ffn_gate":
        g, u = m.q4(p + "ffn_gate"), m.q4(p + "ffn_up")
        F = g.shape[0]
        rows = []
        for r in range(2 * F):
            blk, c = divmod(r, 8)
            rows.append((u if blk & 1 else g)[(blk >> 1) * 8 + c])
        return np.stack(rows)
    return m.q4(p + kind)


def oracle_kv_from_rows(m, il, x_rows, pos):
    """The oracle's fp16 K and V of owning layer il computed from given layer-input
    rows x_rows [r][d] (fp64) at positions pos [r]."""
    p = f"blk.{il}."
    a = oracle.rms_norm(x_rows.astype(np.float64), m.f32(p + "attn_norm"), m.rms_eps)
    r = a.shape[0]
    k = oracle.rope((a @ m.q4(p + "wk").T).reshape(r, m.n_kv_head, m.head_dim), pos, m.rope_base)
    v = a @ m.q4(p + "wv").T
    return k.reshape(r, -1).astype(np.float16), v.astype(np.float16)


def ulp16(x):
    """Spacing of fp16 numbers at |x| (normal range)."""
    ax = np.maximum(np.abs(x), 2.0 ** -14)
    return 2.0 ** (np.floor(np.log2(ax)) - 10)


def kv_within(got, ref):
    """KV tolerance: |d| <= 1e-2 + one fp16 ulp of the reference value."""
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    d = np.abs(got - ref)
    return bool(np.all(d <= 1e-2 + ulp16(ref))), float(d.max())


def logits_ok(got, ref, atol=2e-2):
    """max-abs <= atol and identical top-1 (a top-2 tie within atol passes)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = float(np.abs(got - ref).max())
    top = int(np.argmax(ref))
    srt = np.sort(ref)
    tie = srt[-1] - srt[-2] < atol
    same = int(np.argmax(got)) == top or (tie and int(np.argmax(got)) in set(np.argsort(ref)[-2:]))
    return d <= atol and same, d
