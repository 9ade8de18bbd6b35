"""Oracle: the prompt-prefill forward pass in fp64 (test infrastructure).

What is computed is the plain definition: every prompt row through every
layer, then the logits of the last row.  The pruned schedule is also here so
that it can be checked against that definition; the llama.cpp Gemma 4 prefill
page (section 1) states that KV-shared layers write no cache, so in those
layers a row's output depends only on itself and on caches that are already
final, and only the output row has to be kept (section 3: outputs identical).

Model reading (the pages name a "Gemma-style" decoder without its layer
math; the plainest pre-norm decoder is used):
  x_t      = embd_scale * deq(tok_embd[id_t])
  per layer il (own = il < n_layer_kv_from_start, src = kv source layer):
    a      = rms(x, g_attn);  q = rope(Wq a)
    own:     K[il][pos] = fp16(rope(Wk a)),  V[il][pos] = fp16(Wv a)
    o      = causal attention of q over K[src], V[src] (fp16 cache values)
    x     += Wo o
    b      = rms(x, g_ffn);   x += Wd act(Wg b, Wu b)
    ple_dim > 0:  c = rms(x, g_ple);  P = s_il * deq(ple_table[id_t])[il*E:(il+1)*E]
                  x += Wple_up (gelu(Wple_gate c) * P)
  logits   = W_out rms(x_last, g_out)   (W_out = tok_embd when tied), fp32
All arithmetic is fp64; the only roundings are the fp16 cache store
(round to nearest even) and the fp32 logits.
"""
from __future__ import annotations

import math

import numpy as np

from .model import OracleModel


# ---------------------------------------------------------------- components

def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g, over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope(v: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotary embedding, half-split pairs (i, i + hd/2).

    v: [rows, heads, hd]; pos: [rows] absolute positions.  The angle of pair i
    at position p is p * base^(-2i/hd), in fp64.
    """
    hd = v.shape[-1]
    half = hd // 2
    i = np.arange(half, dtype=np.float64)
    theta = base ** (-2.0 * i / hd)
    ang = pos.astype(np.float64)[:, None] * theta[None, :]  # [rows, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a, b = v[..., :half], v[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def gelu_tanh(z: np.ndarray) -> np.ndarray:
    return 0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """Causal softmax attention.

    q: [rows, H, hd] fp64; K, V: [P, KVH, hd] (cache, any float dtype);
    pos: [rows].  Row t attends to cache positions 0..pos[t].  Query head h
    uses KV head h // (H / KVH).  Returns [rows, H*hd].
    """
    rows, H, hd = q.shape
    KVH = K.shape[1]
    grp = H // KVH
    P = int(pos.max()) + 1
    Kf = K[:P].astype(np.float64)
    Vf = V[:P].astype(np.float64)
    out = np.empty((rows, H, hd), dtype=np.float64)
    scale = 1.0 / math.sqrt(hd)
    j = np.arange(P)
    chunk = max(1, (1 << 24) // max(P, 1))
    for h in range(H):
        g = h // grp
        for s in range(0, rows, chunk):
            e = min(rows, s + chunk)
            sc = (q[s:e, h, :] @ Kf[:, g, :].T) * scale          # [r, P]
            sc = np.where(j[None, :] <= pos[s:e, None], sc, -np.inf)
            sc = sc - sc.max(axis=1, keepdims=True)
            w = np.exp(sc)
            w = w / w.sum(axis=1, keepdims=True)
            out[s:e, h, :] = w @ Vf[:, g, :]
    return out.reshape(rows, H * hd)


# ---------------------------------------------------------------- KV state

class KVState:
    """fp16 K and V for the owning layers: [Ls][n_ctx][kv_dim] each."""

    def __init__(self, m: OracleModel, n_ctx: int):
        ls = m.n_layer_kv_from_start
        self.n_ctx = n_ctx
        self.K = np.zeros((ls, n_ctx, m.kv_dim), dtype=np.float16)
        self.V = np.zeros((ls, n_ctx, m.kv_dim), dtype=np.float16)
        self.n_pos = 0

    def copy(self) -> "KVState":
        c = KVState.__new__(KVState)
        c.n_ctx, c.K, c.V, c.n_pos = self.n_ctx, self.K.copy(), self.V.copy(), self.n_pos
        return c


class UnifiedKV:
    """One fp16 K and V buffer shared by several sequences, [Ls][n_cells][kv_dim]
    each; cell c holds position cell_pos[c] of sequence cell_seq[c] (-1: a
    free cell).  The llama.cpp Gemma 4 prefill page (section 5) contrasts this
    unified cache with one cache per sequence (split)."""

    def __init__(self, m: OracleModel, n_cells: int):
        ls = m.n_layer_kv_from_start
        self.n_cells = n_cells
        self.K = np.zeros((ls, n_cells, m.kv_dim), dtype=np.float16)
        self.V = np.zeros((ls, n_cells, m.kv_dim), dtype=np.float16)
        self.cell_seq = np.full(n_cells, -1, dtype=np.int64)
        self.cell_pos = np.full(n_cells, -1, dtype=np.int64)

    def n_pos(self, s: int) -> int:
        return int(np.count_nonzero(self.cell_seq == s))

    def cells_of(self, s: int) -> np.ndarray:
        """The cells of sequence s in position order."""
        c = np.nonzero(self.cell_seq == s)[0]
        return c[np.argsort(self.cell_pos[c])]

    def seq_rm(self, s: int) -> None:
        """Free every cell of sequence s (their contents stay, never read)."""
        free = self.cell_seq == s
        self.cell_seq[free] = -1
        self.cell_pos[free] = -1


class _UnifiedSeq:
    """Sequence s of a unified cache as _run sees a cache: its position count
    and capacity (the cells that are free or already its own)."""

    def __init__(self, u: UnifiedKV, s: int):
        self.u, self.s = u, s
        self.n_pos = u.n_pos(s)
        self.n_ctx = self.n_pos + int(np.count_nonzero(u.cell_seq == -1))


def attention_cells(q: np.ndarray, K: np.ndarray, V: np.ndarray, cell_seq: np.ndarray, cell_pos: np.ndarray,
                    seq: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """Softmax attention over the cells of one shared buffer: row t sees
    every cell c with cell_seq[c] == seq[t] and cell_pos[c] <= pos[t] (the
    mask by sequence and position); other cells get weight zero.
    q: [rows, H, hd] fp64; K, V: [n_cells, KVH, hd]; returns [rows, H*hd]."""
    rows, H, hd = q.shape
    grp = H // K.shape[1]
    Kf, Vf = K.astype(np.float64), V.astype(np.float64)
    vis = (cell_seq[None, :] == seq[:, None]) & (cell_pos[None, :] >= 0) & (cell_pos[None, :] <= pos[:, None])
    out = np.empty((rows, H, hd), dtype=np.float64)
    scale = 1.0 / math.sqrt(hd)
    for h in range(H):
        g = h // grp
        sc = np.where(vis, (q[:, h, :] @ Kf[:, g, :].T) * scale, -np.inf)
        sc = sc - sc.max(axis=1, keepdims=True)
        w = np.exp(sc)
        out[:, h, :] = (w / w.sum(axis=1, keepdims=True)) @ Vf[:, g, :]
    return out.reshape(rows, H * hd)


# ---------------------------------------------------------------- forward

def embed_rows(m: OracleModel, tokens: np.ndarray) -> np.ndarray:
    return m.embd_scale * m.q4("tok_embd", rows=tokens)


def _layer(m: OracleModel, kvs: list, il: int, x: np.ndarray, pos: np.ndarray,
           toks: np.ndarray, seq: np.ndarray, W: dict, cell: np.ndarray | None = None) -> np.ndarray:
    """Layer il for rows x of sequences seq (row t belongs to kvs[seq[t]]).

    Every row's K/V goes into its own sequence's cache before any row
    attends, and a row attends only to its own sequence's cache.  With a
    unified cache (kvs[s] = _UnifiedSeq) row t's K/V go to cell cell[t] of
    the one buffer and attention masks the buffer's cells by sequence.
    """
    H, KVH, hd = m.n_head, m.n_kv_head, m.head_dim
    own = il < m.n_layer_kv_from_start
    src = il if own else m.kv_src[il]
    r = x.shape[0]

    a = rms_norm(x, W["attn_norm"], m.rms_eps)
    q = rope((a @ W["wq"].T).reshape(r, H, hd), pos, m.rope_base)
    groups = [(int(s), np.nonzero(seq == s)[0]) for s in np.unique(seq)]
    if cell is not None:
        u = kvs[0].u
        sid = np.array([kvs[int(s)].s for s in seq])
        if own:
            u.K[il, cell] = rope((a @ W["wk"].T).reshape(r, KVH, hd), pos, m.rope_base).reshape(r, -1).astype(np.float16)
            u.V[il, cell] = (a @ W["wv"].T).astype(np.float16)
        o = attention_cells(q, u.K[src].reshape(-1, KVH, hd), u.V[src].reshape(-1, KVH, hd),
                            u.cell_seq, u.cell_pos, sid, pos)
        return _layer_tail(m, il, x + o @ W["wo"].T, toks, W)
    if own:
        k = rope((a @ W["wk"].T).reshape(r, KVH, hd), pos, m.rope_base).reshape(r, KVH * hd)
        v = a @ W["wv"].T
        for s, rows in groups:
            kvs[s].K[il, pos[rows]] = k[rows].astype(np.float16)
            kvs[s].V[il, pos[rows]] = v[rows].astype(np.float16)
    o = np.empty((r, H * hd), dtype=np.float64)
    for s, rows in groups:
        kv = kvs[s]
        if own:
            Kc, Vc = kv.K[il], kv.V[il]
        else:
            # a shared layer only reads its source layer's cache
            Kc, Vc = kv.K[src].view(), kv.V[src].view()
            Kc.flags.writeable = False
            Vc.flags.writeable = False
        o[rows] = attention(q[rows], Kc.reshape(-1, KVH, hd), Vc.reshape(-1, KVH, hd), pos[rows])
    return _layer_tail(m, il, x + o @ W["wo"].T, toks, W)


def _layer_tail(m: OracleModel, il: int, x: np.ndarray, toks: np.ndarray, W: dict) -> np.ndarray:
    """The feed-forward block and the per-layer embedding of layer il."""
    b = rms_norm(x, W["ffn_norm"], m.rms_eps)
    gt = b @ W["ffn_gate"].T
    up = b @ W["ffn_up"].T
    hact = (gelu_tanh(gt) if m.act == 0 else silu(gt)) * up
    x = x + hact @ W["ffn_down"].T

    if m.ple_dim:
        E = m.ple_dim
        c = rms_norm(x, W["ple_norm"], m.rms_eps)
        P = m.ple_scale[il] * m.q4("ple_table", rows=toks)[:, il * E:(il + 1) * E]
        x = x + (gelu_tanh(c @ W["ple_gate"].T) * P) @ W["ple_up"].T
    return x


def _layer_weights(m: OracleModel, il: int) -> dict:
    p = f"blk.{il}."
    W = {}
    for name, t in m.tensors.items():
        if name.startswith(p):
            key = name[len(p):]
            W[key] = m.f32(name) if t.ttype == 0 else m.q4(name)
    return W


def head(m: OracleModel, x_last: np.ndarray, chunk: int = 16384, gain: str = "output_norm") -> np.ndarray:
    """fp32 logits of one row: W_out rms(x, g), g the output norm's gain."""
    hn = rms_norm(x_last, m.f32(gain), m.rms_eps)
    name = "tok_embd" if m.tied else "output"
    V = m.n_vocab
    out = np.empty(V, dtype=np.float64)
    for s in range(0, V, chunk):
        e = min(V, s + chunk)
        out[s:e] = m.q4(name, rows=np.arange(s, e)) @ hn
    return out.astype(np.float32)


def _check_prompt(m: OracleModel, kv: KVState, tokens: np.ndarray) -> None:
    n = int(tokens.shape[0])
    if n < 1:
        raise ValueError("empty prompt")
    if tokens.min() < 0 or tokens.max() >= m.n_vocab:
        raise ValueError("token id out of range")
    if kv.n_pos + n > kv.n_ctx:
        raise ValueError("context overflow")


def nextn_head(m: OracleModel, x_prev: np.ndarray, tok_last: int) -> np.ndarray:
    """fp32 logits of the next-n head.

    The pages name a next-n (multi-token prediction) head only through the
    prune predicate's crop_before_nextn clause (the llama.cpp Gemma 4 prefill
    page, section 1); the definition used here is the plainest depth-1
    multi-token predictor, sharing the model's output matrix as such heads
    usually do: it combines the final hidden state of the row BEFORE the last
    one with the embedding of the last token,
        z = x_{n-2} + embd_scale * deq(tok_embd[id_{n-1}]),
        logits = W_out rms(z, g_nextn),
    so it needs a row that the prune drops."""
    z = x_prev + embed_rows(m, np.array([tok_last]))[0]
    return head(m, z, gain="nextn_norm")


def _run(m: OracleModel, kvs: list, prompts: list, prune: bool, n_ubatch: int | None,
         trace: dict | None, layer_inp: dict | None = None, embeddings: list | None = None,
         nextn: list | None = None, unified: UnifiedKV | None = None) -> np.ndarray:
    """The forward pass over the rows of all prompts, laid end to end in
    prompt order; returns the logits of each prompt's last row.

    layer_inp: keys are layer indices il in [0, n_layer]; each value becomes
    the hidden state entering layer il for every row ([rows][d], fp64;
    il = n_layer is the final hidden state before the output norm).
    embeddings: receives every row's output-normed final hidden state.  Both
    need every row, so a pruned run may request only layers before the first
    KV-shared one (the llama.cpp Gemma 4 prefill page, section 1: the
    predicate forbids pruning when a layer from there on, or the embeddings,
    are extracted)."""
    if len({id(kv) for kv in kvs}) != len(kvs):
        raise ValueError("each sequence needs its own cache")
    prompts = [np.asarray(t, dtype=np.int64) for t in prompts]
    for kv, t in zip(kvs, prompts):
        _check_prompt(m, kv, t)
    ls, L = m.n_layer_kv_from_start, m.n_layer
    want = sorted(layer_inp) if layer_inp is not None else []
    if any(il < 0 or il > L for il in want):
        raise ValueError("layer index out of range")
    if prune and 0 < ls < L and (embeddings is not None or any(il >= ls for il in want)):
        raise ValueError("extraction from pruned layers needs every row")
    if nextn is not None:
        if "nextn_norm" not in m.tensors:
            raise ValueError("the model has no next-n head")
        if len(prompts) != 1 or len(prompts[0]) < 2:
            raise ValueError("the next-n head reads the second-to-last row of one prompt")
        if prune and 0 < ls < L:
            raise ValueError("the next-n head needs a row the prune drops")
    toks = np.concatenate(prompts)
    seq = np.concatenate([np.full(len(t), s, dtype=np.int64) for s, t in enumerate(prompts)])
    pos = np.concatenate([kv.n_pos + np.arange(len(t)) for kv, t in zip(kvs, prompts)])
    last = np.cumsum([len(t) for t in prompts]) - 1  # each prompt's output row
    cell = None
    if unified is not None:
        # the rows take the lowest free cells, in row order
        free = np.nonzero(unified.cell_seq == -1)[0]
        if free.shape[0] < toks.shape[0]:
            raise ValueError("context overflow")
        cell = free[:toks.shape[0]]
        unified.cell_seq[cell] = np.array([kvs[int(q)].s for q in seq])
        unified.cell_pos[cell] = pos
    ub = toks.shape[0] if n_ubatch is None else int(n_ubatch)
    x = embed_rows(m, toks)
    for il in range(L):
        if prune and il == ls and 0 < ls < L:
            x, pos, toks, seq = x[last], pos[last], toks[last], seq[last]
            cell = cell[last] if cell is not None else None
            last = np.arange(len(prompts))
        if il in want:
            layer_inp[il] = x.copy()
        W = _layer_weights(m, il)
        parts = []
        for s in range(0, x.shape[0], ub):
            e = min(x.shape[0], s + ub)
            parts.append(_layer(m, kvs, il, x[s:e], pos[s:e], toks[s:e], seq[s:e], W,
                                None if cell is None else cell[s:e]))
        x = np.concatenate(parts, axis=0)
        del W
        if trace is not None:
            trace[il] = x[last[-1]].copy()
    if L in want:
        layer_inp[L] = x.copy()
    if embeddings is not None:
        embeddings.append(rms_norm(x, m.f32("output_norm"), m.rms_eps))
    if nextn is not None:
        nextn.append(nextn_head(m, x[last[0] - 1], int(toks[last[0]])))
    logits = np.stack([head(m, x[r]) for r in last])
    for kv, t in zip(kvs, prompts):
        kv.n_pos += len(t)
    return logits


def prefill(m: OracleModel, kv: KVState, tokens, prune: bool = False,
            n_ubatch: int | None = None, trace: dict | None = None,
            layer_inp: dict | None = None, embeddings: list | None = None,
            nextn: list | None = None) -> np.ndarray:
    """Run the prompt `tokens` from position kv.n_pos; return last-row logits.

    prune=False is the plain definition: all rows through all layers.
    prune=True keeps only the last row from the first KV-shared layer on (the
    pages' schedule: intermediate ubatches stop before that layer, the last
    ubatch carries one row through the remaining layers).

    Layers are the outer loop.  Within a layer the rows are taken in ubatch
    order (n_ubatch rows at a time, or all at once when None); each chunk
    writes its K/V before it attends, so it sees exactly the cache the
    ubatch-by-ubatch schedule would give it.  trace, if given, receives the
    last row's hidden state after each layer.  layer_inp / embeddings: the
    extraction outputs described at _run.  nextn, if given, receives the
    next-n head's logits (nextn_head); the prune cannot serve it.
    """
    return _run(m, [kv], [tokens], prune, n_ubatch, trace, layer_inp, embeddings, nextn)[0]


def prefill_multi(m: OracleModel, kvs: list, prompts: list, prune: bool = False,
                  n_ubatch: int | None = None) -> np.ndarray:
    """Several independent prompts in one pass: prompt s runs from
    kvs[s].n_pos in its own cache, and its last row's logits are row s of
    the result ([n_seq][n_vocab], fp32).

    The rows of all prompts are laid end to end and cut into ubatches of
    n_ubatch rows, so one ubatch can hold the end of one prompt and the start
    of the next; a row attends only to keys of its own sequence.  prune=True
    generalises the pages' single-sequence prune to one output row per
    sequence: before the first KV-shared layer the last row of every prompt
    is gathered, and those rows alone run the KV-shared layers, each reading
    its own sequence's source-layer cache.  By definition the result equals
    running each prompt alone, which is what the pins check.
    """
    if len(prompts) < 1 or len(prompts) != len(kvs):
        raise ValueError("one cache per prompt, at least one prompt")
    return _run(m, list(kvs), list(prompts), prune, n_ubatch, None)


def prefill_unified(m: OracleModel, u: UnifiedKV, seq_ids, prompts, prune: bool = False,
                    n_ubatch: int | None = None) -> np.ndarray:
    """Several prompts in one pass over ONE cache: prompt i belongs to
    sequence seq_ids[i] and runs from that sequence's position count in u.
    The rows take free cells of u (lowest first, in row order); each row's
    K/V go to its cell, and it attends to the cells of its own sequence up
    to its position (attention_cells).  Ubatching and pruning are those of
    prefill_multi; the logits ([n_seq][n_vocab], fp32) and each sequence's
    (position -> K/V) contents are by definition those of prefill_multi
    with one cache per sequence, which is what the pins check."""
    ids = [int(v) for v in seq_ids]
    if len(prompts) < 1 or len(prompts) != len(ids) or len(set(ids)) != len(ids) or min(ids) < 0:
        raise ValueError("one distinct sequence id per prompt, at least one prompt")
    if sum(len(t) for t in prompts) > int(np.count_nonzero(u.cell_seq == -1)):
        raise ValueError("context overflow")
    return _run(m, [_UnifiedSeq(u, s) for s in ids], list(prompts), prune, n_ubatch, None, unified=u)
