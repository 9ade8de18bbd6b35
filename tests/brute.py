"""Brute-force forward pass in scalar pure Python, for micro configs only.

An independent second implementation of the same model reading as the
oracle (pre-norm decoder, KV-shared layers reading a source layer's fp16
cache, last-row logits), written with explicit loops and its own container
parser.  It imports nothing from oracle/ or from the engine; tests compare
the oracle against it on shapes small enough for scalar Python.
"""
from __future__ import annotations

import math
import struct

import numpy as np


def _f16_round(v: float) -> float:
    # struct's 'e' format packs with IEEE round-to-nearest-even
    return struct.unpack("<e", struct.pack("<e", v))[0]


class BruteModel:
    def __init__(self, data: bytes):
        assert data[:4] == b"PPXM"
        h = struct.unpack_from("<12i", data, 8)
        (self.L, self.Ls, self.d, self.H, self.KVH, self.hd, self.F, self.V, self.E,
         self.act, self.tied, nt) = h
        self.eps, self.base, self.escale = struct.unpack_from("<3f", data, 56)
        self.src = list(struct.unpack_from(f"<{self.L}i", data, 128))
        self.s = list(struct.unpack_from(f"<{self.L}f", data, 128 + 4 * self.L))
        toff = (128 + 8 * self.L + 63) // 64 * 64
        self.t = {}
        for i in range(nt):
            e = toff + 96 * i
            name = data[e:e + 64].rstrip(b"\0").decode()
            tt, _, rows, cols, off = struct.unpack_from("<IIQQQ", data, e + 64)
            if tt == 0:
                self.t[name] = [list(struct.unpack_from(f"<{cols}f", data, off))]
            else:
                mat = []
                for r in range(rows):
                    row = []
                    for b in range(cols // 32):
                        bo = off + (r * (cols // 32) + b) * 18
                        (dd,) = struct.unpack_from("<e", data, bo)
                        qs = data[bo + 2:bo + 18]
                        codes = [qs[j] & 15 for j in range(16)] + [qs[j] >> 4 for j in range(16)]
                        row.extend(dd * (c - 8) for c in codes)
                    mat.append(row)
                self.t[name] = mat


def _mv(W, x):
    return [sum(w * v for w, v in zip(row, x)) for row in W]


def _rms(x, g, eps):
    ms = sum(v * v for v in x) / len(x)
    r = 1.0 / math.sqrt(ms + eps)
    return [v * r * gg for v, gg in zip(x, g)]


def _rope(v, p, base):
    hd = len(v)
    half = hd // 2
    out = list(v)
    for i in range(half):
        th = p * base ** (-2.0 * i / hd)
        c, s = math.cos(th), math.sin(th)
        out[i] = v[i] * c - v[i + half] * s
        out[i + half] = v[i] * s + v[i + half] * c
    return out


def _gelu(z):
    return 0.5 * z * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z * z * z)))


def _silu(z):
    return z / (1.0 + math.exp(-z))


def brute_prefill(M: BruteModel, tokens, n_ctx: int, hidden: dict | None = None):
    """Returns (logits list, K, V) with K[il][pos] = list of kv_dim floats.

    hidden, if given, receives "inp": the rows entering each layer il (index
    L: the final rows), and "embd": every final row after the output norm."""
    L, Ls, H, KVH, hd = M.L, M.Ls, M.H, M.KVH, M.hd
    K = [[None] * n_ctx for _ in range(Ls)]
    V = [[None] * n_ctx for _ in range(Ls)]
    xs = []
    for t, tok in enumerate(tokens):
        xs.append([M.escale * w for w in M.t["tok_embd"][tok]])
    inp = []
    for il in range(L):
        inp.append([list(x) for x in xs])
        p = f"blk.{il}."
        g = M.t
        own = il < Ls
        src = il if own else M.src[il]
        # K/V of this layer for every row first (rows attend to earlier rows)
        qs = []
        for t, x in enumerate(xs):
            a = _rms(x, g[p + "attn_norm"][0], M.eps)
            q = _mv(g[p + "wq"], a)
            qs.append([_rope(q[h * hd:(h + 1) * hd], t, M.base) for h in range(H)])
            if own:
                k = _mv(g[p + "wk"], a)
                v = _mv(g[p + "wv"], a)
                kr = []
                for hh in range(KVH):
                    kr.extend(_rope(k[hh * hd:(hh + 1) * hd], t, M.base))
                K[il][t] = [_f16_round(z) for z in kr]
                V[il][t] = [_f16_round(z) for z in v]
        new = []
        for t, x in enumerate(xs):
            o = []
            for h in range(H):
                gh = h // (H // KVH)
                sc = []
                for j in range(t + 1):
                    kj = K[src][j][gh * hd:(gh + 1) * hd]
                    sc.append(sum(a * b for a, b in zip(qs[t][h], kj)) / math.sqrt(hd))
                mx = max(sc)
                ws = [math.exp(s - mx) for s in sc]
                tot = sum(ws)
                for i in range(hd):
                    o.append(sum(ws[j] / tot * V[src][j][gh * hd + i] for j in range(t + 1)))
            x = [a + b for a, b in zip(x, _mv(g[p + "wo"], o))]
            b_ = _rms(x, g[p + "ffn_norm"][0], M.eps)
            gt = _mv(g[p + "ffn_gate"], b_)
            up = _mv(g[p + "ffn_up"], b_)
            act = _gelu if M.act == 0 else _silu
            hv = [act(a) * u for a, u in zip(gt, up)]
            x = [a + b for a, b in zip(x, _mv(g[p + "ffn_down"], hv))]
            if M.E:
                E = M.E
                c = _rms(x, g[p + "ple_norm"][0], M.eps)
                P = [M.s[il] * w for w in g["ple_table"][tokens[t]][il * E:(il + 1) * E]]
                gg = [_gelu(z) * pp for z, pp in zip(_mv(g[p + "ple_gate"], c), P)]
                x = [a + b for a, b in zip(x, _mv(g[p + "ple_up"], gg))]
            new.append(x)
        xs = new
    if hidden is not None:
        hidden["inp"] = inp + [[list(x) for x in xs]]
        hidden["embd"] = [_rms(x, M.t["output_norm"][0], M.eps) for x in xs]
    hn = _rms(xs[-1], M.t["output_norm"][0], M.eps)
    Wout = M.t["tok_embd"] if M.tied else M.t["output"]
    logits = _mv(Wout, hn)
    return logits, K, V


def brute_nextn(M: BruteModel, tokens, n_ctx: int):
    """Logits of the next-n head: the output matrix applied to the row before
    the last one's final state plus the last token's embedding, normed with
    the head's own gain."""
    hb = {}
    brute_prefill(M, tokens, n_ctx, hidden=hb)
    x = hb["inp"][M.L][len(tokens) - 2]
    z = [a + M.escale * w for a, w in zip(x, M.t["tok_embd"][tokens[-1]])]
    hn = _rms(z, M.t["nextn_norm"][0], M.eps)
    return _mv(M.t["tok_embd"] if M.tied else M.t["output"], hn)


def as_arrays(K, n_pos: int) -> np.ndarray:
    return np.array([[K[il][p] for p in range(n_pos)] for il in range(len(K))], dtype=np.float64)
