"""Oracle: KVCP snapshot bytes (test infrastructure).

The PicoLM KV-cache page ("the cache file" section) fixes the content: the
magic KVCP, then the number of cached positions, the layer count and the KV
dimension, then the fp16 K vectors of the first N positions, then the fp16
V vectors.  Reading of the field widths and order: 4 ASCII bytes, three
little-endian int32 (n_pos, n_layers, kv_dim), K as [layer][pos][kv_dim],
V likewise; header 16 bytes.  Only layers that own a cache are stored.  The
load check (magic, layer count, KV dim) follows that page's section on
loading, which falls back to a full prefill on any mismatch.
"""
from __future__ import annotations

import struct

import numpy as np

HEADER = 16

# Token section (an extension outside the page's layout): the page's
# invalidation rules leave checking that a new prompt starts with the cached
# prefix to the caller.  A snapshot may therefore end with "KVTK", an int32
# count equal to the cached positions, and that many int32 token ids; the KVCP
# body before it is unchanged.
TOKEN_MAGIC = b"KVTK"


def payload_bytes(n_layers: int, n_pos: int, kv_dim: int) -> int:
    return 2 * n_layers * n_pos * kv_dim * 2


def dump(K: np.ndarray, V: np.ndarray, n_pos: int) -> bytes:
    """K, V: fp16 [n_layers][>= n_pos][kv_dim]."""
    nl, _, kvd = K.shape
    hdr = b"KVCP" + struct.pack("<3i", n_pos, nl, kvd)
    return (hdr + np.ascontiguousarray(K[:, :n_pos]).astype("<f2").tobytes()
            + np.ascontiguousarray(V[:, :n_pos]).astype("<f2").tobytes())


def dump_tokens(K: np.ndarray, V: np.ndarray, n_pos: int, tokens) -> bytes:
    """The KVCP body of dump() followed by the token section of the first n_pos ids."""
    ids = [int(t) for t in list(tokens)[:n_pos]]
    if len(ids) != n_pos:
        raise ValueError("one token id per cached position")
    return dump(K, V, n_pos) + TOKEN_MAGIC + struct.pack("<i", n_pos) + struct.pack(f"<{n_pos}i", *ids)


class SnapshotError(ValueError):
    pass


def load(data: bytes, n_layers: int, kv_dim: int, n_pos: int, n_ctx: int):
    """Validate a snapshot and return (K, V) of its first n_pos positions."""
    if len(data) < HEADER or data[:4] != b"KVCP":
        raise SnapshotError("bad magic")
    fpos, fl, fkvd = struct.unpack_from("<3i", data, 4)
    if fl != n_layers or fkvd != kv_dim:
        raise SnapshotError("model mismatch")
    if fpos < 0 or len(data) not in (HEADER + payload_bytes(fl, fpos, fkvd), HEADER + payload_bytes(fl, fpos, fkvd) + 8 + 4 * fpos):
        raise SnapshotError("bad size")
    if len(data) != HEADER + payload_bytes(fl, fpos, fkvd) and stored_tokens(data) is None:
        raise SnapshotError("bad size")
    if n_pos < 0 or n_pos > fpos or n_pos > n_ctx:
        raise SnapshotError("position count out of range")
    body = np.frombuffer(data, dtype="<f2", offset=HEADER, count=payload_bytes(fl, fpos, fkvd) // 2)
    K = body[:fl * fpos * fkvd].reshape(fl, fpos, fkvd)[:, :n_pos]
    V = body[fl * fpos * fkvd:].reshape(fl, fpos, fkvd)[:, :n_pos]
    return K.astype(np.float16), V.astype(np.float16)


def stored_tokens(data: bytes):
    """The token ids of a snapshot's token section, or None if it has none."""
    if len(data) < HEADER or data[:4] != b"KVCP":
        return None
    fpos, fl, fkvd = struct.unpack_from("<3i", data, 4)
    if fpos < 0:
        return None
    body = HEADER + payload_bytes(fl, fpos, fkvd)
    if len(data) != body + 8 + 4 * fpos or data[body:body + 4] != TOKEN_MAGIC:
        return None
    (cnt,) = struct.unpack_from("<i", data, body + 4)
    if cnt != fpos:
        return None
    return list(struct.unpack_from(f"<{fpos}i", data, body + 8))


def reusable_prefix(stored, prompt, n_ctx: int) -> int:
    """Longest common prefix of the stored ids and the prompt, leaving at least
    one prompt token to run (it gives the logits) and within the context."""
    cap = min(len(stored), len(prompt) - 1, n_ctx)
    n = 0
    while n < cap and int(stored[n]) == int(prompt[n]):
        n += 1
    return max(n, 0)


def load_prefix(data: bytes, prompt, n_layers: int, kv_dim: int, n_ctx: int):
    """(L, K, V): the reusable prefix length and the first L positions' K, V."""
    ids = stored_tokens(data)
    if ids is None:
        raise SnapshotError("no token section")
    L = reusable_prefix(ids, prompt, n_ctx)
    K, V = load(data, n_layers, kv_dim, L, n_ctx)
    return L, K, V
