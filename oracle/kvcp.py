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


def payload_bytes(n_layers: int, n_pos: int, kv_dim: int) -> int:
    return 2 * n_layers * n_pos * kv_dim * 2


def dump(K: np.ndarray, V: np.ndarray, n_pos: int) -> bytes:
    """K, V: fp16 [n_layers][>= n_pos][kv_dim]."""
    nl, _, kvd = K.shape
    hdr = b"KVCP" + struct.pack("<3i", n_pos, nl, kvd)
    return (hdr + np.ascontiguousarray(K[:, :n_pos]).astype("<f2").tobytes()
            + np.ascontiguousarray(V[:, :n_pos]).astype("<f2").tobytes())


class SnapshotError(ValueError):
    pass


def load(data: bytes, n_layers: int, kv_dim: int, n_pos: int, n_ctx: int):
    """Validate a snapshot and return (K, V) of its first n_pos positions."""
    if len(data) < HEADER or data[:4] != b"KVCP":
        raise SnapshotError("bad magic")
    fpos, fl, fkvd = struct.unpack_from("<3i", data, 4)
    if fl != n_layers or fkvd != kv_dim:
        raise SnapshotError("model mismatch")
    if fpos < 0 or len(data) != HEADER + payload_bytes(fl, fpos, fkvd):
        raise SnapshotError("bad size")
    if n_pos < 0 or n_pos > fpos or n_pos > n_ctx:
        raise SnapshotError("position count out of range")
    body = np.frombuffer(data, dtype="<f2", offset=HEADER)
    K = body[:fl * fpos * fkvd].reshape(fl, fpos, fkvd)[:, :n_pos]
    V = body[fl * fpos * fkvd:].reshape(fl, fpos, fkvd)[:, :n_pos]
    return K.astype(np.float16), V.astype(np.float16)
