"""Oracle: model-container parser and Q4_0 dequantisation (test infrastructure).

Q4_0 is named by the llama.cpp Gemma 4 prefill page (section 2: the
official QAT Q4_0 checkpoints); its bit layout is not on the pages.  Reading
used here: a block holds 32 weights as an fp16 scale d and 16 bytes of 4-bit
codes, code j is the low nibble of byte j for j < 16 and the high nibble of
byte j-16 for j >= 16, and weight j = d * (code_j - 8).  In fp64 this product
is exact, so the oracle's dequantisation is the closed form itself.
"""
from __future__ import annotations

import struct
from dataclasses import dataclass

import numpy as np

_T_F32, _T_Q4_0 = 0, 1


@dataclass
class Tensor:
    name: str
    ttype: int
    rows: int
    cols: int
    raw: np.ndarray  # uint8 view of the tensor's bytes


@dataclass
class OracleModel:
    n_layer: int
    n_layer_kv_from_start: int
    d_model: int
    n_head: int
    n_kv_head: int
    head_dim: int
    n_ff: int
    n_vocab: int
    ple_dim: int
    act: int  # 0 GeGLU, 1 SwiGLU
    tied: bool
    rms_eps: float
    rope_base: float
    embd_scale: float
    kv_src: list
    ple_scale: np.ndarray
    tensors: dict

    @property
    def kv_dim(self) -> int:
        return self.n_kv_head * self.head_dim

    def f32(self, name: str) -> np.ndarray:
        t = self.tensors[name]
        assert t.ttype == _T_F32
        return t.raw.view("<f4").astype(np.float64)

    def q4(self, name: str, rows=None) -> np.ndarray:
        """Dequantised fp64 [rows, cols] (all rows, or the selected ones)."""
        t = self.tensors[name]
        assert t.ttype == _T_Q4_0
        raw = t.raw.reshape(t.rows, t.cols // 32, 18)
        if rows is not None:
            raw = raw[np.asarray(rows)]
        return deq_q4_0(raw).reshape(raw.shape[0], t.cols)


def parse_model(buf) -> OracleModel:
    b = np.frombuffer(buf, dtype=np.uint8) if not isinstance(buf, np.ndarray) else buf
    if bytes(b[:4]) != b"PPXM":
        raise ValueError("not a PPXM container")
    (ver,) = struct.unpack_from("<I", b, 4)
    if ver != 1:
        raise ValueError(f"unsupported container version {ver}")
    h = struct.unpack_from("<12i", b, 8)
    eps, base, escale = struct.unpack_from("<3f", b, 56)
    L = h[0]
    kv_src = list(struct.unpack_from(f"<{L}i", b, 128))
    ple_scale = np.array(struct.unpack_from(f"<{L}f", b, 128 + 4 * L), dtype=np.float64)
    n_t = h[11]
    toff = (128 + 8 * L + 63) // 64 * 64
    tensors = {}
    for i in range(n_t):
        e = toff + 96 * i
        name = bytes(b[e:e + 64]).rstrip(b"\0").decode()
        tt, _, rows, cols, off = struct.unpack_from("<IIQQQ", b, e + 64)
        n = rows * cols * 4 if tt == _T_F32 else rows * (cols // 32) * 18
        tensors[name] = Tensor(name, tt, rows, cols, b[off:off + n])
    return OracleModel(n_layer=L, n_layer_kv_from_start=h[1], d_model=h[2], n_head=h[3],
                       n_kv_head=h[4], head_dim=h[5], n_ff=h[6], n_vocab=h[7], ple_dim=h[8],
                       act=h[9], tied=bool(h[10]), rms_eps=float(eps), rope_base=float(base),
                       embd_scale=float(escale), kv_src=kv_src, ple_scale=ple_scale,
                       tensors=tensors)


def deq_q4_0(blocks: np.ndarray) -> np.ndarray:
    """uint8 [..., 18] Q4_0 blocks -> fp64 [..., 32]: w_j = d * (code_j - 8).

    The product is formed in fp32, where it is exact (an fp16 significand of
    11 bits times an integer of magnitude <= 8 needs at most 15 bits), and
    then widened to fp64.
    """
    blocks = np.ascontiguousarray(blocks)
    d = blocks[..., 0:2].copy().view("<f2")[..., 0].astype(np.float32)
    qs = blocks[..., 2:18]
    codes = np.empty(blocks.shape[:-1] + (32,), dtype=np.int8)
    np.bitwise_and(qs, 0x0F, out=codes[..., :16], casting="unsafe")
    np.right_shift(qs, 4, out=codes[..., 16:], casting="unsafe")
    codes -= 8
    return (d[..., None] * codes).astype(np.float64)
