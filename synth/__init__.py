"""Seeded synthetic inputs: Q4_0 model containers and prompts.

Both the CPU oracle and the HIP engine consume what this module writes, so
it holds no arithmetic of the forward pass: it only draws random numbers and
lays bytes out in the model-container format described below.  The pages
measure on Google's QAT Q4_0 Gemma 4 E2B/E4B checkpoints (trained weights,
not available); seeded random weights of the same shapes stand in for them.

Random recipe (per tensor, independent streams so one tensor can be drawn
without the rest of the model):
  * Q4_0 blocks: fp16 scale d = fp16(U(0.01, 0.05)) drawn in fp32 and rounded
    to fp16 (the stored fp16 is authoritative); the 16 code bytes are uniform
    0..255, so each 4-bit code is uniform 0..15.
  * fp32 norm gains: U(0.8, 1.2).
  * per-layer embedding scales s_il: U(0.5, 1.5), fp32.
  * prompts: uniform int32 ids in [0, n_vocab), no BOS.

Container format "PPXM" v1 (little-endian):
  0    char[4]  magic "PPXM"
  4    u32      version (1)
  8    i32 x12  n_layer, n_layer_kv_from_start, d_model, n_head, n_kv_head,
                head_dim, n_ff, n_vocab, ple_dim, act (0 GeGLU, 1 SwiGLU),
                tied_output (1: head reuses tok_embd), n_tensors
  56   f32 x3   rms_eps, rope_base, embd_scale
  68   zero padding up to 128
  128  i32[n_layer]  kv source layer of each layer (itself when it owns KV)
  ...  f32[n_layer]  per-layer embedding scale s_il (0 when ple_dim == 0)
  T    tensor table at T = align(128 + 8*n_layer, 64), n_tensors entries of
       96 bytes: char name[64] (NUL padded), u32 type (0 F32, 1 Q4_0),
       u32 0, u64 rows, u64 cols, u64 offset (from file start)
  Optional tensor of a next-n head (configs with `nextn`): "nextn_norm"
       (F32 [1][d_model]); the head shares the output matrix.
  data each tensor at a 256-byte aligned offset.  Q4_0 [rows x cols] is
       rows * cols/32 blocks of 18 bytes: fp16 d, then 16 code bytes; code j
       of a block is the low nibble of byte j (j < 16) or the high nibble of
       byte j-16 (j >= 16); the weight is d * (code - 8).
"""
from __future__ import annotations

import math
import struct
import zlib
from dataclasses import dataclass, field, replace

import numpy as np

MAGIC = b"PPXM"
VERSION = 1
HEADER_BYTES = 128
ENTRY_BYTES = 96
NAME_BYTES = 64
T_F32 = 0
T_Q4_0 = 1
QK = 32
Q4_0_BLOCK_BYTES = 18


@dataclass(frozen=True)
class Config:
    name: str
    index: int
    n_layer: int
    n_layer_kv_from_start: int
    d_model: int
    n_head: int
    n_kv_head: int
    head_dim: int
    n_ff: int
    n_vocab: int
    ple_dim: int
    act: str  # "geglu" | "swiglu"
    tied: bool
    n_ubatch: int
    seed: int
    rms_eps: float = 1e-6
    rope_base: float = 10000.0
    # kv source layer of each shared layer; None -> alternating pair below Ls
    donors: tuple | None = None
    prompt_lens: tuple = field(default=())
    # a next-n head: its norm gain is in the container
    nextn: bool = False

    @property
    def embd_scale(self) -> float:
        # Gemma-style models scale token embeddings by sqrt(d_model); the
        # Llama-style model does not.
        return float(np.float32(math.sqrt(self.d_model))) if self.act == "geglu" else 1.0

    def donor_map(self) -> list[int]:
        ls, nl = self.n_layer_kv_from_start, self.n_layer
        if self.donors is not None:
            return list(self.donors)
        out = []
        for il in range(nl):
            if il < ls:
                out.append(il)
            else:
                out.append(ls - 2 + ((il - ls) % 2))
        return out

    @property
    def q_dim(self) -> int:
        return self.n_head * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_head * self.head_dim


CONFIGS: dict[str, Config] = {}


def _add(c: Config):
    CONFIGS[c.name] = c


_add(Config("tiny", 1, 4, 2, 256, 4, 1, 64, 1024, 2048, 0, "geglu", True, 64, 1001,
            prompt_lens=(64,), nextn=True))
_add(Config("tinyllama", 2, 22, 22, 2048, 32, 4, 64, 5632, 32000, 0, "swiglu", False, 512, 1002,
            prompt_lens=(512,)))
_add(Config("e2b", 3, 35, 15, 1536, 8, 1, 256, 6144, 262144, 256, "geglu", True, 512, 1003,
            prompt_lens=(512, 2048, 8192), nextn=True))
_add(Config("e4b", 4, 42, 24, 2560, 8, 2, 256, 10240, 262144, 256, "geglu", True, 512, 1004,
            prompt_lens=(512, 2048, 8192)))
# long-context variant: the same model as "e2b" (same seed), ubatch 1024
_add(replace(CONFIGS["e2b"], name="e2b_long", index=5, n_ubatch=1024, prompt_lens=(16384, 32768)))
# control: every layer writes KV, so pruning cannot apply
_add(replace(CONFIGS["e2b"], name="e2b_ctrl", index=6, n_layer_kv_from_start=35, seed=1006,
             n_ubatch=1024, prompt_lens=(8192,)))


def _tensor_rng(seed: int, name: str) -> np.random.Generator:
    return np.random.default_rng([seed, zlib.crc32(name.encode())])


def tensor_list(cfg: Config) -> list[tuple[str, int, int, int]]:
    """(name, type, rows, cols) in container order."""
    d, L, E = cfg.d_model, cfg.n_layer, cfg.ple_dim
    out = [("tok_embd", T_Q4_0, cfg.n_vocab, d)]
    if not cfg.tied:
        out.append(("output", T_Q4_0, cfg.n_vocab, d))
    out.append(("output_norm", T_F32, 1, d))
    if E:
        out.append(("ple_table", T_Q4_0, cfg.n_vocab, L * E))
    for il in range(L):
        p = f"blk.{il}."
        out.append((p + "attn_norm", T_F32, 1, d))
        out.append((p + "wq", T_Q4_0, cfg.q_dim, d))
        if il < cfg.n_layer_kv_from_start:
            out.append((p + "wk", T_Q4_0, cfg.kv_dim, d))
            out.append((p + "wv", T_Q4_0, cfg.kv_dim, d))
        out.append((p + "wo", T_Q4_0, d, cfg.q_dim))
        out.append((p + "ffn_norm", T_F32, 1, d))
        out.append((p + "ffn_gate", T_Q4_0, cfg.n_ff, d))
        out.append((p + "ffn_up", T_Q4_0, cfg.n_ff, d))
        out.append((p + "ffn_down", T_Q4_0, d, cfg.n_ff))
        if E:
            out.append((p + "ple_norm", T_F32, 1, d))
            out.append((p + "ple_gate", T_Q4_0, E, d))
            out.append((p + "ple_up", T_Q4_0, d, E))
    if cfg.nextn:
        out.append(("nextn_norm", T_F32, 1, d))
    return out


def tensor_nbytes(ttype: int, rows: int, cols: int) -> int:
    if ttype == T_F32:
        return rows * cols * 4
    assert cols % QK == 0
    return rows * (cols // QK) * Q4_0_BLOCK_BYTES


def fill_q4_0(out: np.ndarray, rows: int, cols: int, rng: np.random.Generator) -> None:
    """Write rows*cols/32 random Q4_0 blocks into the uint8 view `out`."""
    nb = rows * (cols // QK)
    blocks = out.reshape(nb, Q4_0_BLOCK_BYTES)
    # draw in bounded chunks to keep temporaries small for the big tables
    chunk = 1 << 22
    for s in range(0, nb, chunk):
        e = min(nb, s + chunk)
        sc = (rng.random(e - s, dtype=np.float32) * np.float32(0.04) + np.float32(0.01)).astype(np.float16)
        blocks[s:e, 0:2] = sc.view(np.uint8).reshape(e - s, 2)
        blocks[s:e, 2:] = rng.integers(0, 256, size=(e - s, 16), dtype=np.uint8)


def random_q4_0(rows: int, cols: int, seed: int) -> np.ndarray:
    """A standalone random Q4_0 matrix as uint8 [rows, cols/32*18]."""
    buf = np.empty(tensor_nbytes(T_Q4_0, rows, cols), dtype=np.uint8)
    fill_q4_0(buf, rows, cols, np.random.default_rng(seed))
    return buf.reshape(rows, -1)


def random_f32(n: int, seed: int, lo=-1.0, hi=1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return (rng.random(n, dtype=np.float32) * np.float32(hi - lo) + np.float32(lo)).astype(np.float32)


def _align(x: int, a: int) -> int:
    return (x + a - 1) // a * a


def build_model(cfg: Config | str) -> np.ndarray:
    """The whole container as a uint8 array."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    tl = tensor_list(cfg)
    L = cfg.n_layer
    table_off = _align(HEADER_BYTES + 8 * L, 64)
    off = _align(table_off + ENTRY_BYTES * len(tl), 256)
    offsets = []
    for (_, tt, r, c) in tl:
        offsets.append(off)
        off = _align(off + tensor_nbytes(tt, r, c), 256)
    total = off
    buf = np.zeros(total, dtype=np.uint8)

    hdr = struct.pack("<4sI12i3f", MAGIC, VERSION, L, cfg.n_layer_kv_from_start, cfg.d_model,
                      cfg.n_head, cfg.n_kv_head, cfg.head_dim, cfg.n_ff, cfg.n_vocab, cfg.ple_dim,
                      0 if cfg.act == "geglu" else 1, 1 if cfg.tied else 0, len(tl),
                      cfg.rms_eps, cfg.rope_base, cfg.embd_scale)
    buf[:len(hdr)] = np.frombuffer(hdr, dtype=np.uint8)
    donors = np.asarray(cfg.donor_map(), dtype="<i4")
    buf[HEADER_BYTES:HEADER_BYTES + 4 * L] = donors.view(np.uint8)
    if cfg.ple_dim:
        s = random_f32(L, cfg.seed * 7 + 3, 0.5, 1.5)
    else:
        s = np.zeros(L, np.float32)
    buf[HEADER_BYTES + 4 * L:HEADER_BYTES + 8 * L] = s.astype("<f4").view(np.uint8)

    for i, ((name, tt, r, c), o) in enumerate(zip(tl, offsets)):
        nb = name.encode()
        assert len(nb) < NAME_BYTES
        ent = nb.ljust(NAME_BYTES, b"\0") + struct.pack("<IIQQQ", tt, 0, r, c, o)
        eo = table_off + i * ENTRY_BYTES
        buf[eo:eo + ENTRY_BYTES] = np.frombuffer(ent, dtype=np.uint8)
        n = tensor_nbytes(tt, r, c)
        rng = _tensor_rng(cfg.seed, name)
        if tt == T_Q4_0:
            fill_q4_0(buf[o:o + n], r, c, rng)
        else:
            g = (rng.random(r * c, dtype=np.float32) * np.float32(0.4) + np.float32(0.8)).astype("<f4")
            buf[o:o + n] = g.view(np.uint8)
    return buf


def prompt(cfg: Config | str, n: int, seed: int | None = None) -> np.ndarray:
    """n uniform-random token ids (int32) for config `cfg`."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if seed is None:
        seed = 2000 + 100 * cfg.index
    rng = np.random.default_rng([seed, n])
    return rng.integers(0, cfg.n_vocab, size=n, dtype=np.int64).astype(np.int32)


def model_file(cfg: Config | str, directory: str) -> str:
    """Write (once) the container of `cfg` under `directory`; return its path."""
    import os
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    os.makedirs(directory, exist_ok=True)
    path = os.path.join(directory, f"{cfg.name}_s{cfg.seed}_v{VERSION}.ppxm")
    if not os.path.exists(path):
        buf = build_model(cfg)
        tmp = path + f".tmp{os.getpid()}"
        buf.tofile(tmp)
        os.replace(tmp, path)
    return path


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("config", choices=sorted(CONFIGS))
    ap.add_argument("--dir", default="/tmp/ppx_models")
    a = ap.parse_args()
    print(model_file(a.config, a.dir))
