"""Python binding of libppx (the MI355X pruned prompt-prefill engine).

Argument marshalling only: every step of the prefill runs in the library's
HIP kernels.  torch provides device memory and the current stream.  The
names follow the C ABI in include/ppx.h.  If libppx.so has not been built,
every entry point raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int, c_size_t, c_uint8, c_void_p

import numpy as np

__all__ = ["PPXError", "lib", "Model", "KVCache", "UnifiedCache", "prune_predicate", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libppx.so")

PPX_OK = 0
STATUS = {0: "PPX_OK", -1: "PPX_E_INVAL", -2: "PPX_E_TOKEN", -3: "PPX_E_CTX", -4: "PPX_E_IO",
          -5: "PPX_E_FORMAT", -6: "PPX_E_MISMATCH", -7: "PPX_E_UNSUPPORTED", -8: "PPX_E_HIP",
          -9: "PPX_E_NOMEM", -10: "PPX_E_EMPTY"}
PRUNE = {"auto": -1, "off": 0, "on": 1}
PRECISION = {"fast": 0, "exact": 1}
PPX_MAX_UBATCH = 4096


class PPXError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        self.name = STATUS.get(status, str(status))
        msg = lib().ppx_status_str(status).decode() if _LIB is not None else self.name
        super().__init__(f"{what}: {self.name} ({msg})" if what else f"{self.name} ({msg})")


class ModelInfo(ctypes.Structure):
    _fields_ = [(n, c_int) for n in ("n_layer", "n_layer_kv_from_start", "d_model", "n_head", "n_kv_head",
                                     "head_dim", "n_ff", "n_vocab", "ple_dim", "kv_dim", "act",
                                     "has_nextn")]


class Timing(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double * 4), ("launches", c_int * 4), ("gemm_flop", ctypes.c_double),
                ("attn_flop", ctypes.c_double), ("row_bytes", ctypes.c_double), ("glu_ms", ctypes.c_double),
                ("glu_launches", c_int), ("glu_flop", ctypes.c_double)]

    def as_dict(self):
        names = ("gemm", "attn", "row", "other")
        return {"ms": dict(zip(names, list(self.ms))), "launches": dict(zip(names, list(self.launches))),
                "gemm_flop": self.gemm_flop, "attn_flop": self.attn_flop, "row_bytes": self.row_bytes,
                "glu_ms": self.glu_ms, "glu_launches": self.glu_launches, "glu_flop": self.glu_flop}


class PrefillParams(ctypes.Structure):
    _fields_ = [("n_ubatch", c_int), ("prune", c_int), ("embeddings", c_int), ("n_seq_max", c_int),
                ("debug_hidden", c_void_p), ("timing", POINTER(Timing)), ("debug_rows", c_void_p),
                ("embeddings_layer_inp", c_void_p), ("layer_inp_out", c_void_p), ("embd_out", c_void_p),
                ("precision", c_int), ("nextn_logits", c_void_p)]


class Seq(ctypes.Structure):
    _fields_ = [("kv", c_void_p), ("tokens_host", c_void_p), ("n_tokens", c_int)]


class USeq(ctypes.Structure):
    _fields_ = [("seq_id", c_int), ("tokens_host", c_void_p), ("n_tokens", c_int)]


# (name, restype, argtypes) of every symbol declared in include/ppx.h
SIGNATURES = [
    ("ppx_model_load", c_int, [c_void_p, c_size_t, c_void_p, POINTER(c_void_p)]),
    ("ppx_model_load_file", c_int, [c_char_p, c_void_p, POINTER(c_void_p)]),
    ("ppx_model_weight_bytes", c_size_t, [c_void_p, c_size_t]),
    ("ppx_model_load_into", c_int, [c_void_p, c_size_t, c_void_p, c_size_t, c_void_p, POINTER(c_void_p)]),
    ("ppx_model_free", None, [c_void_p]),
    ("ppx_model_get_info", c_int, [c_void_p, POINTER(ModelInfo)]),
    ("ppx_model_device_bytes", c_size_t, [c_void_p]),
    ("ppx_kv_bytes", c_size_t, [c_void_p, c_int]),
    ("ppx_kv_init", c_int, [c_void_p, c_void_p, c_size_t, c_int, POINTER(c_void_p)]),
    ("ppx_kv_free", None, [c_void_p]),
    ("ppx_kv_n_pos", c_int, [c_void_p]),
    ("ppx_kv_n_ctx", c_int, [c_void_p]),
    ("ppx_kv_clear", c_int, [c_void_p]),
    ("ppx_kv_save", c_int, [c_void_p, c_char_p, c_int, c_void_p]),
    ("ppx_kv_load", c_int, [c_void_p, c_char_p, c_int, c_void_p]),
    ("ppx_kv_save_tokens", c_int, [c_void_p, c_char_p, c_int, c_void_p, c_void_p]),
    ("ppx_kv_load_prefix", c_int, [c_void_p, c_char_p, c_void_p, c_int, c_void_p, c_void_p]),
    ("ppx_kvfile_validate", c_int, [c_char_p, c_int, c_int, c_int, c_int, POINTER(c_int)]),
    ("ppx_workspace_bytes", c_size_t, [c_void_p, c_int, c_int]),
    ("ppx_workspace_bytes_multi", c_size_t, [c_void_p, c_int, c_int, ctypes.c_long, c_int]),
    ("ppx_prefill_multi", c_int, [c_void_p, POINTER(Seq), c_int, POINTER(PrefillParams), c_void_p, c_size_t,
                                  c_void_p, c_void_p]),
    ("ppx_kvu_bytes", c_size_t, [c_void_p, c_int]),
    ("ppx_kvu_init", c_int, [c_void_p, c_void_p, c_size_t, c_int, c_int, POINTER(c_void_p)]),
    ("ppx_kvu_free", None, [c_void_p]),
    ("ppx_kvu_n_pos", c_int, [c_void_p, c_int]),
    ("ppx_kvu_free_cells", c_int, [c_void_p]),
    ("ppx_kvu_seq_rm", c_int, [c_void_p, c_int]),
    ("ppx_kvu_cells", c_int, [c_void_p, c_int, c_void_p, c_int]),
    ("ppx_workspace_bytes_unified", c_size_t, [c_void_p, c_int, c_int, ctypes.c_long, c_int]),
    ("ppx_prefill_unified", c_int, [c_void_p, c_void_p, POINTER(USeq), c_int, POINTER(PrefillParams), c_void_p,
                                    c_size_t, c_void_p, c_void_p]),
    ("ppx_decode", c_int, [c_void_p, c_void_p, c_int, c_void_p, c_size_t, c_void_p, c_void_p]),
    ("ppx_decode_static", c_int, [c_void_p, c_void_p, c_int, c_void_p, c_void_p]),
    ("ppx_decode_static_limit", c_size_t, []),
    ("ppx_prefill", c_int, [c_void_p, c_void_p, c_void_p, c_int, POINTER(PrefillParams), c_void_p, c_size_t,
                            c_void_p, c_void_p]),
    ("ppx_prune_predicate", c_int, [c_int, c_int, c_int, c_int, POINTER(c_uint8), c_int]),
    ("ppx_op_dequant", c_int, [c_void_p, c_char_p, c_void_p, c_void_p]),
    ("ppx_op_tile_f16", c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p]),
    ("ppx_op_stream_read", c_int, [c_void_p, c_size_t, c_void_p, c_int, c_void_p]),
    ("ppx_op_gemm_workspace_bytes", c_size_t, [c_void_p, c_char_p, c_int]),
    ("ppx_op_gemm", c_int, [c_void_p, c_char_p, c_void_p, c_int, c_void_p, c_void_p, c_size_t, c_void_p]),
    ("ppx_op_gemm_glu", c_int, [c_void_p, c_char_p, c_void_p, c_int, c_void_p, c_void_p, c_size_t, c_void_p]),
    ("ppx_op_gemm_exact", c_int, [c_void_p, c_char_p, c_void_p, c_void_p, c_int, c_void_p, c_void_p]),
    ("ppx_op_gemv", c_int, [c_void_p, c_char_p, c_void_p, c_void_p, c_void_p]),
    ("ppx_op_attention", c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_void_p, c_void_p,
                                 c_size_t, c_void_p]),
    ("ppx_op_attention_1row", c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_void_p, c_void_p,
                                      c_size_t, c_void_p]),
    ("ppx_status_str", c_char_p, [c_int]),
]

_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded libppx.so; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m prompt_prefill_cross_amd.build` (no CPU fallback exists)")
        # torch bundles its own HIP runtime under the same soname as the
        # system one libppx.so links.  Loading torch first makes the library
        # bind to that runtime, so the two share one device context; the
        # other order leaves torch on a runtime whose allocations fail.
        import torch  # noqa: F401
        h = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _LIB = h
    return _LIB


def _check(st: int, what: str):
    if st != PPX_OK:
        raise PPXError(st, what)


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return c_void_p(s.cuda_stream)


def _ptr(t) -> c_void_p:
    return c_void_p(t.data_ptr())


def stream_read(buf, n_workgroups: int = 2048, stream=None) -> int:
    """XOR of the 32-bit words of a device buffer (bytes a multiple of 1024),
    read through the GEMM producers' LDS DMA (ppx_op_stream_read)."""
    import torch
    out = torch.empty(n_workgroups, dtype=torch.int32, device=buf.device)
    _check(lib().ppx_op_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out), n_workgroups,
                                    _stream(stream)), "ppx_op_stream_read")
    x = 0
    for v in out.cpu().numpy().astype(np.uint32).tolist():
        x ^= v
    return x


def prune_predicate(n_layer, n_layer_kv_from_start, embeddings, n_seq_max, embeddings_layer_inp=None,
                    crop_before_nextn=True) -> bool:
    arr = None
    if embeddings_layer_inp is not None:
        a = np.ascontiguousarray(np.asarray(embeddings_layer_inp, dtype=np.uint8))
        if a.shape[0] < n_layer + 1:
            raise ValueError("embeddings_layer_inp needs n_layer + 1 flags")
        arr = a.ctypes.data_as(POINTER(c_uint8))
    return bool(lib().ppx_prune_predicate(n_layer, n_layer_kv_from_start, int(embeddings), n_seq_max, arr,
                                          int(crop_before_nextn)))


def kvfile_validate(path, n_layers: int, kv_dim: int, n_pos: int, n_ctx: int):
    """(status, file_n_pos) of the host-only KVCP check."""
    fp = c_int(-1)
    st = lib().ppx_kvfile_validate(os.fsencode(path), n_layers, kv_dim, n_pos, n_ctx, ctypes.byref(fp))
    return st, fp.value


class Model:
    """A loaded model: `Model(container)` with a numpy uint8 array / bytes, or a path."""

    def __init__(self, src, stream=None, torch_weights: bool = False):
        """torch_weights: place the repacked weights in a torch uint8 tensor
        (ppx_model_load_into) instead of library-allocated device memory."""
        self._h = c_void_p()
        self._weights = None
        L = lib()
        if isinstance(src, (str, os.PathLike)):
            if torch_weights:
                with open(src, "rb") as f:
                    src = f.read()
            else:
                st = L.ppx_model_load_file(os.fsencode(src), _stream(stream), ctypes.byref(self._h))
        if not isinstance(src, (str, os.PathLike)):
            buf = np.ascontiguousarray(np.frombuffer(src, dtype=np.uint8) if not isinstance(src, np.ndarray)
                                       else src.view(np.uint8).reshape(-1))
            if torch_weights:
                import torch
                need = L.ppx_model_weight_bytes(c_void_p(buf.ctypes.data), buf.nbytes)
                if need == 0:
                    raise PPXError(-5, "ppx_model_weight_bytes: invalid container")
                self._weights = torch.empty(need, dtype=torch.uint8, device="cuda")
                st = L.ppx_model_load_into(c_void_p(buf.ctypes.data), buf.nbytes, _ptr(self._weights), need,
                                           _stream(stream), ctypes.byref(self._h))
            else:
                st = L.ppx_model_load(c_void_p(buf.ctypes.data), buf.nbytes, _stream(stream), ctypes.byref(self._h))
        _check(st, "ppx_model_load")
        info = ModelInfo()
        _check(L.ppx_model_get_info(self._h, ctypes.byref(info)), "ppx_model_get_info")
        self.info = {n: getattr(info, n) for n, _ in ModelInfo._fields_}
        self._ws = None
        self._ws_key = None

    @property
    def handle(self):
        return self._h

    @property
    def device_bytes(self) -> int:
        return lib().ppx_model_device_bytes(self._h)

    def close(self):
        if self._h:
            lib().ppx_model_free(self._h)
            self._h = c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace(self, n_ubatch: int, n_ctx: int):
        import torch
        need = lib().ppx_workspace_bytes(self._h, n_ubatch, n_ctx)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        return self._ws

    def prefill(self, tokens, kv: "KVCache", n_ubatch: int = 512, prune: str = "auto", logits=None,
                debug_hidden=None, embeddings: int = 0, n_seq_max: int = 1, stream=None, timing=None,
                debug_rows=None, layer_flags=None, layer_inp_out=None, embd_out=None, precision: str = "fast",
                nextn_logits=None):
        """Run `tokens` (int32) from kv.n_pos; return fp32 logits [n_vocab] of the last token.

        layer_flags (n_layer + 1 truth values) / layer_inp_out and embeddings /
        embd_out are the extraction outputs of ppx_prefill_params;
        nextn_logits (fp32 [n_vocab] on the device) receives the next-n head's."""
        import torch
        toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
        if logits is None:
            logits = torch.empty(self.info["n_vocab"], dtype=torch.float32, device="cuda")
        ws = self.workspace(n_ubatch, kv.n_ctx) if n_ubatch >= 1 else torch.empty(256, dtype=torch.uint8,
                                                                                  device="cuda")
        flags = None
        if layer_flags is not None:
            flags = np.ascontiguousarray(np.asarray(layer_flags, dtype=np.uint8).reshape(-1))
            if flags.size != self.info["n_layer"] + 1:
                raise ValueError("layer_flags needs n_layer + 1 entries")
        p = PrefillParams(n_ubatch, PRUNE[prune] if isinstance(prune, str) else int(prune), embeddings,
                          n_seq_max, c_void_p(debug_hidden.data_ptr()) if debug_hidden is not None else None,
                          ctypes.pointer(timing) if timing is not None else None,
                          c_void_p(debug_rows.data_ptr()) if debug_rows is not None else None,
                          c_void_p(flags.ctypes.data) if flags is not None else None,
                          c_void_p(layer_inp_out.data_ptr()) if layer_inp_out is not None else None,
                          c_void_p(embd_out.data_ptr()) if embd_out is not None else None,
                          PRECISION[precision],
                          c_void_p(nextn_logits.data_ptr()) if nextn_logits is not None else None)
        st = lib().ppx_prefill(self._h, kv.handle, c_void_p(toks.ctypes.data), toks.shape[0], ctypes.byref(p),
                               _ptr(ws), ws.numel(), _ptr(logits), _stream(stream))
        _check(st, "ppx_prefill")
        return logits

    def extract(self, tokens, kv: "KVCache", layers=(), embeddings: bool = False, n_ubatch: int = 512,
                prune: str = "auto"):
        """Prefill with extraction: returns (logits, {il: fp32 [n][d] input of
        layer il for every row}, fp32 [n][d] output-normed final rows or None)."""
        import torch
        n = int(np.asarray(tokens).reshape(-1).shape[0])
        L, d = self.info["n_layer"], self.info["d_model"]
        want = sorted(set(int(il) for il in layers))
        flags = np.zeros(L + 1, np.uint8)
        flags[want] = 1
        inp = torch.empty((max(len(want), 1), n, d), dtype=torch.float32, device="cuda")
        emb = torch.empty((n, d), dtype=torch.float32, device="cuda") if embeddings else None
        lg = self.prefill(tokens, kv, n_ubatch=n_ubatch, prune=prune, embeddings=int(bool(embeddings)),
                          layer_flags=flags, layer_inp_out=inp if want else None, embd_out=emb)
        return lg, {il: inp[j] for j, il in enumerate(want)}, emb

    def prefill_multi(self, prompts, kvs, n_ubatch: int = 512, prune: str = "auto", logits=None,
                      n_seq_max: int | None = None, stream=None, timing=None, precision: str = "fast"):
        """Several prompts in one pass, prompt s from kvs[s].n_pos in its own
        cache; return fp32 logits [n_seq][n_vocab] of each prompt's last token."""
        import torch
        toks = [np.ascontiguousarray(np.asarray(t, dtype=np.int32).reshape(-1)) for t in prompts]
        k = len(toks)
        if k != len(kvs):
            raise ValueError("one cache per prompt")
        seqs = (Seq * max(k, 1))()
        for i, (t, kv) in enumerate(zip(toks, kvs)):
            seqs[i] = Seq(kv.handle, t.ctypes.data if t.size else None, int(t.shape[0]))
        if logits is None:
            logits = torch.empty((max(k, 1), self.info["n_vocab"]), dtype=torch.float32, device="cuda")
        total = max(1, sum(int(t.shape[0]) for t in toks))
        n_ctx = max([kv.n_ctx for kv in kvs] or [1])
        need = lib().ppx_workspace_bytes_multi(self._h, max(n_ubatch, 1), max(min(k, 64), 1), total, n_ctx)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        ws = self._ws
        p = PrefillParams(n_ubatch, PRUNE[prune] if isinstance(prune, str) else int(prune), 0,
                          k if n_seq_max is None else n_seq_max, None,
                          ctypes.pointer(timing) if timing is not None else None, None, None, None, None,
                          PRECISION[precision])
        st = lib().ppx_prefill_multi(self._h, seqs, k, ctypes.byref(p), _ptr(ws), ws.numel(), _ptr(logits),
                                     _stream(stream))
        _check(st, "ppx_prefill_multi")
        return logits

    def prefill_unified(self, prompts, seq_ids, cache: "UnifiedCache", n_ubatch: int = 512, prune: str = "auto",
                        logits=None, n_seq_max: int | None = None, stream=None, timing=None, precision: str = "fast"):
        """Several prompts in one pass over one unified cache, prompt s for
        sequence seq_ids[s]; return fp32 logits [n_seq][n_vocab]."""
        import torch
        toks = [np.ascontiguousarray(np.asarray(t, dtype=np.int32).reshape(-1)) for t in prompts]
        k = len(toks)
        if k != len(seq_ids):
            raise ValueError("one sequence id per prompt")
        seqs = (USeq * max(k, 1))()
        for i, (t, sid) in enumerate(zip(toks, seq_ids)):
            seqs[i] = USeq(int(sid), t.ctypes.data if t.size else None, int(t.shape[0]))
        if logits is None:
            logits = torch.empty((max(k, 1), self.info["n_vocab"]), dtype=torch.float32, device="cuda")
        total = max(1, sum(int(t.shape[0]) for t in toks))
        need = lib().ppx_workspace_bytes_unified(self._h, max(n_ubatch, 1), max(min(k, 64), 1), total,
                                                 cache.n_cells)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        ws = self._ws
        p = PrefillParams(n_ubatch, PRUNE[prune] if isinstance(prune, str) else int(prune), 0,
                          k if n_seq_max is None else n_seq_max, None,
                          ctypes.pointer(timing) if timing is not None else None, None, None, None, None,
                          PRECISION[precision])
        st = lib().ppx_prefill_unified(self._h, cache.handle, seqs, k, ctypes.byref(p), _ptr(ws), ws.numel(),
                                       _ptr(logits), _stream(stream))
        _check(st, "ppx_prefill_unified")
        return logits

    def decode(self, token: int, kv: "KVCache", logits=None, stream=None):
        """One generation step: `token` at kv.n_pos through every layer on the
        single-row path (owning layers append its K/V); return its fp32 logits."""
        import torch
        if logits is None:
            logits = torch.empty(self.info["n_vocab"], dtype=torch.float32, device="cuda")
        ws = self.workspace(1, kv.n_ctx)
        _check(lib().ppx_decode(self._h, kv.handle, int(token), _ptr(ws), ws.numel(), _ptr(logits), _stream(stream)),
               "ppx_decode")
        return logits

    # ---- kernel-level entry points
    def op_dequant(self, name: str):
        import torch
        rows, cols = self._shape(name)
        out = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
        _check(lib().ppx_op_dequant(self._h, name.encode(), _ptr(out), _stream()), "ppx_op_dequant")
        return out

    # fp16 GEMM operands travel in the engine's fragment-tiled layout (see
    # include/ppx.h); these helpers convert on the device.
    @staticmethod
    def untile(t, M: int, K: int):
        """fragment-tiled fp16 buffer -> row-major [M][K] (a torch view + copy)."""
        Mp = (M + 15) // 16 * 16
        return t[:Mp * K].view(Mp // 16, K // 32, 4, 16, 8).permute(0, 3, 1, 2, 4).reshape(Mp, K)[:M]

    def tile(self, a):
        """row-major fp16 [M][K] (device) -> fragment-tiled buffer of ceil(M/16)*16 rows."""
        import torch
        assert a.dtype == torch.float16 and a.is_contiguous() and a.dim() == 2
        M, K = a.shape
        t = torch.zeros(((M + 15) // 16 * 16) * K, dtype=torch.float16, device="cuda")
        _check(lib().ppx_op_tile_f16(_ptr(a), M, K, _ptr(t), _stream()), "ppx_op_tile_f16")
        return t

    def _gemm_ws(self, name: str, M: int, split: bool):
        """(tensor or None, bytes): scratch for a K split over workgroups."""
        import torch
        nb = lib().ppx_op_gemm_workspace_bytes(self._h, name.encode(), M) if split else 0
        if not nb:
            return None, 0
        return torch.empty(nb, dtype=torch.uint8, device="cuda"), nb

    def op_gemm(self, name: str, a, split: bool = True):
        """C = A W^T (fp32 [M][N]) for row-major fp16 A [M][K].  split=False
        runs shapes the engine splits over workgroups without the split."""
        import torch
        rows, cols = self._shape(name)
        assert a.shape[1] == cols
        M = a.shape[0]
        c = torch.empty((M, rows), dtype=torch.float32, device="cuda")
        at = self.tile(a)  # kept alive until the launch is queued
        ws, nb = self._gemm_ws(name, M, split)
        _check(lib().ppx_op_gemm(self._h, name.encode(), _ptr(at), M, _ptr(c), _ptr(ws) if nb else None, nb,
                                 _stream()), "ppx_op_gemm")
        return c

    def op_gemm_glu(self, name: str, a, M: int = None, out=None, raw: bool = False):
        """act(A Wg^T) * (A Wu^T) for a fused gate|up tensor name.  `a` is
        row-major fp16 [M][K], or (with M given) an already tiled buffer; the
        result is row-major fp16 [M][F], or the tiled buffer itself if raw."""
        import torch
        rows, cols = self._shape(name)
        F = rows // 2
        if M is None:
            assert a.shape[1] == cols
            M = a.shape[0]
            a = self.tile(a)
        Mp = (M + 15) // 16 * 16
        if out is None:
            out = torch.empty(Mp * F, dtype=torch.float16, device="cuda")
        assert out.dtype == torch.float16 and out.numel() >= Mp * F
        ws, nb = self._gemm_ws(name, M, True)
        _check(lib().ppx_op_gemm_glu(self._h, name.encode(), _ptr(a), M, _ptr(out), _ptr(ws) if nb else None, nb,
                                     _stream()), "ppx_op_gemm_glu")
        return out if raw else self.untile(out, M, F)

    def op_gemm_exact(self, name: str, a_hi, a_lo):
        import torch
        rows, cols = self._shape(name)
        assert a_hi.dtype == torch.float16 and a_lo.dtype == torch.float16 and a_hi.shape == a_lo.shape
        assert a_hi.shape[1] == cols
        c = torch.empty((a_hi.shape[0], rows), dtype=torch.float32, device="cuda")
        th, tl = self.tile(a_hi), self.tile(a_lo)  # both alive until the launch is queued
        _check(lib().ppx_op_gemm_exact(self._h, name.encode(), _ptr(th), _ptr(tl), a_hi.shape[0], _ptr(c),
                                       _stream()), "ppx_op_gemm_exact")
        return c

    def op_gemv(self, name: str, x):
        import torch
        rows, cols = self._shape(name)
        assert x.dtype == torch.float32 and x.numel() == cols
        y = torch.empty(rows, dtype=torch.float32, device="cuda")
        _check(lib().ppx_op_gemv(self._h, name.encode(), _ptr(x), _ptr(y), _stream()), "ppx_op_gemv")
        return y

    @staticmethod
    def _vt(v):
        """[P][KVH][hd] values -> the cache's transposed layout [KVH][hd][vld], vld = P rounded up to 64."""
        import torch
        P, kvh, hd = v.shape
        vld = (P + 63) // 64 * 64
        vt = torch.zeros((kvh, hd, vld), dtype=v.dtype, device=v.device)
        vt[:, :, :P] = v.permute(1, 2, 0)
        return vt, vld

    def op_attention(self, q, k, v, pos0: int):
        """q [M][H][hd], k/v [P][KVH][hd] (fp16); causal attention of rows at pos0.."""
        import torch
        H, hd = self.info["n_head"], self.info["head_dim"]
        M = q.shape[0]
        vt, vld = self._vt(v)
        o = torch.empty(((M + 15) // 16 * 16) * H * hd, dtype=torch.float16, device="cuda")
        need = lib().ppx_workspace_bytes(self._h, M, pos0 + M)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        _check(lib().ppx_op_attention(self._h, _ptr(q), _ptr(k), _ptr(vt), vld, M, pos0, _ptr(o), _ptr(ws), need,
                                      _stream()), "ppx_op_attention")
        return self.untile(o, M, H * hd)

    def op_attention_1row(self, q, k, v, pos: int):
        import torch
        H, hd = self.info["n_head"], self.info["head_dim"]
        o = torch.empty(H * hd, dtype=torch.float32, device="cuda")
        vt, vld = self._vt(v)
        need = lib().ppx_workspace_bytes(self._h, 1, pos + 1)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        _check(lib().ppx_op_attention_1row(self._h, _ptr(q), _ptr(k), _ptr(vt), vld, pos, _ptr(o), _ptr(ws), need,
                                           _stream()), "ppx_op_attention_1row")
        return o

    def _shape(self, name):
        I = self.info
        d, qd, kvd, F, E, V = (I["d_model"], I["n_head"] * I["head_dim"], I["kv_dim"], I["n_ff"], I["ple_dim"],
                               I["n_vocab"])
        if name in ("tok_embd", "output"):
            return V, d
        il = int(name.split(".")[1])
        kind = name.split(".", 2)[2]
        own = il < I["n_layer_kv_from_start"]
        return {"wq": (qd, d), "wk": (2 * kvd, d), "wo": (d, qd), "ffn_gate": (2 * F, d),
                "ffn_down": (d, F), "ple_gate": (E, d), "ple_up": (d, E)}[kind]


class KVCache:
    """fp16 KV cache of the KV-owning layers in a caller-owned (torch) device buffer."""

    def __init__(self, model: Model, n_ctx: int):
        import torch
        self.model = model
        self.n_ctx = n_ctx
        nbytes = lib().ppx_kv_bytes(model.handle, n_ctx)
        self.buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device="cuda")
        self._h = c_void_p()
        _check(lib().ppx_kv_init(model.handle, _ptr(self.buf), self.buf.numel(), n_ctx, ctypes.byref(self._h)),
               "ppx_kv_init")

    @property
    def handle(self):
        return self._h

    @property
    def n_pos(self) -> int:
        return lib().ppx_kv_n_pos(self._h)

    def clear(self):
        _check(lib().ppx_kv_clear(self._h), "ppx_kv_clear")

    def save(self, path, n_pos=None, stream=None):
        n = self.n_pos if n_pos is None else n_pos
        _check(lib().ppx_kv_save(self._h, os.fsencode(path), n, _stream(stream)), "ppx_kv_save")

    def load(self, path, n_pos, stream=None):
        _check(lib().ppx_kv_load(self._h, os.fsencode(path), n_pos, _stream(stream)), "ppx_kv_load")

    def save_tokens(self, path, tokens, n_pos=None, stream=None):
        """Snapshot with the token ids of the cached positions (tokens[:n_pos])."""
        import numpy as np
        n = self.n_pos if n_pos is None else n_pos
        ids = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32)[:n])
        if ids.size != n:
            raise ValueError("need one token id per saved position")
        _check(lib().ppx_kv_save_tokens(self._h, os.fsencode(path), n, ids.ctypes.data, _stream(stream)),
               "ppx_kv_save_tokens")

    def load_prefix(self, path, tokens, stream=None):
        """Load the longest cached prefix of `tokens` (at most len - 1); returns its length."""
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        out = ctypes.c_int(0)
        _check(lib().ppx_kv_load_prefix(self._h, os.fsencode(path), ids.ctypes.data, int(ids.size),
                                        ctypes.byref(out), _stream(stream)), "ppx_kv_load_prefix")
        return out.value

    def kv_tensors(self):
        """(K, V) as torch fp16 views [Ls][n_ctx][kv_dim] (V is a transposed view
        of the cache's [Ls][kv_dim][vld] layout)."""
        import torch
        I = self.model.info
        ls, kvd = I["n_layer_kv_from_start"], I["kv_dim"]
        n = ls * self.n_ctx * kvd
        kbytes = (2 * n + 255) // 256 * 256
        vld = (self.n_ctx + 63) // 64 * 64
        K = self.buf[:2 * n].view(torch.float16).view(ls, self.n_ctx, kvd)
        VT = self.buf[kbytes:kbytes + 2 * ls * kvd * vld].view(torch.float16).view(ls, kvd, vld)
        return K, VT[:, :, :self.n_ctx].transpose(1, 2)

    def close(self):
        if self._h:
            lib().ppx_kv_free(self._h)
            self._h = c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class UnifiedCache:
    """One fp16 KV buffer for several sequences (ids 0 .. n_seq_max - 1) in a
    caller-owned (torch) device buffer; cells are handed out in pages of 64
    positions of one sequence."""

    def __init__(self, model: Model, n_cells: int, n_seq_max: int):
        import torch
        self.model = model
        self.n_cells = n_cells
        nbytes = lib().ppx_kvu_bytes(model.handle, n_cells)
        if nbytes == 0:
            raise ValueError("n_cells must be a positive multiple of 64")
        self.buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        self._h = c_void_p()
        _check(lib().ppx_kvu_init(model.handle, _ptr(self.buf), self.buf.numel(), n_cells, n_seq_max,
                                  ctypes.byref(self._h)), "ppx_kvu_init")

    @property
    def handle(self):
        return self._h

    def n_pos(self, seq_id: int) -> int:
        return lib().ppx_kvu_n_pos(self._h, seq_id)

    def free_cells(self) -> int:
        return lib().ppx_kvu_free_cells(self._h)

    def seq_rm(self, seq_id: int):
        _check(lib().ppx_kvu_seq_rm(self._h, seq_id), "ppx_kvu_seq_rm")

    def cells(self, seq_id: int):
        """int32 [n_pos]: the cell of each position of the sequence."""
        n = self.n_pos(seq_id)
        out = np.zeros(max(n, 1), np.int32)
        _check(lib().ppx_kvu_cells(self._h, seq_id, out.ctypes.data, n), "ppx_kvu_cells")
        return out[:n]

    def kv_tensors(self):
        """(K, V) as torch fp16 views [Ls][n_cells][kv_dim] (V is a transposed
        view of the [Ls][kv_dim][n_cells] layout)."""
        import torch
        I = self.model.info
        ls, kvd = I["n_layer_kv_from_start"], I["kv_dim"]
        n = ls * self.n_cells * kvd
        kbytes = (2 * n + 255) // 256 * 256
        K = self.buf[:2 * n].view(torch.float16).view(ls, self.n_cells, kvd)
        VT = self.buf[kbytes:kbytes + 2 * n].view(torch.float16).view(ls, kvd, self.n_cells)
        return K, VT.transpose(1, 2)

    def seq_kv(self, seq_id: int):
        """(K, V) of one sequence in position order, torch fp16 [Ls][n_pos][kv_dim]."""
        import torch
        K, V = self.kv_tensors()
        idx = torch.from_numpy(self.cells(seq_id).astype(np.int64)).to(K.device)
        return K[:, idx], V[:, idx]

    def close(self):
        if self._h:
            lib().ppx_kvu_free(self._h)
            self._h = c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
