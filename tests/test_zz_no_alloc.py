"""ppx_decode_static, the allocation-free variant of ppx_decode: the same
kernels on a library-held device scratch array instead of a caller
workspace.  Called through the C ABI and checked against ppx_decode on an
identical cache: logits and the appended K/V rows bit for bit, on two calls
in a row, the second on a shorter cache (less scratch in use, the first
call's contents left behind)."""
import ctypes

import numpy as np
import pytest

import synth
from tests.gpu_common import container

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ppx():
    import prompt_prefill_cross_amd as p
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    p.lib()
    return p


def _static_decode(ppx, mm, kv, token, logits):
    s = torch.cuda.current_stream().cuda_stream
    return ppx.lib().ppx_decode_static(mm.handle, kv.handle, int(token), ctypes.c_void_p(logits.data_ptr()),
                                       ctypes.c_void_p(s))


@pytest.mark.parametrize("cfg", ["tiny", "e2b"])
def test_decode_static_matches_decode(ppx, cfg):
    mm = ppx.Model(container(cfg))
    V = mm.info["n_vocab"]
    toks = synth.prompt(cfg, 700)
    assert ppx.lib().ppx_decode_static_limit() == 32 << 20
    for n0, n_ctx in ((600, 640), (40, 64)):  # the second call: a shorter cache, less scratch in use
        kva, kvb = ppx.KVCache(mm, n_ctx), ppx.KVCache(mm, n_ctx)
        mm.prefill(toks[:n0], kva, n_ubatch=512)
        mm.prefill(toks[:n0], kvb, n_ubatch=512)
        torch.cuda.synchronize()
        assert torch.equal(kva.buf, kvb.buf)
        ref = mm.decode(int(toks[n0]), kva).clone()
        got = torch.full((V,), float("nan"), dtype=torch.float32, device="cuda")
        st = _static_decode(ppx, mm, kvb, toks[n0], got)
        torch.cuda.synchronize()
        assert st == 0
        assert kvb.n_pos == kva.n_pos == n0 + 1
        assert torch.equal(got, ref), (cfg, n0, float((got - ref).abs().max()))
        assert torch.equal(kva.buf, kvb.buf)
        kva.close()
        kvb.close()
    mm.close()


def test_decode_static_refuses_a_context_beyond_its_scratch(ppx):
    mm = ppx.Model(container("tiny"))
    L = ppx.lib()
    n_ctx = 1 << 20
    assert L.ppx_workspace_bytes(mm.handle, 1, n_ctx) > L.ppx_decode_static_limit()
    kv = ppx.KVCache(mm, n_ctx)
    logits = torch.empty(mm.info["n_vocab"], dtype=torch.float32, device="cuda")
    assert _static_decode(ppx, mm, kv, 1, logits) == -9
    assert kv.n_pos == 0
    kv.close()
    mm.close()
