"""spec_verify_chain_noalloc (no workspace argument, the library's static scratch) gives
the results of spec_verify_chain with a caller workspace, call after call.

Both are called through the C ABI (ctypes) on the same device inputs: two calls in a row,
the second on a smaller batch with a smaller vocabulary (the static scratch keeps the
first call's contents), then the first shape again; outputs must be bitwise identical to
the workspace entry point's (same kernels, same launch shapes).  Sizes beyond the static
scratch are refused on the host with SPEC_ERR_TOO_LARGE.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

from lossless_rejection_sampling_verify_amd import _lib as L
from lossless_rejection_sampling_verify_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _inputs(c, dev):
    lg = np.ascontiguousarray(c.logits)
    logits = (torch.from_numpy(lg.view(np.int16)).view(torch.bfloat16) if c.dtype == wl.BF16
              else torch.from_numpy(lg)).to(dev)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return dict(logits=logits, dtype=L.SPEC_BF16 if c.dtype == wl.BF16 else L.SPEC_F32,
                q=t(c.draft_probs), x=t(c.draft_tokens), u=t(c.coins), T=t(c.temperature))


def _call(lib, d, c, noalloc, ws=None):
    dev = d["logits"].device
    acc = torch.full((c.B,), -7, dtype=torch.int32, device=dev)
    out = torch.full((c.B, c.R), -7, dtype=torch.int32, device=dev)
    probs = torch.full((c.B, c.R), -7.0, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = [d["logits"].data_ptr(), d["dtype"], d["q"].data_ptr(), d["x"].data_ptr(),
            d["u"].data_ptr(), d["T"].data_ptr(), c.B, c.G, c.V, acc.data_ptr(),
            out.data_ptr(), probs.data_ptr()]
    if noalloc:
        rc = lib.spec_verify_chain_noalloc(*args, stream)
    else:
        rc = lib.spec_verify_chain(*args, ws.data_ptr(), ws.numel(), stream)
    assert rc == L.SPEC_OK, L.status_str(rc)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), out.cpu().numpy(), probs.cpu().numpy()


def test_noalloc_matches_the_workspace_entry_point():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = L.lib()
    dev = torch.device("cuda:0")
    big = wl.make_chain(5, seed=61, B=256, G=4, V=152064)
    small = wl.make_chain(3, seed=62, B=24, G=6, V=50021, dtype=wl.F32, T=0.8)
    for c in (big, small, big):
        print(f"[gpu-case] noalloc chain B={c.B} G={c.G} V={c.V} {c.dtype}", flush=True)
        d = _inputs(c, dev)
        ws = torch.zeros(L.workspace_bytes(L.SPEC_OP_CHAIN, c.B, c.R, c.V), dtype=torch.uint8,
                         device=dev)
        want = _call(lib, d, c, False, ws)
        got = _call(lib, d, c, True)
        for a, b in zip(got, want):
            np.testing.assert_array_equal(a, b)
        assert (got[0] >= 0).all()


def test_noalloc_refuses_sizes_beyond_its_scratch():
    lib = L.lib()
    P = 1 << 20
    # B = 4096 requests of G = 4 at V = 152064 need about 110 MB of workspace
    rc = lib.spec_verify_chain_noalloc(P, L.SPEC_BF16, P, P, P, P, 4096, 4, 152064, P, P, None,
                                       None)
    assert rc == L.SPEC_ERR_TOO_LARGE
    assert "static" in L.status_str(rc)
    assert lib.spec_verify_chain_noalloc(P, L.SPEC_BF16, P, P, P, P, 8, 0, 1000, P, P, None,
                                         None) == L.SPEC_ERR_SHAPE
    assert lib.spec_verify_chain_noalloc(None, L.SPEC_BF16, P, P, P, P, 8, 4, 1000, P, P, None,
                                         None) == L.SPEC_ERR_NULL
