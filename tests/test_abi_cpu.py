"""The C ABI without a GPU: the library loads, exports what the header declares, sizes
its workspace, and rejects bad arguments on the host before anything is enqueued.

Every call below fails validation, so no kernel is ever launched (the pointers are
placeholders that are never dereferenced)."""
from __future__ import annotations

import ctypes
import os

import pytest

from lossless_rejection_sampling_verify_amd import _lib as L

P = 1 << 20          # a 256-byte aligned placeholder address (never dereferenced)


@pytest.fixture(scope="module")
def lib():
    return L.lib()


def test_exports_every_declared_symbol(lib):
    names = L.declared_functions()
    assert set(names) >= {"spec_verify_greedy", "spec_verify_chain", "spec_verify_tree",
                          "spec_tree_mask", "spec_tree_commit_kv", "spec_verify_chain_filtered",
                          "spec_verify_tree_mss",
                          "spec_workspace_bytes",
                          "spec_status_str"}
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert L.status_str(code) and L.status_str(code) != "unknown status"
    assert L.status_str(17) == "unknown status"


def test_workspace_bytes(lib):
    a = L.workspace_bytes(L.SPEC_OP_CHAIN, 256, 5, 152064)
    assert a > 0 and a % 256 == 0
    assert L.workspace_bytes(L.SPEC_OP_CHAIN, 512, 5, 152064) > a
    assert L.workspace_bytes(L.SPEC_OP_GREEDY, 1, 65, 10) > 0
    assert L.workspace_bytes(L.SPEC_OP_GREEDY, 1, 66, 10) == 0       # G > 64
    assert L.workspace_bytes(L.SPEC_OP_CHAIN, 1, 1, 10) == 0         # G = 0
    assert L.workspace_bytes(L.SPEC_OP_TREE, 4, 1024, 10) > 0
    assert L.workspace_bytes(L.SPEC_OP_TREE, 4, 1025, 10) == 0
    assert L.workspace_bytes(7, 4, 5, 10) == 0
    assert L.workspace_bytes(L.SPEC_OP_CHAIN, 4, 5, 0) == 0


def _greedy(lib, logits=P, dtype=L.SPEC_BF16, tokens=P, B=2, G=4, V=1000, acc=P, out=P,
            ws=P, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = L.workspace_bytes(L.SPEC_OP_GREEDY, max(B, 1), G + 1, max(V, 1)) or 1 << 20
    return lib.spec_verify_greedy(logits, dtype, tokens, B, G, V, acc, out, ws, ws_bytes, None)


def test_greedy_rejects_bad_arguments(lib):
    assert _greedy(lib, logits=None) == L.SPEC_ERR_NULL
    assert _greedy(lib, tokens=None) == L.SPEC_ERR_NULL
    assert _greedy(lib, acc=None) == L.SPEC_ERR_NULL
    assert _greedy(lib, ws=None) == L.SPEC_ERR_NULL
    assert _greedy(lib, dtype=5) == L.SPEC_ERR_DTYPE
    assert _greedy(lib, G=0) == L.SPEC_ERR_SHAPE
    assert _greedy(lib, G=65) == L.SPEC_ERR_SHAPE
    assert _greedy(lib, V=0) == L.SPEC_ERR_SHAPE
    assert _greedy(lib, V=1 << 30) == L.SPEC_ERR_SHAPE                    # 2^31 bytes a row
    assert _greedy(lib, V=1 << 29, dtype=L.SPEC_F32) == L.SPEC_ERR_SHAPE
    assert _greedy(lib, B=-1) == L.SPEC_ERR_SHAPE
    assert _greedy(lib, logits=P + 1) == L.SPEC_ERR_PARAM                 # not bf16-aligned
    assert _greedy(lib, logits=P + 2, dtype=L.SPEC_F32) == L.SPEC_ERR_PARAM
    assert _greedy(lib, ws=P + 16) == L.SPEC_ERR_WORKSPACE
    assert _greedy(lib, ws_bytes=64) == L.SPEC_ERR_WORKSPACE
    assert _greedy(lib, B=0) == L.SPEC_OK                                 # nothing to do


def _chain(lib, **kw):
    a = dict(logits=P, dtype=L.SPEC_BF16, q=P, tokens=P, coins=P, temp=P, B=3, G=4, V=2000,
             acc=P, out=P, probs=None, ws=P, ws_bytes=None)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = L.workspace_bytes(L.SPEC_OP_CHAIN, max(a["B"], 1), a["G"] + 1, max(a["V"], 1)) or 1 << 20
    return lib.spec_verify_chain(a["logits"], a["dtype"], a["q"], a["tokens"], a["coins"],
                                 a["temp"], a["B"], a["G"], a["V"], a["acc"], a["out"],
                                 a["probs"], a["ws"], a["ws_bytes"], None)


def test_chain_rejects_bad_arguments(lib):
    for k in ("logits", "q", "tokens", "coins", "temp", "acc", "out", "ws"):
        assert _chain(lib, **{k: None}) == L.SPEC_ERR_NULL, k
    assert _chain(lib, dtype=2) == L.SPEC_ERR_DTYPE
    assert _chain(lib, G=0) == L.SPEC_ERR_SHAPE
    assert _chain(lib, G=65) == L.SPEC_ERR_SHAPE
    assert _chain(lib, V=1 << 30) == L.SPEC_ERR_SHAPE  # a bf16 row of 2^31 bytes
    assert _chain(lib, q=P + 2) == L.SPEC_ERR_PARAM
    assert _chain(lib, ws_bytes=1024) == L.SPEC_ERR_WORKSPACE
    assert _chain(lib, B=0) == L.SPEC_OK


def _tree(lib, **kw):
    a = dict(logits=P, dtype=L.SPEC_F32, tok=P, par=P, coins=P, temp=P, B=2, N=64, V=500, D=6,
             mode=L.SPEC_TREE_SAMPLING, ts=1.0, ta=1.0, acc=P, out=P, nodes=P, probs=None,
             ws=P, ws_bytes=None)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = L.workspace_bytes(L.SPEC_OP_TREE, max(a["B"], 1), max(a["N"], 1), max(a["V"], 1)) or 1 << 20
    return lib.spec_verify_tree(a["logits"], a["dtype"], a["tok"], a["par"], a["coins"], a["temp"],
                                a["B"], a["N"], a["V"], a["D"], a["mode"], a["ts"], a["ta"],
                                a["acc"], a["out"], a["nodes"], a["probs"], a["ws"],
                                a["ws_bytes"], None)


def test_tree_rejects_bad_arguments(lib):
    for k in ("logits", "tok", "par", "acc", "out", "nodes", "ws", "coins", "temp"):
        assert _tree(lib, **{k: None}) == L.SPEC_ERR_NULL, k
    assert _tree(lib, mode=2) == L.SPEC_ERR_PARAM
    assert _tree(lib, V=1 << 29) == L.SPEC_ERR_SHAPE  # an fp32 row of 2^31 bytes
    assert _tree(lib, ts=0.0) == L.SPEC_ERR_PARAM
    assert _tree(lib, ta=-1.0) == L.SPEC_ERR_PARAM
    assert _tree(lib, ta=float("nan")) == L.SPEC_ERR_PARAM
    assert _tree(lib, N=1025) == L.SPEC_ERR_SHAPE
    assert _tree(lib, N=0) == L.SPEC_ERR_SHAPE
    assert _tree(lib, D=0) == L.SPEC_ERR_SHAPE
    assert _tree(lib, dtype=9) == L.SPEC_ERR_DTYPE
    assert _tree(lib, ws_bytes=1000) == L.SPEC_ERR_WORKSPACE
    # greedy mode needs neither coins nor temperature: check only up to validation
    assert _tree(lib, mode=L.SPEC_TREE_GREEDY, coins=None, temp=None, ws=None) == L.SPEC_ERR_NULL
    assert _tree(lib, B=0, mode=L.SPEC_TREE_GREEDY, coins=None, temp=None) == L.SPEC_OK



def test_tree_mask_rejects_bad_arguments(lib):
    assert lib.spec_tree_mask(None, None, 2, 8, P, P, None) == L.SPEC_ERR_NULL
    assert lib.spec_tree_mask(P, None, 2, 8, None, P, None) == L.SPEC_ERR_NULL
    assert lib.spec_tree_mask(P, None, -1, 8, P, P, None) == L.SPEC_ERR_SHAPE
    assert lib.spec_tree_mask(P, None, 2, 0, P, P, None) == L.SPEC_ERR_SHAPE
    assert lib.spec_tree_mask(P, None, 2, L.SPEC_MAX_N + 1, P, P, None) == L.SPEC_ERR_SHAPE
    assert lib.spec_tree_mask(P, None, 0, 8, P, None, None) == L.SPEC_OK



def test_tree_commit_kv_rejects_bad_arguments(lib):
    f = lib.spec_tree_commit_kv
    assert f(None, P, 2, 4, 8, P, P, 64, P, None) == L.SPEC_ERR_NULL
    assert f(P, None, 2, 4, 8, P, P, 64, P, None) == L.SPEC_ERR_NULL
    assert f(P, P, 2, 4, 8, None, P, 64, P, None) == L.SPEC_ERR_NULL
    assert f(P, P, 2, 4, 8, P, None, 64, P, None) == L.SPEC_ERR_NULL
    assert f(P, P, -1, 4, 8, P, P, 64, P, None) == L.SPEC_ERR_SHAPE
    assert f(P, P, 2, 0, 8, P, P, 64, P, None) == L.SPEC_ERR_SHAPE
    assert f(P, P, 2, 4, 0, P, P, 64, P, None) == L.SPEC_ERR_SHAPE
    assert f(P, P, 2, 4, L.SPEC_MAX_N + 1, P, P, 64, P, None) == L.SPEC_ERR_SHAPE
    assert f(P, P, 2, 4, 8, P, P, 0, P, None) == L.SPEC_ERR_SHAPE
    assert f(P, P, 0, 4, 8, P, P, 64, None, None) == L.SPEC_OK



def test_chain_filtered_rejects_bad_arguments(lib):
    f = lib.spec_verify_chain_filtered
    ws = L.workspace_bytes(L.SPEC_OP_CHAIN_FILTERED, 2, 5, 1000)
    assert ws > 0
    args = dict(lg=P, dl=P, dt=L.SPEC_BF16, tok=P, coins=P, T=P, k=None, p=None, B=2, G=4,
                V=1000, acc=P, out=P, probs=None, ws=P, wsb=ws)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["lg"], a["dl"], a["dt"], a["tok"], a["coins"], a["T"], a["k"], a["p"], a["B"],
                 a["G"], a["V"], a["acc"], a["out"], a["probs"], a["ws"], a["wsb"], None)
    assert call(lg=None) == L.SPEC_ERR_NULL
    assert call(dl=None) == L.SPEC_ERR_NULL
    assert call(coins=None) == L.SPEC_ERR_NULL
    assert call(G=0) == L.SPEC_ERR_SHAPE
    assert call(G=65) == L.SPEC_ERR_SHAPE
    assert call(dt=7) == L.SPEC_ERR_DTYPE
    assert call(wsb=ws - 1) == L.SPEC_ERR_WORKSPACE
    assert call(dl=P + 1) == L.SPEC_ERR_PARAM
    assert call(B=0) == L.SPEC_OK


def test_tree_mss_rejects_bad_arguments(lib):
    f = lib.spec_verify_tree_mss
    ws = L.workspace_bytes(L.SPEC_OP_TREE_MSS, 2, 64, 1000)
    assert 0 < ws < L.workspace_bytes(L.SPEC_OP_TREE, 2, 64, 1000)   # no row records
    assert L.workspace_bytes(L.SPEC_OP_TREE_MSS, 2, L.SPEC_MAX_N + 1, 1000) == 0
    args = dict(lg=P, dt=L.SPEC_BF16, q=P, tok=P, par=P, coins=P, T=P, B=2, N=64, V=1000, D=6,
                acc=P, out=P, nodes=P, probs=None, ws=P, wsb=ws)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["lg"], a["dt"], a["q"], a["tok"], a["par"], a["coins"], a["T"], a["B"], a["N"],
                 a["V"], a["D"], a["acc"], a["out"], a["nodes"], a["probs"], a["ws"], a["wsb"], None)
    for k in ("lg", "q", "tok", "par", "coins", "T", "acc", "out", "nodes", "ws"):
        assert call(**{k: None}) == L.SPEC_ERR_NULL, k
    assert call(N=0) == L.SPEC_ERR_SHAPE
    assert call(N=L.SPEC_MAX_N + 1) == L.SPEC_ERR_SHAPE
    assert call(D=0) == L.SPEC_ERR_SHAPE
    assert call(dt=5) == L.SPEC_ERR_DTYPE
    assert call(wsb=ws - 1) == L.SPEC_ERR_WORKSPACE
    assert call(q=P + 2) == L.SPEC_ERR_PARAM
    assert call(B=0) == L.SPEC_OK


def test_calibration_utilities_reject_bad_arguments(lib):
    """Argument errors of the measurement utilities are found on the host, before any
    launch (these pointers are never dereferenced)."""
    fake = ctypes.c_void_p(1 << 20)  # 16-byte aligned, non-null, never read
    assert lib.spec_calib_read(None, 0, None, None) == L.SPEC_OK        # nothing to read
    assert lib.spec_calib_read(None, 16, fake, None) == L.SPEC_ERR_NULL
    assert lib.spec_calib_read(fake, 16, None, None) == L.SPEC_ERR_NULL
    assert lib.spec_calib_read(ctypes.c_void_p((1 << 20) + 4), 16, fake, None) == L.SPEC_ERR_PARAM
    assert lib.spec_calib_read(fake, 24, fake, None) == L.SPEC_ERR_PARAM
    assert lib.spec_calib_exp(1, 1, None, None) == L.SPEC_ERR_NULL
    for blocks, iters in ((0, 1), (65536, 1), (1, 0), (1, (1 << 20) + 1)):
        assert lib.spec_calib_exp(blocks, iters, fake, None) == L.SPEC_ERR_PARAM


def test_c_consumer_is_built_and_checks_its_arguments():
    """The plain C consumer of the ABI links against the library and rejects a bad command
    line before any device call (no GPU needed)."""
    import subprocess
    demo = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "lossless_rejection_sampling_verify_amd", "abi_demo")
    assert os.path.exists(demo), "build the package first"
    r = subprocess.run([demo], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr


def test_options_are_checked_on_the_host(lib):
    """The *_opt entry points reject bad launch options before anything is enqueued; NULL
    options and all-zero options are the defaults."""
    ws = L.workspace_bytes(L.SPEC_OP_CHAIN, 3, 5, 2000)

    def chain(o):
        return lib.spec_verify_chain_opt(P, L.SPEC_BF16, P, P, P, P, 0, 4, 2000, P, P, None, P, ws,
                                         None, o)
    assert chain(None) == L.SPEC_OK
    assert chain(ctypes.byref(L.SpecOptions())) == L.SPEC_OK
    for bad in (dict(path=2), dict(path=-1), dict(cluster=-1), dict(splits=-3),
                dict(row_loads=3), dict(spin_limit=-1)):
        o = L.SpecOptions(**bad)
        assert chain(ctypes.byref(o)) == L.SPEC_ERR_PARAM, bad
        assert lib.spec_verify_greedy_opt(P, L.SPEC_BF16, P, 0, 4, 1000, P, P, P,
                                          L.workspace_bytes(L.SPEC_OP_GREEDY, 1, 5, 1000), None,
                                          ctypes.byref(o)) == L.SPEC_ERR_PARAM, bad
        assert lib.spec_verify_tree_opt(P, L.SPEC_F32, P, P, P, P, 0, 8, 500, 3, 1, 1.0, 1.0,
                                        P, P, P, None, P,
                                        L.workspace_bytes(L.SPEC_OP_TREE, 1, 8, 500), None,
                                        ctypes.byref(o)) == L.SPEC_ERR_PARAM, bad
        assert lib.spec_verify_tree_mss_opt(P, L.SPEC_F32, P, P, P, P, P, 0, 8, 500, 3, P, P, P,
                                            None, P,
                                            L.workspace_bytes(L.SPEC_OP_TREE_MSS, 1, 8, 500),
                                            None, ctypes.byref(o)) == L.SPEC_ERR_PARAM, bad
    # argument errors still come first
    assert lib.spec_verify_chain_opt(None, L.SPEC_BF16, P, P, P, P, 3, 4, 2000, P, P, None, P, ws,
                                     None, ctypes.byref(L.SpecOptions(path=9))) == L.SPEC_ERR_NULL


def test_python_options_helper():
    o = L.options(dict(path="eager", cluster=3, row_loads="streaming", spin_limit=7))
    assert (o.path, o.cluster, o.splits, o.row_loads, o.spin_limit) == \
        (L.SPEC_PATH_EAGER, 3, 0, L.SPEC_LOADS_STREAMING, 7)
    assert L.options(None) is None
    with pytest.raises(ValueError):
        L.options(dict(eager=1))


def test_workspace_header_is_shape_independent(lib):
    """The walks' call counter and per-request exit words sit in a header of fixed size at
    the start of every workspace, so one zero-filled buffer can serve calls of any shape
    in turn: the smallest workspace of every kind is at least that header."""
    sizes = [L.workspace_bytes(op, 1, r, 1) for op, r in
             ((L.SPEC_OP_GREEDY, 2), (L.SPEC_OP_CHAIN, 2), (L.SPEC_OP_TREE, 1),
              (L.SPEC_OP_CHAIN_FILTERED, 2), (L.SPEC_OP_TREE_MSS, 1))]
    assert min(sizes) >= 256 + 4 * 4096
