"""Python access to the plain fp64 CPU oracle (``liboracle.so``).

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the library path never does.  The oracle is
C compiled with gcc (``build()``); it shares no source with the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC = os.path.join(_HERE, "spec_oracle.c")

F32, BF16 = 0, 1
TREE_GREEDY, TREE_SAMPLING = 0, 1

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (OpenMP over requests, IEEE double arithmetic)."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True, cwd=_HERE)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        vp, ip = ctypes.c_void_p, ctypes.c_int
        L.oracle_verify_greedy.argtypes = [vp, ip, vp, ip, ip, ip, vp, vp]
        L.oracle_verify_chain.argtypes = [vp, ip, vp, vp, vp, vp, ip, ip, ip, vp, vp, vp, vp, vp,
                                          vp]
        L.oracle_verify_tree.argtypes = [vp, ip, vp, vp, vp, vp, ip, ip, ip, ip, ip,
                                         ctypes.c_float, ctypes.c_float, vp, vp, vp, vp, vp, vp]
        for f in (L.oracle_verify_greedy, L.oracle_verify_chain, L.oracle_verify_tree):
            f.restype = ctypes.c_int
        L.oracle_tree_mask.argtypes = [vp, vp, ip, ip, vp, vp]
        L.oracle_tree_mask.restype = ctypes.c_int
        L.oracle_tree_commit_kv.argtypes = [vp, vp, ip, ip, ip, vp, vp, ctypes.c_size_t, vp]
        L.oracle_tree_commit_kv.restype = ctypes.c_int
        L.oracle_verify_chain_filtered.argtypes = [vp, vp, ip, vp, vp, vp, vp, vp, ip, ip, ip,
                                                   vp, vp, vp, vp, vp]
        L.oracle_verify_chain_filtered.restype = ctypes.c_int
        L.oracle_verify_tree_mss.argtypes = [vp, ip, vp, vp, vp, vp, vp, ip, ip, ip, ip,
                                             vp, vp, vp, vp, vp, vp]
        L.oracle_verify_tree_mss.restype = ctypes.c_int
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_num_threads.argtypes = [ip]
        L.oracle_set_num_threads.restype = None
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for this Python thread's later oracle calls."""
    lib().oracle_set_num_threads(int(n))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(dtype: str) -> int:
    return BF16 if dtype == "bf16" else F32


def _logits_array(logits, dtype):
    want = np.uint16 if dtype == "bf16" else np.float32
    a = np.ascontiguousarray(logits)
    if a.dtype != want:
        if dtype == "bf16" and a.dtype == np.int16:
            a = a.view(np.uint16)
        else:
            raise TypeError(f"logits must be {want} for dtype {dtype}, got {a.dtype}")
    return a


def verify_greedy(logits, dtype, draft_tokens, B=None, G=None, V=None):
    """Returns (accept_len [B], out_tokens [B][G+1])."""
    lg = _logits_array(logits, dtype)
    dt = np.ascontiguousarray(draft_tokens, dtype=np.int32)
    B = dt.shape[0] if B is None else B
    G = dt.shape[1] if G is None else G
    V = lg.shape[-1] if V is None else V
    acc = np.empty(B, np.int32)
    out = np.empty((B, G + 1), np.int32)
    rc = lib().oracle_verify_greedy(_ptr(lg), _dtype_code(dtype), _ptr(dt), B, G, V,
                                    _ptr(acc), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_verify_greedy rejected its arguments ({rc})")
    return acc, out


def verify_chain(logits, dtype, draft_probs, draft_tokens, coins, temperature, *, beta=False):
    """Returns dict(accept_len, out_tokens, probs, margin, accept_margin[, beta])."""
    lg = _logits_array(logits, dtype)
    q = np.ascontiguousarray(draft_probs, dtype=np.float32)
    dt = np.ascontiguousarray(draft_tokens, dtype=np.int32)
    cn = np.ascontiguousarray(coins, dtype=np.float32)
    tp = np.ascontiguousarray(temperature, dtype=np.float32)
    B, G = dt.shape
    V = lg.shape[-1]
    acc = np.empty(B, np.int32)
    out = np.empty((B, G + 1), np.int32)
    probs = np.empty((B, G + 1), np.float64)
    margin = np.empty(B, np.float64)
    amargin = np.empty(B, np.float64)
    bt = np.empty((B, G), np.float64) if beta else None
    rc = lib().oracle_verify_chain(_ptr(lg), _dtype_code(dtype), _ptr(q), _ptr(dt), _ptr(cn),
                                   _ptr(tp), B, G, V, _ptr(acc), _ptr(out), _ptr(probs),
                                   _ptr(margin), _ptr(bt), _ptr(amargin))
    if rc != 0:
        raise ValueError(f"oracle_verify_chain rejected its arguments ({rc})")
    res = dict(accept_len=acc, out_tokens=out, probs=probs, margin=margin, accept_margin=amargin)
    if beta:
        res["beta"] = bt
    return res


def verify_tree(logits, dtype, node_tokens, parents, coins, temperature, D, mode,
                threshold_single=1.0, threshold_acc=1.0):
    """Returns dict(accept_len, out_tokens, accepted_nodes, probs, margin, accept_margin)."""
    lg = _logits_array(logits, dtype)
    tk = np.ascontiguousarray(node_tokens, dtype=np.int32)
    pa = np.ascontiguousarray(parents, dtype=np.int32)
    cn = None if coins is None else np.ascontiguousarray(coins, dtype=np.float32)
    tp = None if temperature is None else np.ascontiguousarray(temperature, dtype=np.float32)
    B, N = tk.shape
    V = lg.shape[-1]
    acc = np.empty(B, np.int32)
    out = np.empty((B, D + 1), np.int32)
    nodes = np.empty((B, D), np.int32)
    probs = np.empty((B, D + 1), np.float64)
    margin = np.empty(B, np.float64)
    amargin = np.empty(B, np.float64)
    rc = lib().oracle_verify_tree(_ptr(lg), _dtype_code(dtype), _ptr(tk), _ptr(pa), _ptr(cn),
                                  _ptr(tp), B, N, V, D, mode, float(threshold_single),
                                  float(threshold_acc), _ptr(acc), _ptr(out), _ptr(nodes),
                                  _ptr(probs), _ptr(margin), _ptr(amargin))
    if rc != 0:
        raise ValueError(f"oracle_verify_tree rejected its arguments ({rc})")
    return dict(accept_len=acc, out_tokens=out, accepted_nodes=nodes, probs=probs,
                margin=margin, accept_margin=amargin)


def tree_mask(parents, base_pos=None):
    """Returns (mask [B][N][ceil(N/32)] uint32 bit rows, positions [B][N] int32)."""
    pa = np.ascontiguousarray(parents, dtype=np.int32)
    B, N = pa.shape
    W = (N + 31) // 32
    bp = None if base_pos is None else np.ascontiguousarray(base_pos, dtype=np.int32)
    mask = np.empty((B, N, W), np.uint32)
    pos = np.empty((B, N), np.int32)
    rc = lib().oracle_tree_mask(_ptr(pa), _ptr(bp), B, N, _ptr(mask), _ptr(pos))
    if rc != 0:
        raise ValueError(f"oracle_tree_mask rejected its arguments ({rc})")
    return mask, pos


def tree_commit_kv(accepted_nodes, accept_len, kv_tree, kv_out):
    """kv_tree [B][N][row_bytes] uint8, kv_out [B][D+1][row_bytes] uint8 (updated in place).
    Returns slots [B][D+1] int32."""
    nodes = np.ascontiguousarray(accepted_nodes, dtype=np.int32)
    acc = np.ascontiguousarray(accept_len, dtype=np.int32)
    B, D = nodes.shape
    src = np.ascontiguousarray(kv_tree, dtype=np.uint8)
    if not (kv_out.flags["C_CONTIGUOUS"] and kv_out.dtype == np.uint8):
        raise TypeError("kv_out must be a C-contiguous uint8 array")
    N, row_bytes = src.shape[1], src.shape[2]
    slots = np.empty((B, D + 1), np.int32)
    rc = lib().oracle_tree_commit_kv(_ptr(nodes), _ptr(acc), B, D, N, _ptr(src), _ptr(kv_out),
                                     row_bytes, _ptr(slots))
    if rc != 0:
        raise ValueError(f"oracle_tree_commit_kv rejected its arguments ({rc})")
    return slots


def verify_chain_filtered(logits, draft_logits, dtype, draft_tokens, coins, temperature,
                          top_k=None, top_p=None):
    """Returns dict(accept_len, out_tokens, probs, margin, accept_margin)."""
    lg = _logits_array(logits, dtype)
    dl = _logits_array(draft_logits, dtype)
    dt = np.ascontiguousarray(draft_tokens, dtype=np.int32)
    cn = np.ascontiguousarray(coins, dtype=np.float32)
    tp = np.ascontiguousarray(temperature, dtype=np.float32)
    tk = None if top_k is None else np.ascontiguousarray(top_k, dtype=np.int32)
    pp = None if top_p is None else np.ascontiguousarray(top_p, dtype=np.float32)
    B, G = dt.shape
    V = lg.shape[-1]
    acc = np.empty(B, np.int32)
    out = np.empty((B, G + 1), np.int32)
    probs = np.empty((B, G + 1), np.float64)
    margin = np.empty(B, np.float64)
    amargin = np.empty(B, np.float64)
    rc = lib().oracle_verify_chain_filtered(_ptr(lg), _ptr(dl), _dtype_code(dtype), _ptr(dt),
                                            _ptr(cn), _ptr(tp), _ptr(tk), _ptr(pp), B, G, V,
                                            _ptr(acc), _ptr(out), _ptr(probs), _ptr(margin),
                                            _ptr(amargin))
    if rc != 0:
        raise ValueError(f"oracle_verify_chain_filtered rejected its arguments ({rc})")
    return dict(accept_len=acc, out_tokens=out, probs=probs, margin=margin, accept_margin=amargin)


def verify_tree_mss(logits, dtype, draft_probs, node_tokens, parents, coins, temperature, D):
    """Tree verify by multi-step speculative sampling with draft rows [B][N][V] and per-node
    coins [B][N].  Returns dict(accept_len, out_tokens, accepted_nodes, probs, margin,
    accept_margin)."""
    lg = _logits_array(logits, dtype)
    q = np.ascontiguousarray(draft_probs, dtype=np.float32)
    tk = np.ascontiguousarray(node_tokens, dtype=np.int32)
    pa = np.ascontiguousarray(parents, dtype=np.int32)
    cn = np.ascontiguousarray(coins, dtype=np.float32)
    tp = np.ascontiguousarray(temperature, dtype=np.float32)
    B, N = tk.shape
    V = lg.shape[-1]
    acc = np.empty(B, np.int32)
    out = np.empty((B, D + 1), np.int32)
    nodes = np.empty((B, D), np.int32)
    probs = np.empty((B, D + 1), np.float64)
    margin = np.empty(B, np.float64)
    amargin = np.empty(B, np.float64)
    rc = lib().oracle_verify_tree_mss(_ptr(lg), _dtype_code(dtype), _ptr(q), _ptr(tk), _ptr(pa),
                                      _ptr(cn), _ptr(tp), B, N, V, D, _ptr(acc), _ptr(out),
                                      _ptr(nodes), _ptr(probs), _ptr(margin), _ptr(amargin))
    if rc != 0:
        raise ValueError(f"oracle_verify_tree_mss rejected its arguments ({rc})")
    return dict(accept_len=acc, out_tokens=out, accepted_nodes=nodes, probs=probs,
                margin=margin, accept_margin=amargin)
