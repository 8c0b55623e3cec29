"""ctypes loader of the HIP library ``libspecverify.so`` (argument marshalling only).

The library must have been built (``python -m lossless_rejection_sampling_verify_amd.build``
or ``__graft_entry__.build()``); there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspecverify.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "spec_verify.h")

SPEC_OK, SPEC_ERR_NULL, SPEC_ERR_SHAPE, SPEC_ERR_DTYPE = 0, -1, -2, -3
SPEC_ERR_PARAM, SPEC_ERR_WORKSPACE, SPEC_ERR_HIP, SPEC_ERR_TOO_LARGE = -4, -5, -6, -7
SPEC_F32, SPEC_BF16 = 0, 1
SPEC_TREE_GREEDY, SPEC_TREE_SAMPLING = 0, 1
SPEC_OP_GREEDY, SPEC_OP_CHAIN, SPEC_OP_TREE, SPEC_OP_CHAIN_FILTERED, SPEC_OP_TREE_MSS = 0, 1, 2, 3, 4
SPEC_MAX_G, SPEC_MAX_N = 64, 1024
SPEC_ROW_INVALID, SPEC_ROW_RETRY = -1, -2
SPEC_PATH_WALK, SPEC_PATH_EAGER = 0, 1
SPEC_LOADS_DEFAULT, SPEC_LOADS_CACHED, SPEC_LOADS_STREAMING = 0, 1, 2


class SpecOptions(ctypes.Structure):
    """struct spec_options of include/spec_verify.h (every field 0: the defaults)."""
    _fields_ = [("path", ctypes.c_int), ("cluster", ctypes.c_int), ("splits", ctypes.c_int),
                ("row_loads", ctypes.c_int), ("spin_limit", ctypes.c_int)]


def options(opts) -> "SpecOptions | None":
    """A SpecOptions from None, a SpecOptions, or a dict of its fields (path may be
    'walk' / 'eager'; row_loads may be 'cached' / 'streaming')."""
    if opts is None or isinstance(opts, SpecOptions):
        return opts
    d = dict(opts)
    unknown = set(d) - {f for f, _ in SpecOptions._fields_}
    if unknown:
        raise ValueError(f"unknown option(s) {sorted(unknown)}")
    if isinstance(d.get("path"), str):
        d["path"] = {"walk": SPEC_PATH_WALK, "eager": SPEC_PATH_EAGER}[d["path"]]
    if isinstance(d.get("row_loads"), str):
        d["row_loads"] = {"default": SPEC_LOADS_DEFAULT, "cached": SPEC_LOADS_CACHED,
                          "streaming": SPEC_LOADS_STREAMING}[d["row_loads"]]
    return SpecOptions(**{k: int(v) for k, v in d.items()})

_lib = None


class SpecVerifyError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_str(status)} ({status})")
        self.status = status


def declared_functions() -> list[str]:
    """Names of the functions include/spec_verify.h declares."""
    text = open(HEADER).read()
    return re.findall(r"^\s*(?:size_t|int|const char\*)\s+(spec_\w+)\s*\(", text, re.M)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        vp, ip, fp, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.spec_workspace_bytes.argtypes = [ip, ip, ip, ip]
        L.spec_workspace_bytes.restype = sz
        L.spec_status_str.argtypes = [ip]
        L.spec_status_str.restype = ctypes.c_char_p
        op = ctypes.POINTER(SpecOptions)
        L.spec_verify_greedy.argtypes = [vp, ip, vp, ip, ip, ip, vp, vp, vp, sz, vp]
        L.spec_verify_greedy.restype = ip
        L.spec_verify_greedy_opt.argtypes = L.spec_verify_greedy.argtypes + [op]
        L.spec_verify_greedy_opt.restype = ip
        L.spec_verify_chain.argtypes = [vp, ip, vp, vp, vp, vp, ip, ip, ip, vp, vp, vp, vp, sz, vp]
        L.spec_verify_chain.restype = ip
        L.spec_verify_chain_opt.argtypes = L.spec_verify_chain.argtypes + [op]
        L.spec_verify_chain_opt.restype = ip
        L.spec_verify_chain_noalloc.argtypes = [vp, ip, vp, vp, vp, vp, ip, ip, ip, vp, vp, vp,
                                                vp]
        L.spec_verify_chain_noalloc.restype = ip
        L.spec_verify_tree.argtypes = [vp, ip, vp, vp, vp, vp, ip, ip, ip, ip, ip, fp, fp,
                                       vp, vp, vp, vp, vp, sz, vp]
        L.spec_verify_tree.restype = ip
        L.spec_verify_tree_opt.argtypes = L.spec_verify_tree.argtypes + [op]
        L.spec_verify_tree_opt.restype = ip
        L.spec_verify_chain_filtered.argtypes = [vp, vp, ip, vp, vp, vp, vp, vp, ip, ip, ip, vp, vp,
                                                 vp, vp, sz, vp]
        L.spec_verify_chain_filtered.restype = ip
        L.spec_verify_tree_mss.argtypes = [vp, ip, vp, vp, vp, vp, vp, ip, ip, ip, ip, vp, vp, vp,
                                           vp, vp, sz, vp]
        L.spec_verify_tree_mss.restype = ip
        L.spec_verify_tree_mss_opt.argtypes = L.spec_verify_tree_mss.argtypes + [op]
        L.spec_verify_tree_mss_opt.restype = ip
        L.spec_tree_mask.argtypes = [vp, vp, ip, ip, vp, vp, vp]
        L.spec_tree_mask.restype = ip
        L.spec_tree_commit_kv.argtypes = [vp, vp, ip, ip, ip, vp, vp, sz, vp, vp]
        L.spec_tree_commit_kv.restype = ip
        L.spec_calib_read.argtypes = [vp, sz, vp, vp]
        L.spec_calib_read.restype = ip
        L.spec_calib_exp.argtypes = [ip, ip, vp, vp]
        L.spec_calib_exp.restype = ip
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().spec_status_str(int(status)).decode()


def workspace_bytes(op: int, B: int, R: int, V: int) -> int:
    return int(lib().spec_workspace_bytes(op, B, R, V))
