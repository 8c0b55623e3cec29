"""MI355X (gfx950) batched speculative-decoding verify: greedy, chain rejection sampling
and target-only token-tree walk, as hand-written HIP kernels behind a C ABI
(include/spec_verify.h).  ``api`` holds the torch-facing binding with the C names."""
from . import _lib  # noqa: F401
from ._lib import (SPEC_BF16, SPEC_F32, SPEC_TREE_GREEDY, SPEC_TREE_SAMPLING,  # noqa: F401
                   SpecVerifyError)

__all__ = ["api", "workloads", "SPEC_F32", "SPEC_BF16", "SPEC_TREE_GREEDY",
           "SPEC_TREE_SAMPLING", "SpecVerifyError"]


def __getattr__(name):
    if name in ("api", "workloads", "build"):
        import importlib
        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)
