"""Resources of the walk kernels, read from the built library's gfx950 code object.

The walks size their clusters from how many workgroups the device holds at once, and
their speed depends on code the compiler may quietly change: a kernel that spills, grows
past a residency step, or gains LDS it does not declare runs slower with no change in its
results.  Each walk is held to
  - no scratch (no spills, no private arrays left in memory);
  - an LDS budget: the shared structures it declares, with under 1 KB of slack.  A private array
    that the compiler moves into LDS shows up here (a 12-byte draw state copied whole left
    3 KB of LDS in the tree walk and cost tree sampling 10 us, with residency unchanged);
  - a register limit for the residency its clusters are sized for, with one 256-lane
    workgroup per CU putting one wave on each SIMD: 512 VGPRs per SIMD lane slot give
    four waves at up to 128 and five at up to 96 (granules of 8).  The greedy walk runs
    five workgroups per CU, the chain and tree walks four, the multi-step walk three; the
    filtered calls' row kernel (not a walk) keeps five for its two rounds of rows.

No other kernel of the library may use scratch either.

The metadata is read with the ROCm LLVM tools from the library built here (the code-object
notes that the loader itself reads); the test skips when the library or a tool is missing.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from lossless_rejection_sampling_verify_amd import _lib as L

LLVM = "/opt/rocm/llvm/bin"
TOOLS = ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf")
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"

# kernel name fragment -> (LDS budget in bytes, max VGPRs + AGPRs)
LIMITS = {
    "k_greedy_walk": (1 * 1024, 96),
    "k_chain_walk": (35 * 1024, 128),  # with the chunk masses kept in LDS for the draw
    "k_tree_walk": (37 * 1024 + 512, 128),
    "k_mss_walk": (49 * 1024, 168),
    "k_filter_rows": (29 * 1024, 96),  # one row per workgroup, five per CU
}


def _kernels(tmp_path) -> dict:
    if not os.path.exists(L.LIB_PATH):
        pytest.skip(f"{L.LIB_PATH} is not built")
    for t in TOOLS:
        if not os.access(os.path.join(LLVM, t), os.X_OK):
            pytest.skip(f"{t} is not available")
    fb, co = tmp_path / "fb.bin", tmp_path / "co.o"
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fb}",
                    L.LIB_PATH, str(tmp_path / "lib.so")], check=True)
    subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--type=o",
                    f"--targets={TARGET}", f"--input={fb}", f"--output={co}", "--unbundle"],
                   check=True)
    notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", str(co)], check=True,
                           capture_output=True, text=True).stdout
    out = {}
    for blk in notes.split("  - .agpr_count:")[1:]:
        def field(key):
            m = re.search(rf"^\s+\.{key}:\s+(\S+)", blk, re.M)
            return m.group(1) if m else None
        name = field("name")
        if name is None:
            continue
        out[name] = {"lds": int(field("group_segment_fixed_size")),
                     "scratch": int(field("private_segment_fixed_size")),
                     "vgpr": int(field("vgpr_count")), "agpr": int(blk.split("\n", 1)[0])}
    return out


def test_walk_kernels_keep_their_budgets(tmp_path):
    ks = _kernels(tmp_path)
    seen = set()
    for name, r in ks.items():
        for frag, (lds_max, vgpr_max) in LIMITS.items():
            if frag not in name:
                continue
            seen.add(frag)
            what = f"{name}: {r}"
            assert r["scratch"] == 0, f"spills to scratch: {what}"
            assert r["lds"] <= lds_max, f"LDS above its {lds_max}-byte budget: {what}"
            assert r["vgpr"] + r["agpr"] <= vgpr_max, f"registers above {vgpr_max}: {what}"
    assert seen == set(LIMITS), f"walk kernels not found in the code object: {set(LIMITS) - seen}"


def test_no_kernel_uses_scratch(tmp_path):
    """No kernel of the library keeps anything in private (scratch) memory: a spill or a
    private array there costs a memory round trip per access."""
    ks = _kernels(tmp_path)
    assert ks
    bad = {n: r for n, r in ks.items() if r["scratch"] != 0}
    assert not bad, f"kernels with scratch: {bad}"
