"""The C ABI used from plain C: lossless_rejection_sampling_verify_amd/abi_demo (built from
csrc/abi_demo.c by the package build) allocates its own device buffers, zeroes the
workspaces once, and calls spec_verify_greedy and spec_verify_chain.  Its outputs must
match the oracle on the same inputs."""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

import oracle
from lossless_rejection_sampling_verify_amd import workloads as wl

from test_gpu_parity import compare, say

pytestmark = pytest.mark.gpu

DEMO = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "lossless_rejection_sampling_verify_amd", "abi_demo")


@pytest.mark.parametrize("B,G,V", [(6, 3, 3001), (33, 5, 32000)])
def test_plain_c_consumer(tmp_path, B, G, V):
    assert os.path.exists(DEMO), f"{DEMO} is missing: build the package first"
    c = wl.make_chain(2, seed=B + V, B=B, G=G, V=V, dtype=wl.F32)
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        np.array([B, G, V], np.int32).tofile(f)
        for a, dt in ((c.logits, np.float32), (c.draft_probs, np.float32),
                      (c.greedy_tokens, np.int32), (c.draft_tokens, np.int32),
                      (c.coins, np.float32), (c.temperature, np.float32)):
            np.ascontiguousarray(a, dtype=dt).tofile(f)
    say(f"plain C consumer B={B} G={G} V={V}")
    subprocess.run([DEMO, str(inp), str(out)], check=True, timeout=120)
    raw = np.fromfile(out, np.int32)
    R = G + 1
    n = [B, B * R, B, B * R, B * R]
    parts = np.split(raw, np.cumsum(n)[:-1])
    acc_g, out_g, acc_c, out_c = parts[0], parts[1].reshape(B, R), parts[2], parts[3].reshape(B, R)
    probs = parts[4].view(np.float32).reshape(B, R)
    oa, oo = oracle.verify_greedy(c.logits, c.dtype, c.greedy_tokens)
    np.testing.assert_array_equal(acc_g, oa)
    np.testing.assert_array_equal(out_g, oo)
    o = oracle.verify_chain(c.logits, c.dtype, c.draft_probs, c.draft_tokens, c.coins,
                            c.temperature)
    compare(dict(accept_len=acc_c, out_tokens=out_c, probs=probs), o,
            ["accept_len", "out_tokens"], o["margin"], label=f"C consumer B={B}")
