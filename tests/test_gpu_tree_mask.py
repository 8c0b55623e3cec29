"""spec_tree_mask (HIP) vs the oracle's tree attention mask, bit for bit.

Covers the tree workload's shape (B=32, N=64, depth 6, <= 8 children), mask widths on
both sides of every 32-bit word boundary, rows kept in LDS (N <= 512) and rows built in
the output buffer (N > 512), depth-1023 chains, stars, malformed parent arrays, and the
optional base positions and position output.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from lossless_rejection_sampling_verify_amd import workloads as wl

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_rejection_sampling_verify_amd import api
    return api


def gpu_mask(parents, base_pos=None, want_positions=True):
    api = _api()
    p = torch.from_numpy(np.ascontiguousarray(parents, dtype=np.int32)).cuda()
    bp = None if base_pos is None else torch.from_numpy(np.ascontiguousarray(base_pos, dtype=np.int32)).cuda()
    mask, pos = api.spec_tree_mask(p, bp, want_positions=want_positions)
    torch.cuda.synchronize()
    return mask.cpu().numpy().view(np.uint32), None if pos is None else pos.cpu().numpy()


def check(parents, base_pos=None, label=""):
    print(f"[gpu-case] tree mask {label} B={parents.shape[0]} N={parents.shape[1]}", flush=True)
    gm, gp = gpu_mask(parents, base_pos)
    om, op = oracle.tree_mask(parents, base_pos)
    np.testing.assert_array_equal(gm, om, err_msg=label)
    np.testing.assert_array_equal(gp, op, err_msg=label)


def forest(seed, B, N, D, kids):
    rng = np.random.default_rng(seed)
    return np.stack([wl._random_tree(rng, N, D, kids) for _ in range(B)])


def test_tree_workload_shape():
    t = wl.make_tree(4)
    check(t.parents, np.arange(t.B, dtype=np.int32) * 1000, "workload 4")


@pytest.mark.parametrize("N", [1, 2, 31, 32, 33, 63, 64, 65, 200, 512, 513, 1000, 1024])
def test_sizes(N):
    D = max(1, min(N - 1, 12))
    check(forest(N, 6, N, D, 8 if N > 40 else 3), np.arange(6, dtype=np.int32) * 7, f"N={N}")


@pytest.mark.parametrize("N", [512, 1024])
def test_deep_chains_and_stars(N):
    chain = np.arange(-1, N - 1, dtype=np.int32)
    star = np.zeros(N, np.int32)
    star[0] = -1
    check(np.stack([chain, star, chain]), None, f"chain/star N={N}")


def test_malformed_and_optional_outputs():
    par = forest(9, 5, 40, 6, 4)
    par[1, 10] = 10
    par[3, 0] = 2
    check(par, np.full(5, 3, np.int32), "malformed")
    gm, gp = gpu_mask(par, None, want_positions=False)
    om, _ = oracle.tree_mask(par)
    assert gp is None
    np.testing.assert_array_equal(gm, om)
