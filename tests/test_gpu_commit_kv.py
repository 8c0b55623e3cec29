"""spec_tree_commit_kv (HIP) vs the oracle's accepted-path KV commit, byte for byte.

Covers the pipeline tree verify -> commit on the tree workload's shape, row sizes on
both sides of the vector path (16-byte multiples) and of the 16 KB chunk, a 128 KiB row,
rows past the path left untouched, slots, and invalid requests.
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


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_both(nodes, acc, kv, label):
    api = _api()
    B, D = nodes.shape
    row = kv.shape[2]
    print(f"[gpu-case] commit kv {label} B={B} D={D} N={kv.shape[1]} row={row}", flush=True)
    sentinel = np.random.default_rng(B * 7 + row).integers(0, 256, (B, D + 1, row), dtype=np.uint8)
    want = sentinel.copy()
    want_slots = oracle.tree_commit_kv(nodes, acc, kv, want)
    out = dev(sentinel)
    slots = api.spec_tree_commit_kv(dev(nodes.astype(np.int32)), dev(acc.astype(np.int32)),
                                    dev(kv), out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), want, err_msg=label)
    np.testing.assert_array_equal(slots.cpu().numpy(), want_slots, err_msg=label)


def test_after_gpu_tree_verify_on_the_tree_workload_shape():
    api = _api()
    t = wl.make_tree(4, seed=2, V=20000, sigma=6.0, T=0.5)
    lg = torch.from_numpy(np.ascontiguousarray(t.logits).view(np.int16)).view(torch.bfloat16).cuda()
    acc, _, nodes, _ = api.spec_verify_tree(lg, dev(t.node_tokens), dev(t.parents), dev(t.coins),
                                            dev(t.temperature), t.D, api.L.SPEC_TREE_SAMPLING)
    torch.cuda.synchronize()
    acc, nodes = acc.cpu().numpy(), nodes.cpu().numpy()
    assert acc.max() >= 1
    kv = np.random.default_rng(0).integers(0, 256, (t.B, t.N, 4096), dtype=np.uint8)
    run_both(nodes, acc, kv, "after tree verify")


@pytest.mark.parametrize("row", [16, 48, 100, 16384, 16400, 131072])
def test_row_sizes(row):
    rng = np.random.default_rng(row)
    B, N, D = 9, 30, 5
    nodes = np.stack([np.sort(rng.choice(np.arange(1, N), D, replace=False)) for _ in range(B)])
    acc = rng.integers(0, D + 1, B).astype(np.int32)
    kv = rng.integers(0, 256, (B, N, row), dtype=np.uint8)
    run_both(nodes.astype(np.int32), acc, kv, f"row={row}")


def test_invalid_requests():
    rng = np.random.default_rng(3)
    B, N, D = 6, 12, 4
    nodes = np.tile(np.array([1, 3, 5, 7], np.int32), (B, 1))
    nodes[2, 1] = 12
    nodes[3, 0] = -5
    acc = np.array([-1, 4, 2, 3, 5, 0], np.int32)
    kv = rng.integers(0, 256, (B, N, 64), dtype=np.uint8)
    run_both(nodes, acc, kv, "invalid")
