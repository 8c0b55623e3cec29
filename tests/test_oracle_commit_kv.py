"""Pins of the oracle's accepted-path KV commit for token trees (CPU only).

llm-infra-atlas "Speculative Decoding": the tree chapter covers how a token tree's KV is
laid out and rolled back after a rejection, and the serving section names rolling back
the KV of rejected drafts as a cost speculation adds; spec_origins, SpecInfer: one verify
forward computes every node of the flattened tree over one shared KV.

The property that fixes the layout: a KV row depends on the whole token prefix before
it.  So after a tree verify, the committed rows must be exactly the rows sequential
decoding of the emitted tokens would have written, in that order.  The tests build tree
KV from a toy prefix-dependent KV function, run the oracle's tree verify, commit, and
compare with the rows of the emitted prefix decoded alone.
"""
from __future__ import annotations

import hashlib

import numpy as np
import pytest

import oracle
from lossless_rejection_sampling_verify_amd import workloads as wl

ROW = 48  # bytes per KV row in these tests


def kv_of_prefix(tokens):
    """Toy KV row of the last position of a token prefix: depends on every token."""
    h = hashlib.sha256(np.asarray(tokens, np.int64).tobytes()).digest()
    return np.frombuffer((h * 2)[:ROW], np.uint8)


def tree_kv(t, root_token=12345):
    """kv_tree [B][N][ROW]: node j's row is the KV of (root, tokens on the path to j)."""
    kv = np.empty((t.B, t.N, ROW), np.uint8)
    for b in range(t.B):
        for j in range(t.N):
            path = []
            k = j
            while k > 0:
                path.append(int(t.node_tokens[b, k]))
                k = int(t.parents[b, k])
            kv[b, j] = kv_of_prefix([root_token] + path[::-1])
    return kv


@pytest.mark.parametrize("mode,seed", [(oracle.TREE_SAMPLING, 0), (oracle.TREE_SAMPLING, 1),
                                       (oracle.TREE_GREEDY, 2)])
def test_committed_rows_equal_sequential_decode_of_the_emitted_prefix(mode, seed):
    t = wl.make_tree(4, seed=seed, B=24, N=40, V=64, D=6, sigma=4.0, T=0.6)
    o = oracle.verify_tree(t.logits, t.dtype, t.node_tokens, t.parents, t.coins, t.temperature,
                           t.D, mode)
    kv = tree_kv(t)
    out = np.full((t.B, t.D + 1, ROW), 0xAB, np.uint8)
    slots = oracle.tree_commit_kv(o["accepted_nodes"], o["accept_len"], kv, out)
    assert (o["accept_len"] >= 1).any(), "every walk stopped at the root"
    for b in range(t.B):
        k = int(o["accept_len"][b])
        emitted = [12345] + o["out_tokens"][b, :k].tolist()
        for d in range(k + 1):
            np.testing.assert_array_equal(out[b, d], kv_of_prefix(emitted[: d + 1]))
        assert (out[b, k + 1:] == 0xAB).all()             # rows past the path untouched
        assert slots[b, 0] == 0
        assert slots[b, 1: k + 1].tolist() == o["accepted_nodes"][b, :k].tolist()
        assert (slots[b, k + 1:] == -1).all()


def test_chain_shaped_tree_commits_in_place_order():
    """A chain-shaped tree's accepted path is nodes 0..k, so the commit is the identity."""
    B, N, D = 3, 6, 5
    kv = np.random.default_rng(0).integers(0, 256, (B, N, ROW), dtype=np.uint8)
    nodes = np.tile(np.arange(1, D + 1, dtype=np.int32), (B, 1))
    acc = np.array([0, 2, 5], np.int32)
    out = np.zeros((B, D + 1, ROW), np.uint8)
    oracle.tree_commit_kv(nodes, acc, kv, out)
    for b in range(B):
        np.testing.assert_array_equal(out[b, : acc[b] + 1], kv[b, : acc[b] + 1])
        assert not out[b, acc[b] + 1:].any()


def test_invalid_requests_copy_nothing():
    B, N, D = 4, 10, 3
    kv = np.full((B, N, ROW), 7, np.uint8)
    nodes = np.array([[1, 2, 3], [1, 10, 2], [1, 2, 3], [4, 5, 6]], np.int32)
    acc = np.array([-1, 2, 4, 3], np.int32)
    out = np.zeros((B, D + 1, ROW), np.uint8)
    slots = oracle.tree_commit_kv(nodes, acc, kv, out)
    for b in (0, 1, 2):  # invalid: accept_len -1, node out of range, accept_len > D
        assert not out[b].any() and (slots[b] == -1).all()
    assert (out[3] == 7).all() and slots[3].tolist() == [0, 4, 5, 6]
