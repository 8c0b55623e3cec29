"""Pins of the oracle's chain verify from draft logits with top-k / top-p filtering (CPU).

ricardokevins "Speculative Decoding": serving samples with temperature, top-p and top-k,
and correction sampling keeps the target's law only when acceptance and residual use
the distributions actually sampled from.  Reading: target and draft rows are filtered
alike (top-k keeps ties at the k-th logit; top-p, on the top-k-filtered row, keeps every
token at least as probable as the end of the shortest head reaching top_p of the mass),
renormalised, then verified by the usual rule.

Pins: with no filter the result is the unfiltered chain verify with q = softmax(d/T)
(another code path); top-k = 1 turns it into greedy verify (another code path); the exact
law over coins and drafts equals the filtered target row computed here by sorting;
hand-worked golden cases; invalid knobs.
"""
from __future__ import annotations

import itertools
import json
import os

import numpy as np
import pytest

import lawengine as le
import oracle
from lossless_rejection_sampling_verify_amd import workloads as wl

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "filtered_cases.json")))
BAND = 1e-6


def softmax64(x, T):
    z = np.asarray(x, np.float64) / T
    z = z - z.max(-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(-1, keepdims=True)


def filtered(row, T, k, top_p):
    """The filtered distribution of one logit row, by sorting (the reading in words)."""
    row = np.asarray(row, np.float64)
    p = softmax64(row, T)
    keep = np.ones(len(row), bool)
    if 0 < k < len(row):
        keep &= row >= np.sort(row)[::-1][k - 1]
    p = np.where(keep, p, 0.0)
    if top_p < 1.0:
        order = np.sort(p)[::-1]
        cum = np.cumsum(order)
        tau = order[np.searchsorted(cum, top_p * p.sum())]
        p = np.where(p >= tau, p, 0.0)
    return p / p.sum()


def test_no_filter_equals_unfiltered_chain_on_softmax_q():
    c = wl.make_chain(2, seed=3, B=40, G=4, V=300)
    d = wl.logits_as_f32(c.logits[:, :4], c.dtype) + np.random.default_rng(1).standard_normal(
        (40, 4, 300)).astype(np.float32)
    q = softmax64(d, 1.0).astype(np.float32)
    f = oracle.verify_chain_filtered(c.logits, d, c.dtype, c.draft_tokens, c.coins, c.temperature)
    u = oracle.verify_chain(c.logits, c.dtype, q, c.draft_tokens, c.coins, c.temperature)
    far = (f["margin"] > 1e-5) & (u["margin"] > 1e-5)
    assert far.sum() > 30
    np.testing.assert_array_equal(f["accept_len"][far], u["accept_len"][far])
    np.testing.assert_array_equal(f["out_tokens"][far], u["out_tokens"][far])


def test_top1_is_greedy_verify():
    c = wl.make_chain(2, seed=4, B=64, G=4, V=500)
    rng = np.random.default_rng(2)
    d = wl.logits_as_f32(c.logits[:, :4], c.dtype) + rng.standard_normal((64, 4, 500)).astype(np.float32)
    x = np.argmax(d, -1).astype(np.int32)
    f = oracle.verify_chain_filtered(c.logits, d, c.dtype, x, c.coins, c.temperature,
                                     np.ones(64, np.int32), None)
    ga, go = oracle.verify_greedy(c.logits, c.dtype, x)
    np.testing.assert_array_equal(f["accept_len"], ga)
    np.testing.assert_array_equal(f["out_tokens"], go)


@pytest.mark.parametrize("seed,k,top_p,T", [(0, 3, 1.0, 1.0), (1, 0, 0.6, 1.0), (2, 4, 0.8, 0.7)])
def test_filtered_round_emits_filtered_target_law(seed, k, top_p, T):
    """Exact over coins and drafts x_i ~ filtered q_i: every emitted token follows the
    filtered target row (the losslessness of the filtered verify)."""
    rng = np.random.default_rng(seed)
    V, G = 5, 2
    logits = (rng.standard_normal((G + 1, V)) * 1.5).astype(np.float32)
    dlog = (logits[:G] + rng.standard_normal((G, V))).astype(np.float32)
    p = np.stack([filtered(r, T, k, top_p) for r in logits])
    q = np.stack([filtered(r, T, k, top_p) for r in dlog])
    runner = le.filtered_runner(k, top_p)
    law = {}
    for x in itertools.product(range(V), repeat=G):
        wx = float(np.prod([q[i, x[i]] for i in range(G)]))
        if wx == 0.0:
            continue
        for out, pr in le.chain_round_law(logits, "f32", dlog, list(x), T, runner).items():
            law[out] = law.get(out, 0.0) + wx * pr
    assert abs(sum(law.values()) - 1.0) < 1e-6
    first = np.zeros(V)
    for out, pr in law.items():
        first[out[1]] += pr
    np.testing.assert_allclose(first, p[0], atol=2e-6)
    for j in range(1, G + 1):
        cond = {}
        for out, pr in law.items():
            if out[0] + 1 > j:
                cond.setdefault(out[1: 1 + j], np.zeros(V))[out[1 + j]] += pr
        for prefix, dist in cond.items():
            if dist.sum() < 1e-3:
                continue
            np.testing.assert_allclose(dist / dist.sum(), p[j], atol=8e-6 / dist.sum())


@pytest.mark.parametrize("case", GOLDEN["cases"], ids=[c["name"] for c in GOLDEN["cases"]])
def test_golden(case):
    lg = np.array(case["logits"], np.float32)[None]
    dl = np.array(case["draft_logits"], np.float32)[None]
    o = oracle.verify_chain_filtered(lg, dl, "f32", np.array([case["x"]], np.int32),
                                     np.array([case["coins"]], np.float32),
                                     np.array([case["T"]], np.float32),
                                     np.array([case["top_k"]], np.int32),
                                     np.array([case["top_p"]], np.float32))
    assert o["accept_len"][0] == case["accept_len"]
    assert o["out_tokens"][0].tolist() == case["out_tokens"]


def test_knob_edges():
    c = wl.make_chain(2, seed=5, B=6, G=3, V=200)
    d = wl.logits_as_f32(c.logits[:, :3], c.dtype) * 0.5
    base = oracle.verify_chain_filtered(c.logits, d, c.dtype, c.draft_tokens, c.coins, c.temperature)
    off = oracle.verify_chain_filtered(c.logits, d, c.dtype, c.draft_tokens, c.coins, c.temperature,
                                       np.array([0, -3, 200, 500, 0, 0], np.int32),
                                       np.array([1.0, 1.0, 1.0, 1.0, 2.0, 1.0], np.float32))
    np.testing.assert_array_equal(base["out_tokens"], off["out_tokens"])
    bad = oracle.verify_chain_filtered(c.logits, d, c.dtype, c.draft_tokens, c.coins, c.temperature,
                                       None, np.array([0.0, -0.5, np.nan, 0.5, 1.0, 1.0], np.float32))
    assert (bad["accept_len"][:3] == -1).all() and (bad["accept_len"][3:] >= 0).all()


def test_signed_zeros_tie_at_the_top_k_boundary():
    """-0.0 and +0.0 are the same logit: with the k-th largest logit at zero, every zero is
    kept whatever its sign, so the filtered row is uniform over them.  A draft on the -0.0
    token (q uniform over the same three zeros) is then accepted at any coin, and the
    bonus token is drawn uniformly from the three zeros (coins at thirds)."""
    row = np.array([-1.0, 0.0, -0.0, -2.0, 0.0, -3.0], np.float32)
    assert np.signbit(row[2])
    lg = np.broadcast_to(row, (3, 2, 6)).copy()
    dl = np.broadcast_to(row, (3, 1, 6)).copy()
    x = np.array([[2], [2], [2]], np.int32)
    coins = np.array([[0.999, 0.2], [0.999, 0.5], [0.999, 0.9]], np.float32)
    o = oracle.verify_chain_filtered(lg, dl, wl.F32, x, coins, np.ones(3, np.float32),
                                     top_k=np.full(3, 2, np.int32), top_p=np.ones(3, np.float32))
    assert (o["accept_len"] == 1).all()
    # inverse CDF over the kept zeros in ascending id: tokens 1, 2, 4 at thirds
    assert o["out_tokens"][:, 1].tolist() == [1, 2, 4]
    np.testing.assert_allclose(o["probs"][:, 0], 1.0 / 3.0, rtol=1e-6)
