"""Seeded random shapes and launch options: the HIP path against the oracle.

Each case draws its shape (batch, draft length or tree size and depth, a vocabulary
between 1 and 60000 tokens, log-uniform), dtype, temperature, logit spread and launch
options (walk or eager path, cluster width, split count, row loads) from a generator
seeded with the case number, builds the inputs with the workload generators, and holds
every output to the bar of test_gpu_parity.compare: bit-exact outside the near-tie band,
near-ties counted and bounded, and every near-tie that differs reached by the oracle with
a coin nudged by a rounding-sized amount.  A second set draws from the edges of the
input space (near-uniform bf16 rows full of ties, nearly one-hot rows, very low and high
temperatures, drafts equal to the target, coins next to 1 or at 2^-24, extreme tree
thresholds).  The shapes are small, so the file runs in seconds; the cases are fixed by
their seeds, so a failure names its case and repeats.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
from lossless_rejection_sampling_verify_amd import workloads as wl

from test_gpu_parity import (check_chain, check_greedy, check_tree, launch,  # noqa: F401
                             say)
from test_gpu_mss import check_mss
from test_gpu_filtered import check as check_filtered

# SPEC_RANDOM_SCALE=k runs k times as many cases per test (new seeds, new shapes); 1 by
# default.
_SCALE = max(1, int(os.environ.get("SPEC_RANDOM_SCALE", "1")))

pytestmark = pytest.mark.gpu

SEED = 20261203


def _rng(kind: str, i: int) -> np.random.Generator:
    return np.random.default_rng([SEED, sum(map(ord, kind)), i])


def _vocab(rng, hi=60000) -> int:
    return int(np.exp(rng.uniform(0.0, np.log(hi))))


def _dtype(rng) -> str:
    return wl.BF16 if rng.random() < 0.6 else wl.F32


def _chain_opts(rng) -> dict:
    """One launch configuration: the default walk, a given cluster width, streaming row
    loads, or the eager passes with a given split count."""
    pick = int(rng.integers(0, 4))
    if pick == 0:
        return {}
    if pick == 1:
        return {"cluster": int(rng.choice([1, 2, 3, 5, 7, 16]))}
    if pick == 2:
        return {"row_loads": "streaming"}
    return {"path": "eager", "splits": int(rng.choice([1, 3, 8, 64]))}


@pytest.mark.parametrize("i", range(16 * _SCALE))
def test_random_chain_and_greedy(i, launch):
    rng = _rng("chain", i)
    B, G, V = int(rng.integers(1, 49)), int(rng.integers(1, 11)), _vocab(rng)
    dtype, T = _dtype(rng), float(rng.uniform(0.25, 2.5))
    sigma, dv = float(rng.uniform(0.5, 4.0)), float(rng.uniform(0.05, 3.0))
    opts = _chain_opts(rng)
    launch.update(opts)
    c = wl.make_chain(2, seed=i, B=B, G=G, V=V, dtype=dtype, T=T, sigma=sigma, draft_var=dv,
                      boost=None)
    label = f"random chain {i}: B={B} G={G} V={V} {dtype} T={T:.2f} {opts}"
    say(label)
    check_chain(c, label)
    check_greedy(c, label.replace("chain", "greedy", 1))


@pytest.mark.parametrize("i", range(12 * _SCALE))
def test_random_tree(i, launch):
    rng = _rng("tree", i)
    B, N = int(rng.integers(1, 17)), int(rng.integers(1, 81))
    D = int(rng.integers(1, max(min(N - 1, 12), 1) + 1))  # D >= 1 (a root alone: D = 1)
    kids = int(rng.integers(2, 9))
    V, dtype = _vocab(rng, 40000), _dtype(rng)
    T, sigma = float(rng.uniform(0.3, 2.0)), float(rng.uniform(0.5, 5.0))
    th_single = float(rng.choice([1.0, 0.5, 0.1]))
    th_acc = float(rng.choice([1.0, 0.7, 1.5]))
    if rng.random() < 0.3:
        launch.update({"path": "eager"})
    elif rng.random() < 0.5:
        launch.update({"cluster": int(rng.choice([1, 2, 4, 16]))})
    try:
        t = wl.make_tree(4, seed=i, B=B, N=N, V=max(V, N), D=D, max_children=kids, dtype=dtype,
                         T=T, sigma=sigma)
    except ValueError:  # the tree shape cannot hold N nodes: a wider one can
        t = wl.make_tree(4, seed=i, B=B, N=N, V=max(V, N), D=D, max_children=N, dtype=dtype,
                         T=T, sigma=sigma)
    # With a vocabulary not much larger than the tree, the rejected children can cover
    # nearly all of it, and the final draw's residual mass is then itself near zero in
    # every such request: those margins are not a coin's distance to a threshold, so the
    # per-call bound on near-ties does not apply (each one that differs is still checked).
    max_near = B if t.V <= 2 * N else None
    for mode in (oracle.TREE_GREEDY, oracle.TREE_SAMPLING):
        label = (f"random tree {i} mode {mode}: B={B} N={N} D={D} V={t.V} {dtype} "
                 f"th={th_single},{th_acc} {dict(launch)}")
        check_tree(t, mode, label, max_near=max_near, th_single=th_single, th_acc=th_acc)


@pytest.mark.parametrize("i", range(8 * _SCALE))
def test_random_multi_step_tree(i, launch):
    rng = _rng("mss", i)
    B, N = int(rng.integers(1, 9)), int(rng.integers(1, 41))
    D = int(rng.integers(1, max(min(N - 1, 8), 1) + 1))  # D >= 1 (a root alone: D = 1)
    kids = int(rng.integers(2, 7))
    V, dtype = _vocab(rng, 20000), _dtype(rng)
    T, sigma = float(rng.uniform(0.3, 2.0)), float(rng.uniform(0.5, 4.0))
    dv = float(rng.uniform(0.05, 2.0))
    if rng.random() < 0.5:
        launch.update({"cluster": int(rng.choice([1, 2, 5, 16]))})
    try:
        t = wl.make_tree_mss(4, seed=i, B=B, N=N, V=max(V, N), D=D, max_children=kids,
                             dtype=dtype, T=T, sigma=sigma, draft_var=dv)
    except ValueError:
        t = wl.make_tree_mss(4, seed=i, B=B, N=N, V=max(V, N), D=D, max_children=N,
                             dtype=dtype, T=T, sigma=sigma, draft_var=dv)
    check_mss(t, f"random multi-step tree {i}: B={B} N={N} D={D} V={t.V} {dtype} {dict(launch)}")


@pytest.mark.parametrize("i", range(8 * _SCALE))
def test_random_filtered(i):
    rng = _rng("filtered", i)
    B, G, V = int(rng.integers(1, 25)), int(rng.integers(1, 7)), _vocab(rng)
    dtype, T = _dtype(rng), float(rng.uniform(0.3, 2.0))
    top_k = rng.choice([0, 1, 5, 50, 300, 5000], size=B).astype(np.int32)
    top_p = rng.choice([1.0, 0.95, 0.8, 0.3], size=B).astype(np.float32)
    c = wl.make_chain_logits(2, seed=i, B=B, G=G, V=V, dtype=dtype, T=T, top_k=top_k,
                             top_p=top_p)
    check_filtered(c, f"random filtered {i}: B={B} G={G} V={V} {dtype} T={T:.2f}")


@pytest.mark.parametrize("i", range(8 * _SCALE))
def test_random_filtered_extremes(i):
    """Filtered chains at the edges of the kept-token list that the final draw reads: top-k
    at 1, 2, 255 and 256 (the list's limit; ties on bf16 rows can push the kept set past
    it, and then the full draw runs), with or without top-p, drafts equal to the target
    (every residual near empty, the plain kept weights drawn instead) or perturbed by a
    rounding-sized amount, and coins pinned next to 1 or to 2^-24."""
    rng = _rng("filtered-extreme", i)
    B, G, V = int(rng.integers(1, 25)), int(rng.integers(1, 6)), _vocab(rng, 40000)
    V = max(V, 300)
    dtype, T = _dtype(rng), float(rng.choice([0.3, 1.0, 3.0]))
    top_k = rng.choice([1, 2, 255, 256], size=B).astype(np.int32)
    top_p = rng.choice([1.0, 0.99, 0.5], size=B).astype(np.float32)
    c = wl.make_chain_logits(2, seed=400 + i, B=B, G=G, V=V, dtype=dtype, T=T, top_k=top_k,
                             top_p=top_p)
    eps = float(rng.choice([0.0, 1e-3]))
    d = wl.logits_as_f32(c.logits[:, :G], dtype) + np.float32(eps) * rng.standard_normal(
        (B, G, V), dtype=np.float32)
    c.draft_logits[:] = wl.f32_to_bf16_bits(d) if dtype == wl.BF16 else d
    pin = rng.random(c.coins.shape) < 0.3
    c.coins[pin] = np.where(rng.random(int(pin.sum())) < 0.5, 1.0 - 2.0 ** -24,
                            2.0 ** -24).astype(np.float32)
    check_filtered(c, f"extreme filtered {i}: B={B} G={G} V={V} {dtype} T={T} eps={eps}")


@pytest.mark.parametrize("i", range(12 * _SCALE))
def test_random_chain_extremes(i, launch):
    """Chains at the edges of the input space: logits nearly equal (bf16 ties) or spread
    far apart at a low or high temperature (nearly one-hot rows, underflowing weights),
    drafts equal to the target (every residual empty: the fallback draw) or far from it,
    and coins pinned next to 1 or to 2^-24.  Such inputs put coins at the thresholds by
    construction (a draft equal to the target makes p/q one up to rounding), so the
    per-call bound on near-ties does not apply; every near-tie that differs is still
    checked against the oracle with the coin nudged.  (A coin of exactly 1 is avoided only
    because a nudge could not move it up.)"""
    rng = _rng("extreme", i)
    B, G, V = int(rng.integers(1, 33)), int(rng.integers(1, 9)), _vocab(rng, 40000)
    dtype = _dtype(rng)
    sigma = float(rng.choice([0.01, 0.3, 8.0, 15.0]))
    T = float(rng.choice([0.05, 0.2, 1.0, 5.0]))
    dv = float(rng.choice([0.0, 1e-4, 1.0, 10.0]))
    opts = _chain_opts(rng)
    launch.update(opts)
    c = wl.make_chain(2, seed=100 + i, B=B, G=G, V=V, dtype=dtype, T=T, sigma=sigma,
                      draft_var=dv, boost=None)
    pin = rng.random(c.coins.shape) < 0.2
    c.coins[pin] = np.where(rng.random(int(pin.sum())) < 0.5, 1.0 - 2.0 ** -24,
                            2.0 ** -24).astype(np.float32)
    label = (f"extreme chain {i}: B={B} G={G} V={V} {dtype} sigma={sigma} T={T} "
             f"draft_var={dv} {opts}")
    say(label)
    check_chain(c, label, max_near=B)
    check_greedy(c, label.replace("chain", "greedy", 1))


@pytest.mark.parametrize("i", range(8 * _SCALE))
def test_random_tree_extremes(i, launch):
    """Trees on nearly uniform (bf16 ties) or nearly one-hot rows, at a very low or high
    temperature, with extreme thresholds; near-ties by construction, as above."""
    rng = _rng("tree-extreme", i)
    B, N = int(rng.integers(1, 13)), int(rng.integers(2, 65))
    D = int(rng.integers(1, min(N - 1, 10) + 1))
    V, dtype = _vocab(rng, 30000), _dtype(rng)
    sigma = float(rng.choice([0.01, 0.3, 10.0]))
    T = float(rng.choice([0.05, 1.0, 5.0]))
    th_single = float(rng.choice([1.0, 1e-3, 0.99]))
    th_acc = float(rng.choice([1.0, 0.05, 3.0]))
    if rng.random() < 0.3:
        launch.update({"path": "eager"})
    try:
        t = wl.make_tree(4, seed=200 + i, B=B, N=N, V=max(V, N), D=D,
                         max_children=int(rng.integers(2, 9)), dtype=dtype, T=T, sigma=sigma)
    except ValueError:
        t = wl.make_tree(4, seed=200 + i, B=B, N=N, V=max(V, N), D=D, max_children=N,
                         dtype=dtype, T=T, sigma=sigma)
    for mode in (oracle.TREE_GREEDY, oracle.TREE_SAMPLING):
        label = (f"extreme tree {i} mode {mode}: B={B} N={N} D={D} V={t.V} {dtype} "
                 f"sigma={sigma} T={T} th={th_single},{th_acc} {dict(launch)}")
        check_tree(t, mode, label, max_near=B, th_single=th_single, th_acc=th_acc)


@pytest.mark.parametrize("i", range(6 * _SCALE))
def test_random_multi_step_tree_extremes(i, launch):
    """Multi-step trees whose draft rows equal the target (every child accepted, up to
    rounding) or are far from it, on peaked or flat rows."""
    rng = _rng("mss-extreme", i)
    B, N = int(rng.integers(1, 7)), int(rng.integers(2, 33))
    D = int(rng.integers(1, min(N - 1, 8) + 1))
    V, dtype = _vocab(rng, 8000), _dtype(rng)
    sigma = float(rng.choice([0.01, 0.3, 10.0]))
    T = float(rng.choice([0.1, 1.0, 4.0]))
    dv = float(rng.choice([0.0, 1e-3, 8.0]))
    try:
        t = wl.make_tree_mss(4, seed=300 + i, B=B, N=N, V=max(V, N), D=D,
                             max_children=int(rng.integers(2, 7)), dtype=dtype, T=T,
                             sigma=sigma, draft_var=dv)
    except ValueError:
        t = wl.make_tree_mss(4, seed=300 + i, B=B, N=N, V=max(V, N), D=D, max_children=N,
                             dtype=dtype, T=T, sigma=sigma, draft_var=dv)
    label = f"extreme multi-step tree {i}: B={B} N={N} D={D} V={t.V} {dtype} sigma={sigma} T={T} dv={dv}"
    say(label)
    from test_gpu_mss import gpu_mss, mss_recheck, oracle_mss
    from test_gpu_parity import compare
    g, o = gpu_mss(t), oracle_mss(t)
    compare(g, o, ["accept_len", "out_tokens", "accepted_nodes"], o["margin"], label=label,
            max_near=B, recheck=mss_recheck(t, g))
