"""Exact output laws of the oracle over the coin lattice, found by black-box search.

The coins the workloads draw are u = (k+1)/2^24, k uniform in [0, 2^24).  With every
other input fixed, the verify output as a function of one coin is a step function
whose pieces carry distinct values: an acceptance test flips once as u crosses its
threshold, an inverse-CDF draw moves through the tokens in ascending order, and a
sibling walk moves through the children in ascending order.  ``segments`` finds every
breakpoint of such a function with batched oracle calls (fan-out search), so the
probability of each outcome is an exact count of lattice points divided by 2^24.

Nothing here re-implements the verify rules: outcomes are read off the oracle, and the
tests compare the resulting laws with what the pages' mathematics fixes (the target
distribution, the closed form for E[#tokens], ...).
"""
from __future__ import annotations

import numpy as np

import oracle

LATTICE = 1 << 24


def coin(k) -> np.ndarray:
    return ((np.asarray(k, dtype=np.int64) + 1).astype(np.float64) / LATTICE).astype(np.float32)


def segments(eval_many, n: int = LATTICE, fan: int = 256):
    """All pieces of a step function f on the integer range [0, n).

    ``eval_many(ks)`` returns a list of hashable values f(k).  Pieces must carry
    pairwise-distinct values (so f(a) == f(b) implies f is constant on [a, b]).
    Returns [(start, stop, value)] covering [0, n) in order.
    """
    ends = eval_many(np.array([0, n - 1], dtype=np.int64))
    known = {0: ends[0], n - 1: ends[1]}
    todo = [(0, n - 1)] if ends[0] != ends[1] else []
    change = []                       # k such that f(k-1) != f(k)
    while todo:
        probes, spans = [], []
        for a, b in todo:
            if b - a == 1:
                change.append(b)
                continue
            pts = np.unique(np.linspace(a, b, min(fan, b - a + 1)).astype(np.int64))
            inner = [p for p in pts if p not in known]
            probes.extend(inner)
            spans.append((a, b, pts))
        if probes:
            vals = eval_many(np.array(probes, dtype=np.int64))
            for p, v in zip(probes, vals):
                known[int(p)] = v
        todo = []
        for a, b, pts in spans:
            for lo, hi in zip(pts[:-1], pts[1:]):
                if known[int(lo)] != known[int(hi)]:
                    todo.append((int(lo), int(hi)))
    change.sort()
    bounds = [0] + change + [n]
    return [(s, e, known[s] if s in known else eval_many(np.array([s]))[0])
            for s, e in zip(bounds[:-1], bounds[1:])]


# ---------------------------------------------------------------------------------------
# chain: one request, fixed rows

def _run_chain(lg, dtype, qq, xx, coin_sets, Ts):
    return oracle.verify_chain(lg, dtype, qq, xx, coin_sets, Ts)


def filtered_runner(top_k, top_p):
    """Runner for chain_outcomes / chain_round_law: q holds draft logits, and both rows
    are filtered with top_k / top_p by the oracle."""
    def run(lg, dtype, dl, xx, coin_sets, Ts):
        B = len(Ts)
        return oracle.verify_chain_filtered(lg, dl, dtype, xx, coin_sets, Ts,
                                            np.full(B, top_k, np.int32),
                                            np.full(B, top_p, np.float32))
    return run


def chain_outcomes(logits, dtype, q, x, T, coin_sets, runner=_run_chain):
    """Run the oracle on one request under many coin vectors; returns tuples
    (accept_len, emitted tokens...)."""
    coin_sets = np.asarray(coin_sets, dtype=np.float32)
    B = coin_sets.shape[0]
    G = len(x)
    lg = np.broadcast_to(logits, (B,) + logits.shape)
    qq = np.broadcast_to(q, (B,) + q.shape)
    xx = np.broadcast_to(np.asarray(x, np.int32), (B, G))
    res = runner(np.ascontiguousarray(lg), dtype, np.ascontiguousarray(qq),
                 np.ascontiguousarray(xx), coin_sets, np.full(B, T, np.float32))
    out = []
    for b in range(B):
        k = int(res["accept_len"][b])
        out.append((k,) + tuple(int(t) for t in res["out_tokens"][b, : k + 1]))
    return out


def chain_round_law(logits, dtype, q, x, T, runner=_run_chain):
    """Exact law of one chain verify with drafts x fixed, over lattice coins.

    Returns {(accept_len, tok_0, ..., tok_k): probability}.
    """
    G = len(x)
    R = G + 1
    base = coin(np.zeros(R, dtype=np.int64))
    law = {}
    mass = 1.0
    prefix_coins = base.copy()
    for i in range(G + 1):
        # outcome as a function of coin i with coins < i at the smallest lattice value
        # (which accepts whenever acceptance at that position is possible at all)
        if i < G:
            def f(ks, i=i):
                cs = np.repeat(prefix_coins[None, :], len(ks), axis=0)
                cs[:, i] = coin(ks)
                return [o[0] > i for o in chain_outcomes(logits, dtype, q, x, T, cs, runner)]
            segs = segments(f)
            acc_pts = sum(e - s for s, e, v in segs if v)
            rej_start = next((s for s, e, v in segs if not v), None)
            p_acc = acc_pts / LATTICE
        else:
            p_acc, rej_start = 0.0, None
        # where the walk stops at i: rejection at i < G, or the bonus at i = G
        stop_mass = mass * (1.0 - p_acc)
        if stop_mass > 0.0:
            stop_coins = prefix_coins.copy()
            if i < G:
                stop_coins[i] = coin(rej_start)

            def g(ks):
                cs = np.repeat(stop_coins[None, :], len(ks), axis=0)
                cs[:, G] = coin(ks)
                return chain_outcomes(logits, dtype, q, x, T, cs, runner)
            for s, e, v in segments(g):
                law[v] = law.get(v, 0.0) + stop_mass * (e - s) / LATTICE
        mass *= p_acc
        if mass == 0.0 or i == G:
            break
    return law


# ---------------------------------------------------------------------------------------
# tree: one request

def tree_outcomes(logits, dtype, tokens, parents, T, D, coin_sets, th_single=1.0, th_acc=1.0):
    coin_sets = np.asarray(coin_sets, dtype=np.float32)
    B = coin_sets.shape[0]
    N = len(parents)
    lg = np.ascontiguousarray(np.broadcast_to(logits, (B,) + logits.shape))
    tk = np.ascontiguousarray(np.broadcast_to(np.asarray(tokens, np.int32), (B, N)))
    pa = np.ascontiguousarray(np.broadcast_to(np.asarray(parents, np.int32), (B, N)))
    res = oracle.verify_tree(lg, dtype, tk, pa, coin_sets, np.full(B, T, np.float32), D,
                             oracle.TREE_SAMPLING, th_single, th_acc)
    out = []
    for b in range(B):
        k = int(res["accept_len"][b])
        out.append((k,) + tuple(int(t) for t in res["out_tokens"][b, : k + 1]) +
                   tuple(int(nd) for nd in res["accepted_nodes"][b, :k]))
    return out


def tree_law(logits, dtype, tokens, parents, T, D):
    """Exact law of the target-only tree walk over lattice coins.

    Returns {(accept_len, tok_0, ..., tok_k, node_0, ..., node_{k-1}): probability}.
    """
    law = {}

    def walk(level, fixed, mass):
        # outcome as a function of the coin of this level, later coins at their minimum
        def f(ks):
            cs = np.repeat(fixed[None, :], len(ks), axis=0)
            cs[:, level] = coin(ks)
            return [(o[0], o[1: 2 + level]) for o in tree_outcomes(logits, dtype, tokens,
                                                                  parents, T, D, cs)]
        if level < D:
            pieces = segments(f)
        else:
            pieces = [(0, LATTICE, None)]
        for s, e, v in pieces:
            pm = mass * (e - s) / LATTICE
            if pm == 0.0:
                continue
            cs = fixed.copy()
            cs[level] = coin(s)
            if level < D and v[0] > level:
                walk(level + 1, cs, pm)       # a child was accepted at this level
            else:
                def g(ks, cs=cs):
                    c2 = np.repeat(cs[None, :], len(ks), axis=0)
                    c2[:, D] = coin(ks)
                    return tree_outcomes(logits, dtype, tokens, parents, T, D, c2)
                for s2, e2, v2 in segments(g):
                    law[v2] = law.get(v2, 0.0) + pm * (e2 - s2) / LATTICE

    walk(0, coin(np.zeros(D + 1, dtype=np.int64)), 1.0)
    return law


# ---------------------------------------------------------------------------------------
# tree by multi-step speculative sampling: one coin per tested node, one final coin

def mss_outcomes(logits, dtype, q, tokens, parents, T, D, coin_sets):
    coin_sets = np.asarray(coin_sets, dtype=np.float32)
    B = coin_sets.shape[0]
    N = len(parents)
    lg = np.ascontiguousarray(np.broadcast_to(logits, (B,) + logits.shape))
    qq = np.ascontiguousarray(np.broadcast_to(q, (B,) + q.shape))
    tk = np.ascontiguousarray(np.broadcast_to(np.asarray(tokens, np.int32), (B, N)))
    pa = np.ascontiguousarray(np.broadcast_to(np.asarray(parents, np.int32), (B, N)))
    res = oracle.verify_tree_mss(lg, dtype, qq, tk, pa, coin_sets, np.full(B, T, np.float32), D)
    out = []
    for b in range(B):
        k = int(res["accept_len"][b])
        out.append((k,) + tuple(int(t) for t in res["out_tokens"][b, : k + 1]) +
                   tuple(int(nd) for nd in res["accepted_nodes"][b, :k]))
    return out


def mss_law(logits, dtype, q, tokens, parents, T, D):
    """Exact law of the multi-step speculative sampling walk over lattice coins.

    Node c is tested with coin c-1 and the final draw uses coin N-1.  Returns
    {(accept_len, tok_0, ..., tok_k, node_0, ..., node_{k-1}): probability}.
    """
    parents = np.asarray(parents)
    N = len(parents)
    law = {}

    def outcomes(cs):
        return mss_outcomes(logits, dtype, q, tokens, parents, T, D, cs)

    def walk(cur, fixed, mass):
        fixed = fixed.copy()
        for c in [c for c in range(cur + 1, N) if parents[c] == cur]:
            def f(ks, c=c, fixed=fixed):
                cs = np.repeat(fixed[None, :], len(ks), axis=0)
                cs[:, c - 1] = coin(ks)
                return [c in o[2 + o[0]:] for o in outcomes(cs)]
            segs = segments(f)
            acc = [(s, e) for s, e, v in segs if v]
            p_acc = sum(e - s for s, e in acc) / LATTICE
            if p_acc > 0.0:
                sub = fixed.copy()
                sub[c - 1] = coin(acc[0][0])
                walk(c, sub, mass * p_acc)
            rej = next((s for s, e, v in segs if not v), None)
            if rej is None:
                return
            mass *= 1.0 - p_acc
            fixed[c - 1] = coin(rej)
            if mass == 0.0:
                return

        def g(ks):
            cs = np.repeat(fixed[None, :], len(ks), axis=0)
            cs[:, N - 1] = coin(ks)
            return outcomes(cs)
        for s, e, v in segments(g):
            law[v] = law.get(v, 0.0) + mass * (e - s) / LATTICE

    walk(0, coin(np.zeros(N, dtype=np.int64)), 1.0)
    return law
