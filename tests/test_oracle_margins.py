"""Pins of the oracle's near-tie margins and of its acceptance-rate diagnostic (CPU only).

The margin of a request is how far its coins are from flipping its result: the parity
tests exempt requests whose margin is <= 1e-6 from bit-exactness, so a margin that came
out too large would let real differences through, and one too small would exempt
requests for nothing.  These tests pin the margins to something other than the oracle's
own arithmetic: the breakpoints of its OUTPUT as one coin moves with every other input
fixed, found by the black-box law engine over the coin lattice (tests/lawengine.py).

  - A coin that decides an acceptance test (chain: u_i <= p/q; tree: u_d <= prob_acc)
    flips the result exactly where it crosses its threshold, so the oracle's acceptance
    margin must equal the smallest distance of those coins to the nearest breakpoint
    (plus the residual mass and the threshold_single distances where they apply).
  - The final draw's coin moves through the tokens' steps of the inverse CDF; its margin
    is kept in weight units (S times the coin-space distance, S the drawn row's total
    weight), so it must equal S times the coin's distance to the nearer end of its step.
  - beta_i = sum_x min(p_i(x), q_i(x)) is the probability that position i accepts
    (zdszero spec_origins, "Speculative Decoding", acceptance rule: x ~ q is kept with
    probability min(1, p(x)/q(x))), so it must equal the q-weighted lattice frequency of
    acceptance found by the same search.

Each breakpoint is known to one lattice step (2^-24), which bounds the tolerances.
"""
from __future__ import annotations

import numpy as np
import pytest
import scipy.special

import oracle

import lawengine as le

STEP = 1.0 / le.LATTICE
TOL = 2.5 * STEP


def kidx(u: float) -> int:
    """Lattice index of an exact lattice coin u = (k+1)/2^24."""
    return int(round(float(u) * le.LATTICE)) - 1


def piece_distances(segs, u):
    """Distances from coin u to the two ends of the piece of `segs` that holds it, in coin
    units (each within one lattice step); the ends of (0, 1] are exact (0 and 1)."""
    k = kidx(u)
    for s, e, _ in segs:
        if s <= k < e:
            # an end between lattice points j-1 and j (j = s or e) lies in
            # [coin(j-1), coin(j)): take the middle of that step
            lo = float(u) if s == 0 else float(u) - (float(le.coin(s - 1)) + 0.5 * STEP)
            hi = 1.0 - float(u) if e == le.LATTICE else (float(le.coin(e - 1)) + 0.5 * STEP) - float(u)
            return lo, hi, s, e
    raise AssertionError("coin outside every piece")


def inner_breakpoints(segs):
    """Coin-space positions of the breakpoints between pieces (middle of their step)."""
    return [float(le.coin(s - 1)) + 0.5 * STEP for s, _, _ in segs[1:]]


# ---------------------------------------------------------------------------------------
# chain

def _chain_case(rng, V, G, T):
    logits = (rng.standard_normal((G + 1, V)) * 1.5).astype(np.float32)
    q = np.exp(rng.standard_normal((G, V)) * 1.5)
    q = (q / q.sum(1, keepdims=True)).astype(np.float32)
    p = scipy.special.softmax(logits.astype(np.float64) / T, axis=-1)
    # drafts whose ratio p/q is below 1 (so every tested coin has a breakpoint in (0, 1)),
    # drawn from q restricted to those tokens
    x = []
    for i in range(G):
        ok = q[i].astype(np.float64) > p[i] * (1 + 1e-6)
        w = np.where(ok, q[i], 0.0)
        x.append(int(rng.choice(V, p=w / w.sum())))
    return logits, q, x


def _chain_one(logits, q, x, coins, T, beta=False):
    return oracle.verify_chain(logits[None], "f32", q[None], np.asarray(x, np.int32)[None],
                               np.asarray(coins, np.float32)[None], np.array([T], np.float32),
                               beta=beta)


def _chain_segments(logits, q, x, coins, T, i):
    """The oracle's output as a function of coin i, every other coin fixed."""
    base = np.asarray(coins, np.float32)

    def f(ks):
        cs = np.repeat(base[None, :], len(ks), axis=0)
        cs[:, i] = le.coin(ks)
        return le.chain_outcomes(logits, "f32", q, x, T, cs)
    return le.segments(f)


@pytest.mark.parametrize("seed,T", [(0, 1.0), (1, 0.7), (2, 1.3)])
def test_chain_margins_equal_breakpoint_distances(seed, T):
    rng = np.random.default_rng(100 + seed)
    V, G = 8, 3
    seen_kinds = set()
    for trial in range(30):
        logits, q, x = _chain_case(rng, V, G, T)
        coins = le.coin(rng.integers(0, le.LATTICE, G + 1))
        r = _chain_one(logits, q, x, coins, T, beta=True)
        k = int(r["accept_len"][0])
        assert 0 <= k <= G
        # acceptance coins: positions 0..min(k, G-1) were tested, each with one breakpoint
        acc = np.inf
        for i in range(min(k, G - 1) + 1):
            segs = _chain_segments(logits, q, x, coins, T, i)
            assert len(segs) == 2, "a tested acceptance coin flips the result exactly once"
            (bp,) = inner_breakpoints(segs)
            acc = min(acc, abs(float(coins[i]) - bp))
        S = 1.0 if k == G else 1.0 - float(r["beta"][0, k])   # the drawn row's total weight
        if k < G:
            acc = min(acc, S)
        # the final draw's coin: S times its distance to the ends of its token's step
        lo, hi, _, _ = piece_distances(_chain_segments(logits, q, x, coins, T, G), coins[G])
        draw = S * min(lo, hi)
        assert abs(r["accept_margin"][0] - acc) <= TOL, (trial, r["accept_margin"][0], acc)
        assert abs(r["margin"][0] - min(acc, draw)) <= TOL, (trial, r["margin"][0], acc, draw)
        seen_kinds.add("draw" if draw < acc else "accept")
    assert seen_kinds == {"draw", "accept"}, "both kinds of margin should decide some trial"


def test_chain_margin_is_small_exactly_when_a_nudge_flips_the_result():
    """Nudging any coin by less than the margin never changes the result; for the trials
    whose margin comes from a coin, nudging that coin by a little more than the margin
    (in its own units) does."""
    rng = np.random.default_rng(7)
    V, G, T = 8, 3, 1.0
    for trial in range(40):
        logits, q, x = _chain_case(rng, V, G, T)
        coins = le.coin(rng.integers(0, le.LATTICE, G + 1)).astype(np.float64)
        r = _chain_one(logits, q, x, coins, T, beta=True)
        m, k = float(r["margin"][0]), int(r["accept_len"][0])
        base = le.chain_outcomes(logits, "f32", q, x, T, coins[None].astype(np.float32))[0]
        S = 1.0 if k == G else 1.0 - float(r["beta"][0, k])
        nudged = []
        for i in range(G + 1):
            for sgn in (-1.0, 1.0):
                c = coins.copy()
                c[i] = min(1.0, max(STEP, c[i] + sgn * (m - 2 * STEP)))
                nudged.append(c)
        outs = le.chain_outcomes(logits, "f32", q, x, T, np.array(nudged, np.float32))
        assert all(o == base for o in outs), trial
        draw_kind = r["accept_margin"][0] > m + TOL
        at_range_end = draw_kind and min(abs(m - S * coins[G]), abs(m - S * (1 - coins[G]))) <= TOL
        if (draw_kind and not at_range_end) or (not draw_kind and k < G and abs(m - S) > TOL) \
                or (not draw_kind and k == G):
            # the margin is a coin's own distance (the draw's is m / S in coin units); a draw
            # coin nearest to an end of (0, 1] has no flip on that side and is left out
            scale = 1.0 / S if draw_kind else 1.0
            over = []
            for i in range(G + 1):
                for sgn in (-1.0, 1.0):
                    c = coins.copy()
                    c[i] = c[i] + sgn * (m * scale + 3 * STEP)
                    if STEP <= c[i] <= 1.0:
                        over.append(c)
            outs = le.chain_outcomes(logits, "f32", q, x, T, np.array(over, np.float32))
            assert any(o != base for o in outs), trial


@pytest.mark.parametrize("seed", [0, 1])
def test_beta_equals_lattice_acceptance_rate(seed):
    """beta_i from the oracle equals sum_x q_i(x) P(position i accepts x), the acceptance
    frequency over the coin lattice, with earlier positions accepted (their drafts have
    p/q >= 1)."""
    rng = np.random.default_rng(300 + seed)
    V, G, T = 6, 3, 1.0
    logits = (rng.standard_normal((G + 1, V)) * 1.5).astype(np.float32)
    q = np.exp(rng.standard_normal((G, V)) * 1.5)
    q[rng.random((G, V)) < 0.2] = 0.0
    q[:, 0] += 1e-3
    q = (q / q.sum(1, keepdims=True)).astype(np.float32)
    p = scipy.special.softmax(logits.astype(np.float64) / T, axis=-1)
    # drafts that are always accepted at the earlier positions: the token with the largest
    # p/q (its ratio is >= 1, since both rows sum to 1)
    sure = [int(np.argmax(np.where(q[i] > 0, p[i] / np.maximum(q[i], 1e-30), np.inf)))
            for i in range(G)]
    coins = np.full(G + 1, 0.5, np.float32)
    r = _chain_one(logits, q, sure, coins, T, beta=True)
    for i in range(G):
        rate = 0.0
        for xv in range(V):
            if q[i, xv] == 0.0:
                continue
            x = list(sure)
            x[i] = xv

            def f(ks, x=x, i=i):
                cs = np.repeat(coins[None, :], len(ks), axis=0)
                cs[:, i] = le.coin(ks)
                return [o[0] > i for o in le.chain_outcomes(logits, "f32", q, x, T, cs)]
            acc_pts = sum(e - s for s, e, v in le.segments(f) if v)
            rate += float(q[i, xv]) * acc_pts / le.LATTICE
        assert abs(float(r["beta"][0, i]) - rate) <= 2 * STEP, (i, r["beta"][0, i], rate)


# ---------------------------------------------------------------------------------------
# target-only tree

def _tree_segments(logits, tokens, parents, coins, T, D, d):
    base = np.asarray(coins, np.float32)

    def f(ks):
        cs = np.repeat(base[None, :], len(ks), axis=0)
        cs[:, d] = le.coin(ks)
        return le.tree_outcomes(logits, "f32", tokens, parents, T, D, cs)
    return le.segments(f)


@pytest.mark.parametrize("seed,sigma", [(0, 1.5), (1, 1.5), (2, 6.0), (3, 6.0)])
def test_tree_margins_equal_breakpoint_distances(seed, sigma):
    """Per level, the coin's breakpoints are the running sums prob_acc of the children's
    target probabilities; the tested children's probabilities come from them too (for
    the threshold_single distance, here 1 - p), and the last level's excluded mass sets
    the final draw's total weight S = 1 - (sum of the excluded children's p).  The
    children carry their parent row's top tokens (as a drafter's top-k would), in a
    random order; sharp rows (sigma 6) give children with p near 1, where the
    threshold_single distance decides the margin."""
    rng = np.random.default_rng(500 + seed)
    V, T = 10, 1.0
    parents = [-1, 0, 0, 0, 1, 1, 2, 4]
    N, D = len(parents), 3
    kinds, checked = set(), 0
    for trial in range(25):
        logits = (rng.standard_normal((N, V)) * sigma).astype(np.float32)
        tokens = [0] * N
        for cur in range(N):
            kids = [c for c in range(N) if parents[c] == cur]
            if kids:
                picks = rng.permutation(np.argsort(-logits[cur])[:len(kids)])
                for c, t in zip(kids, picks):
                    tokens[c] = int(t)
        coins = le.coin(rng.integers(0, le.LATTICE, D + 1))
        r = oracle.verify_tree(logits[None], "f32", np.asarray(tokens, np.int32)[None],
                               np.asarray(parents, np.int32)[None], coins[None].astype(np.float32),
                               np.array([T], np.float32), D, oracle.TREE_SAMPLING)
        k = int(r["accept_len"][0])
        path = [0] + [int(n) for n in r["accepted_nodes"][0, :k]]
        acc, S = np.inf, 1.0
        resolved = True
        for d in range(k + 1):
            cur = path[d]
            kids = [c for c in range(N) if parents[c] == cur]
            if not kids:
                break                                    # a leaf: no test, bonus draw
            segs = _tree_segments(logits, tokens, parents, coins, T, D, d)
            bps = inner_breakpoints(segs)               # prob_acc after each child
            if len(bps) != len(kids):
                # a child's probability is below one lattice step, so its piece is not
                # resolved; only sharp rows do this
                assert sigma > 2, (trial, d)
                resolved = False
                break
            u = float(coins[d])
            tested = d < k and path[d + 1] in kids
            n_tested = kids.index(path[d + 1]) + 1 if tested else len(kids)
            for j in range(n_tested):
                acc = min(acc, abs(u - bps[j]))
                pc = bps[j] - (bps[j - 1] if j else 0.0)
                acc = min(acc, abs(pc - 1.0))
            if not tested:                               # every child rejected
                S = 1.0 - bps[-1]
                acc = min(acc, S)
        if not resolved:
            continue
        checked += 1
        lo, hi, _, _ = piece_distances(_tree_segments(logits, tokens, parents, coins, T, D, D),
                                       coins[D])
        draw = S * min(lo, hi)
        tol = TOL * (1 + D)
        assert abs(r["accept_margin"][0] - acc) <= tol, (trial, r["accept_margin"][0], acc)
        assert abs(r["margin"][0] - min(acc, draw)) <= tol, (trial, r["margin"][0], acc, draw)
        kinds.add("draw" if draw < acc else "accept")
    assert checked >= 12
    assert kinds == {"draw", "accept"} or sigma > 2
