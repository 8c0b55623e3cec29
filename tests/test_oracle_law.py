"""Pins of the fp64 oracle to what the pages and the mathematics fix (CPU only).

Each test checks the oracle against something other than itself:
  - the losslessness identity min(p,q) + max(0, p-q) = p, which makes every emitted
    token follow the target distribution whatever q is (zdszero spec_origins,
    "Speculative Decoding", acceptance rule and the paragraph on why it is lossless;
    atlas "Speculative Decoding" section 0), checked exactly over the coin lattice with
    the black-box law engine, for one round and over several rounds of a toy LM;
  - the closed form E[#tokens] = (1 - alpha^(gamma+1)) / (1 - alpha) for i.i.d.
    positions (spec_origins, "closed form of the gain");
  - Monte-Carlo chi-square / z tests on the tiny chain workload;
  - the temperature softmax against scipy, the final draw against numpy's
    searchsorted on a cumulative sum, special cases with a known answer.
"""
from __future__ import annotations

import itertools

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
from lossless_rejection_sampling_verify_amd import workloads as wl

import lawengine as le

TOL_LAW = 2e-6        # lattice quantisation: a few breakpoints x 2^-24 each


def softmax64(logits, T=1.0):
    return scipy.special.softmax(np.asarray(logits, np.float64) / T, axis=-1)


def rand_rows(rng, R, V, sigma=1.5):
    return (rng.standard_normal((R, V)) * sigma).astype(np.float32)


def rand_q(rng, G, V, zero_frac=0.0, sigma=1.5):
    q = np.exp(rng.standard_normal((G, V)) * sigma)
    if zero_frac:
        q[rng.random((G, V)) < zero_frac] = 0.0
        for i in range(G):
            if q[i].sum() == 0:
                q[i, 0] = 1.0
    q /= q.sum(axis=1, keepdims=True)
    return q.astype(np.float32)


def law_over_drafts(logits, q, T, dtype="f32"):
    """Exact law of one chain round with the drafts x_i ~ q_i enumerated (i.i.d. given q)."""
    G, V = q.shape
    law = {}
    for x in itertools.product(range(V), repeat=G):
        wx = float(np.prod([q[i, x[i]] for i in range(G)], dtype=np.float64))
        if wx == 0.0:
            continue
        for out, pr in le.chain_round_law(logits, dtype, q, list(x), T).items():
            law[out] = law.get(out, 0.0) + wx * pr
    return law


# ----------------------------------------------------------------------------------
# losslessness, one round, fixed target rows

@pytest.mark.parametrize("seed,zero_frac,T", [(0, 0.0, 1.0), (1, 0.3, 1.0), (2, 0.0, 0.7),
                                              (3, 0.5, 1.3)])
def test_chain_round_emits_target_law(seed, zero_frac, T):
    """Every emitted token follows its target row, whatever q is (exact over coins)."""
    rng = np.random.default_rng(seed)
    V, G = 4, 2
    logits = rand_rows(rng, G + 1, V)
    q = rand_q(rng, G, V, zero_frac)
    p = softmax64(logits, T)
    law = law_over_drafts(logits, q, T)
    assert abs(sum(law.values()) - 1.0) < 1e-6
    # position 0: marginal = p_0
    first = np.zeros(V)
    for out, pr in law.items():
        first[out[1]] += pr
    np.testing.assert_allclose(first, p[0], atol=TOL_LAW)
    # position j >= 1, conditional on the emitted prefix: law = p_j
    for j in range(1, G + 1):
        cond = {}
        for out, pr in law.items():
            k = out[0]
            if k + 1 > j:                       # token j was emitted
                cond.setdefault(out[1: 1 + j], np.zeros(V))[out[1 + j]] += pr
        assert cond, "no emitted continuation at all"
        for prefix, dist in cond.items():
            if dist.sum() < 1e-3:
                continue
            np.testing.assert_allclose(dist / dist.sum(), p[j], atol=TOL_LAW / dist.sum() * 4)


def test_chain_acceptance_rate_and_residual_law():
    """P(accept x) = min(1, p/q) and the correction token follows norm(max(0, p-q))."""
    rng = np.random.default_rng(11)
    V = 6
    logits = rand_rows(rng, 2, V)
    q = rand_q(rng, 1, V, 0.2)
    p = softmax64(logits)
    for x in range(V):
        if q[0, x] == 0:
            continue
        law = le.chain_round_law(logits, "f32", q, [x], 1.0)
        acc = sum(pr for out, pr in law.items() if out[0] == 1)
        assert abs(acc - min(1.0, p[0, x] / float(q[0, x]))) < 2e-7
        rej = {out[1]: pr for out, pr in law.items() if out[0] == 0}
        if acc < 1.0 - 1e-6:
            resid = np.maximum(p[0] - q[0].astype(np.float64), 0.0)
            resid /= resid.sum()
            got = np.zeros(V)
            for t, pr in rej.items():
                got[t] = pr / (1.0 - acc)
            np.testing.assert_allclose(got, resid, atol=1e-5)


# ----------------------------------------------------------------------------------
# losslessness over several rounds of a toy language model

class ToyLM:
    """Prefix-dependent target and draft distributions over a tiny vocabulary."""

    def __init__(self, V, seed, sigma=1.5, noise=1.0):
        self.V, self.seed, self.sigma, self.noise = V, seed, sigma, noise

    def _rng(self, prefix, salt):
        return np.random.default_rng([self.seed, salt, len(prefix)] + list(prefix))

    def target_logits(self, prefix):
        return (self._rng(prefix, 1).standard_normal(self.V) * self.sigma).astype(np.float32)

    def draft_probs(self, prefix):
        d = self.target_logits(prefix).astype(np.float64) + \
            self._rng(prefix, 2).standard_normal(self.V) * self.noise
        return softmax64(d).astype(np.float32)


def round_law_toy(lm, prefix, G, T=1.0):
    """Exact law of one speculative round from ``prefix``: drafts enumerated, coins exact."""
    V = lm.V
    law = {}
    for x in itertools.product(range(V), repeat=G):
        wx, qs = 1.0, []
        for i in range(G):
            qi = lm.draft_probs(prefix + x[:i])
            qs.append(qi)
            wx *= float(qi[x[i]])
        if wx == 0.0:
            continue
        rows = np.stack([lm.target_logits(prefix + x[:i]) for i in range(G + 1)])
        for out, pr in le.chain_round_law(rows, "f32", np.stack(qs), list(x), T).items():
            toks = out[1:]
            law[toks] = law.get(toks, 0.0) + wx * pr
    return law


def test_multi_round_sequence_law_equals_target():
    """Several rounds of draft/verify produce sequences with the target's own law."""
    lm = ToyLM(V=3, seed=5)
    G, n = 2, 3
    cache = {}

    def seq_law(prefix, need):
        key = (prefix, need)
        if key in cache:
            return cache[key]
        out = {}
        for toks, pr in round_law_toy(lm, prefix, G).items():
            if len(toks) >= need:
                out[toks[:need]] = out.get(toks[:need], 0.0) + pr
            else:
                for rest, pr2 in seq_law(prefix + toks, need - len(toks)).items():
                    out[toks + rest] = out.get(toks + rest, 0.0) + pr * pr2
        cache[key] = out
        return out

    law = seq_law((), n)
    for seq in itertools.product(range(lm.V), repeat=n):
        target = 1.0
        for t in range(n):
            target *= softmax64(lm.target_logits(seq[:t]))[seq[t]]
        assert abs(law.get(seq, 0.0) - target) < 1e-5, (seq, law.get(seq), target)


# ----------------------------------------------------------------------------------
# closed form for the expected number of tokens per verify

@pytest.mark.parametrize("seed,G", [(21, 1), (22, 3), (23, 4)])
def test_expected_tokens_closed_form(seed, G):
    """Same (p, q) at every position, x_i ~ q i.i.d.:  E[#tokens] = (1-a^(G+1))/(1-a)."""
    rng = np.random.default_rng(seed)
    V = 4
    row = rand_rows(rng, 1, V)[0]
    q1 = rand_q(rng, 1, V)[0]
    logits = np.stack([row] * (G + 1))
    q = np.stack([q1] * G)
    p = softmax64(row)
    alpha = float(np.minimum(p, q1.astype(np.float64)).sum())
    expect = (1 - alpha ** (G + 1)) / (1 - alpha)
    law = law_over_drafts(logits, q, 1.0)
    e_tau = sum(pr * (len(out) - 1) for out, pr in law.items())   # out = (k, tokens...)
    assert abs(e_tau - expect) < 1e-5
    # the whole length distribution: P(k) = a^k (1 - a), P(G) = a^G
    for k in range(G + 1):
        pk = sum(pr for out, pr in law.items() if out[0] == k)
        want = alpha ** k * (1 - alpha) if k < G else alpha ** G
        assert abs(pk - want) < 1e-5


def test_beta_diagnostic_is_overlap():
    c = wl.make_chain(2, seed=3, V=2000)
    r = oracle.verify_chain(c.logits, c.dtype, c.draft_probs, c.draft_tokens, c.coins,
                            c.temperature, beta=True)
    for b in range(c.B):
        for i in range(c.G):
            p = softmax64(c.logits[b, i], 1.0)
            want = np.minimum(p, c.draft_probs[b, i].astype(np.float64)).sum()
            assert abs(r["beta"][b, i] - want) < 1e-12


# ----------------------------------------------------------------------------------
# Monte Carlo on the tiny chain workload

def _chisq_pvalue(counts, probs):
    exp = probs * counts.sum()
    order = np.argsort(exp)
    c, e = counts[order].astype(float), exp[order]
    # merge the smallest bins until each expected count is >= 5
    cc, ee, acc_c, acc_e = [], [], 0.0, 0.0
    for ci, ei in zip(c, e):
        acc_c += ci
        acc_e += ei
        if acc_e >= 5:
            cc.append(acc_c)
            ee.append(acc_e)
            acc_c = acc_e = 0.0
    if acc_e > 0:
        cc[-1] += acc_c
        ee[-1] += acc_e
    return scipy.stats.chisquare(cc, ee).pvalue


def test_tiny_chain_monte_carlo_chi_square():
    """10k trials of the tiny workload: first emitted token ~ p_0 (chi-square)."""
    c = wl.make_chain(1, seed=0)
    trials = 10_000
    rng = np.random.default_rng(1234)
    q = c.draft_probs[0].astype(np.float64)
    x = np.stack([rng.choice(c.V, size=trials, p=q[i] / q[i].sum()) for i in range(c.G)], 1)
    coins = wl.draw_coins(rng, (trials, c.G + 1))
    lg = np.ascontiguousarray(np.broadcast_to(c.logits[0], (trials,) + c.logits.shape[1:]))
    qq = np.ascontiguousarray(np.broadcast_to(c.draft_probs[0], (trials,) + c.draft_probs.shape[1:]))
    r = oracle.verify_chain(lg, c.dtype, qq, x.astype(np.int32), coins,
                            np.full(trials, 1.0, np.float32))
    p = softmax64(c.logits[0])
    counts = np.bincount(r["out_tokens"][:, 0], minlength=c.V)
    assert _chisq_pvalue(counts, p[0]) > 1e-3
    # second position, among trials where token 0 was accepted
    sel = r["accept_len"] >= 1
    counts1 = np.bincount(r["out_tokens"][sel, 1], minlength=c.V)
    assert _chisq_pvalue(counts1, p[1]) > 1e-3


def test_tiny_chain_monte_carlo_expected_tokens():
    """i.i.d. variant of the tiny workload: mean tokens per verify vs the closed form (z-test)."""
    c = wl.make_chain(1, seed=0)
    trials = 20_000
    rng = np.random.default_rng(99)
    row, q1 = c.logits[0, 0], c.draft_probs[0, 0].astype(np.float64)
    G = c.G
    lg = np.ascontiguousarray(np.broadcast_to(row, (trials, G + 1, c.V)))
    qq = np.ascontiguousarray(np.broadcast_to(c.draft_probs[0, 0], (trials, G, c.V)))
    x = rng.choice(c.V, size=(trials, G), p=q1 / q1.sum()).astype(np.int32)
    coins = wl.draw_coins(rng, (trials, G + 1))
    r = oracle.verify_chain(lg, c.dtype, qq, x, coins, np.ones(trials, np.float32))
    tau = r["accept_len"] + 1.0
    alpha = float(np.minimum(softmax64(row), q1).sum())
    mean = (1 - alpha ** (G + 1)) / (1 - alpha)
    pk = np.array([alpha ** k * (1 - alpha) for k in range(G)] + [alpha ** G])
    var = float((pk * (np.arange(1, G + 2) - mean) ** 2).sum())
    z = (tau.mean() - mean) / np.sqrt(var / trials)
    assert abs(z) < 3.5


# ----------------------------------------------------------------------------------
# softmax, final draw and special cases against library routines / known answers

@pytest.mark.parametrize("dtype,T", [("f32", 1.0), ("bf16", 0.7), ("f32", 2.5)])
def test_probs_match_scipy_softmax(dtype, T):
    c = wl.make_chain(2, seed=7, V=5000, dtype=dtype, T=T)
    r = oracle.verify_chain(c.logits, c.dtype, c.draft_probs, c.draft_tokens, c.coins,
                            c.temperature)
    lg = wl.logits_as_f32(c.logits, c.dtype)
    for b in range(c.B):
        k = r["accept_len"][b]
        for i in range(k + 1):
            p = softmax64(lg[b, i], float(np.float32(T)))   # T as passed, in fp32
            want = p[r["out_tokens"][b, i]]
            assert abs(r["probs"][b, i] - want) <= 1e-12 * max(want, 1e-300)


def _searchsorted_draw(w, u):
    """Textbook inverse CDF: first index whose inclusive cumulative sum reaches u * sum."""
    C = np.cumsum(w)
    return int(np.searchsorted(C, u * C[-1], side="left"))


def test_bonus_draw_is_inverse_cdf():
    """q_0(x0) = 0 < p_0(x0) forces acceptance; the bonus is the inverse-CDF draw of p_1."""
    rng = np.random.default_rng(5)
    B, V = 400, 300
    logits = (rng.standard_normal((B, 2, V)) * 2).astype(np.float32)
    x = rng.integers(0, V, size=(B, 1)).astype(np.int32)
    q = rand_q(rng, B, V)[:, None, :].copy()
    q[np.arange(B), 0, x[:, 0]] = 0.0
    coins = wl.draw_coins(rng, (B, 2))
    r = oracle.verify_chain(logits, "f32", q, x, coins, np.ones(B, np.float32))
    assert (r["accept_len"] == 1).all()
    checked = 0
    for b in range(B):
        if r["margin"][b] <= 1e-9:
            continue
        want = _searchsorted_draw(softmax64(logits[b, 1]), float(coins[b, 1]))
        assert r["out_tokens"][b, 1] == want
        checked += 1
    assert checked > B * 0.9


def test_one_hot_draft_on_impossible_token_gives_plain_target_draw():
    """q one-hot on x with p(x) = 0: rejected at once, correction = plain draw from p_0."""
    rng = np.random.default_rng(6)
    B, V, G = 300, 200, 3
    logits = (rng.standard_normal((B, G + 1, V)) * 2).astype(np.float32)
    x = rng.integers(0, V, size=(B, G)).astype(np.int32)
    logits[np.arange(B), 0, x[:, 0]] = -np.inf
    q = np.zeros((B, G, V), np.float32)
    for i in range(G):
        q[np.arange(B), i, x[:, i]] = 1.0
    coins = wl.draw_coins(rng, (B, G + 1))
    r = oracle.verify_chain(logits, "f32", q, x, coins, np.ones(B, np.float32))
    assert (r["accept_len"] == 0).all()
    for b in range(B):
        if r["margin"][b] <= 1e-9:
            continue
        assert r["out_tokens"][b, 0] == _searchsorted_draw(softmax64(logits[b, 0]), float(coins[b, G]))


def test_degenerate_p_q_cases():
    rng = np.random.default_rng(8)
    V, G = 10, 1
    logits = rand_rows(rng, 2, V)
    p = softmax64(logits)
    # q(a) = 0 < p(a): accepted for every coin
    q = rand_q(rng, 1, V)
    q[0, 3] = 0.0
    law = le.chain_round_law(logits, "f32", q, [3], 1.0)
    assert abs(sum(pr for o, pr in law.items() if o[0] == 1) - 1.0) < 1e-12
    # p(a) = 0 < q(a): rejected for every coin
    lg2 = logits.copy()
    lg2[0, 4] = -np.inf
    law = le.chain_round_law(lg2, "f32", rand_q(rng, 1, V), [4], 1.0)
    assert abs(sum(pr for o, pr in law.items() if o[0] == 0) - 1.0) < 1e-12
    # q(a) <= p(a): always accepted (draft under-confident)
    q = rand_q(rng, 1, V)
    a = int(np.argmax(p[0] - q[0]))
    assert q[0, a] <= p[0, a]
    law = le.chain_round_law(logits, "f32", q, [a], 1.0)
    assert abs(sum(pr for o, pr in law.items() if o[0] == 1) - 1.0) < 1e-12
    # one-hot target row: every output token is that one
    lg3 = np.full((2, V), -np.inf, np.float32)
    lg3[0, 7] = 0.0
    lg3[1, 2] = 1.5
    law = le.chain_round_law(lg3, "f32", rand_q(rng, 1, V), [5], 1.0)
    assert set(law) == {(0, 7)}
    law = le.chain_round_law(lg3, "f32", rand_q(rng, 1, V), [7], 1.0)
    assert set(law) == {(1, 7, 2)}


def test_q_equal_p_never_rejects_outside_band():
    rng = np.random.default_rng(9)
    B, G, V = 200, 4, 500
    logits = (rng.standard_normal((B, G + 1, V)) * 3).astype(np.float32)
    q = softmax64(logits[:, :G]).astype(np.float32)
    q64 = q.astype(np.float64)
    q64 /= q64.sum(axis=-1, keepdims=True)
    x = np.stack([[rng.choice(V, p=q64[b, i]) for i in range(G)] for b in range(B)]).astype(np.int32)
    coins = wl.draw_coins(rng, (B, G + 1))
    r = oracle.verify_chain(logits, "f32", q, x, coins, np.ones(B, np.float32))
    far = r["margin"] > 1e-6
    assert (r["accept_len"][far] == G).all()
