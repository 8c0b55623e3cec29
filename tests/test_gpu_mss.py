"""HIP token-tree verify by multi-step speculative sampling vs the fp64 oracle.

Same bar as the other verify paths: accept_len, emitted tokens and accepted node ids
bit-exact outside the 1e-6 near-tie band of the oracle's decision trace (coin tests,
residual masses, the final inverse CDF); probabilities within 1e-5 relative.  Covers the
tree workload at full size with draft rows (the shape the benchmark times), ragged and
unaligned vocabularies over several tiles, both logit dtypes and temperatures, deep
and wide trees, the root-only tree, residuals that run out of mass, invalid requests and
bitwise determinism.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from lossless_rejection_sampling_verify_amd import workloads as wl

from test_gpu_parity import (_api, _opts, _tree_out, compare, dev, dev_logits, launch,  # noqa: F401
                             nudge_reaches, say, torch)

pytestmark = pytest.mark.gpu


def gpu_mss(t, **kw):
    api = _api()
    q = kw.get("q", t.draft_probs)
    acc, out, nodes, probs = api.spec_verify_tree_mss(
        dev_logits(kw.get("logits", t.logits), t.dtype), dev(q.astype(np.float32)),
        dev(kw.get("tokens", t.node_tokens).astype(np.int32)),
        dev(kw.get("parents", t.parents).astype(np.int32)),
        dev(kw.get("coins", t.coins).astype(np.float32)),
        dev(kw.get("temperature", t.temperature).astype(np.float32)), kw.get("D", t.D),
        want_probs=True, opts=_opts())
    torch.cuda.synchronize()
    return dict(accept_len=acc.cpu().numpy(), out_tokens=out.cpu().numpy(),
                accepted_nodes=nodes.cpu().numpy(), probs=probs.cpu().numpy())


def oracle_mss(t, **kw):
    return oracle.verify_tree_mss(kw.get("logits", t.logits), t.dtype, kw.get("q", t.draft_probs),
                                  kw.get("tokens", t.node_tokens), kw.get("parents", t.parents),
                                  kw.get("coins", t.coins), kw.get("temperature", t.temperature),
                                  kw.get("D", t.D))


def mss_recheck(t, g, **kw):
    """recheck for compare(): request b of a multi-step tree call."""
    def run_b(b):
        def run(cs):
            n = len(cs)
            rep = lambda a: np.ascontiguousarray(np.broadcast_to(a[b], (n,) + a.shape[1:]))
            r = oracle.verify_tree_mss(rep(kw.get("logits", t.logits)), t.dtype,
                                       rep(kw.get("q", t.draft_probs)),
                                       rep(kw.get("tokens", t.node_tokens)),
                                       rep(kw.get("parents", t.parents)), cs,
                                       np.full(n, kw.get("temperature", t.temperature)[b],
                                               np.float32), kw.get("D", t.D))
            return [_tree_out(r, i) for i in range(n)]
        return nudge_reaches(run, kw.get("coins", t.coins)[b], _tree_out(g, b))
    return run_b


def check_mss(t, label, **kw):
    say(f"mss {label}: B={t.B} N={t.N} D={kw.get('D', t.D)} V={t.V} {t.dtype}")
    g = gpu_mss(t, **kw)
    o = oracle_mss(t, **kw)
    stats = compare(g, o, ["accept_len", "out_tokens", "accepted_nodes"], o["margin"], label=label,
                    recheck=mss_recheck(t, g, **kw))
    return stats, g, o


def test_tree_workload_with_draft_rows_in_fp32():
    """The same shape with fp32 logits (the draft rows are fp32 either way)."""
    t = wl.make_tree_mss(4, seed=33, dtype=wl.F32)
    stats, g, o = check_mss(t, "tree workload with draft rows, fp32")
    assert stats["near_accept"] <= 2


def test_tree_workload_with_draft_rows_full_size():
    t = wl.make_tree_mss(4)
    stats, g, o = check_mss(t, "tree workload with draft rows")
    assert stats["near_accept"] <= 2
    assert (o["accept_len"] >= 0).all() and o["accept_len"].mean() > 1.0


@pytest.mark.parametrize("dtype,V,T", [(wl.BF16, 12289, 1.0), (wl.F32, 12289, 0.7),
                                       (wl.BF16, 4999, 0.7), (wl.F32, 4999, 1.0),
                                       (wl.BF16, 40960, 1.3), (wl.F32, 7, 1.0)])
def test_ragged_vocabularies(dtype, V, T):
    t = wl.make_tree_mss(4, seed=V % 97, B=24, N=24, V=V, D=4, dtype=dtype, T=T,
                         max_children=5 if V > 7 else 3)
    check_mss(t, f"ragged V={V} {dtype} T={T}")


def test_wide_and_deep_trees():
    t = wl.make_tree_mss(4, seed=3, B=8, N=200, V=3000, D=12, max_children=16, dtype=wl.F32)
    check_mss(t, "wide and deep")
    t = wl.make_tree_mss(4, seed=4, B=4, N=1024, V=600, D=40, max_children=32, dtype=wl.BF16)
    check_mss(t, "1024 nodes")


def test_close_draft_gives_long_walks():
    """A draft close to the target accepts most tests: long walks, few residual passes."""
    t = wl.make_tree_mss(4, seed=7, B=32, N=48, V=9000, D=8, max_children=4, draft_var=0.05)
    stats, g, o = check_mss(t, "close draft")
    assert o["accept_len"].mean() > 3


def test_far_draft_gives_many_rejections():
    """A poor draft rejects most children: many residual updates per node."""
    t = wl.make_tree_mss(4, seed=8, B=32, N=48, V=9000, D=4, max_children=8, draft_var=16.0)
    check_mss(t, "far draft")


def test_root_only_tree_is_a_plain_draw():
    t = wl.make_tree_mss(4, seed=9, B=16, N=1, V=5000, D=1, dtype=wl.F32)
    stats, g, o = check_mss(t, "root only")
    assert (g["accept_len"] == 0).all()


def test_residual_without_mass_falls_back():
    """q = 2p (used as given): after a rejection no residual mass is left; the walk stops
    testing siblings and draws from the target row."""
    t = wl.make_tree_mss(4, seed=10, B=16, N=6, V=700, D=1, max_children=5, dtype=wl.F32)
    parents = np.tile(np.array([-1, 0, 0, 0, 0, 0], np.int32), (t.B, 1))
    lg = wl.logits_as_f32(t.logits, t.dtype).astype(np.float64)
    p = np.exp(lg - lg.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    q = (2.0 * p).astype(np.float32)
    coins = t.coins.copy()
    coins[:, :5] = 0.999   # every tested child is rejected (ratio about 1/2)
    kw = dict(parents=parents, q=q, coins=coins)
    say(f"mss no residual mass: B={t.B} N={t.N} V={t.V}")
    g, o = gpu_mss(t, **kw), oracle_mss(t, **kw)
    # the oracle records the empty residual as a zero margin, so compare directly: both
    # stop after the first child and draw from the root's target row
    assert (o["accept_len"] == 0).all() and (g["accept_len"] == 0).all()
    cdf = np.cumsum(p[:, 0], axis=-1)
    target = coins[:, t.N - 1].astype(np.float64) * cdf[:, -1]
    near = np.abs(cdf - target[:, None]).min(axis=1) <= 1e-6
    want = np.array([np.searchsorted(cdf[b], target[b]) for b in range(t.B)])
    np.testing.assert_array_equal(o["out_tokens"][~near, 0], want[~near])
    np.testing.assert_array_equal(g["out_tokens"][~near, 0], want[~near])
    assert (~near).sum() >= t.B - 1


def test_invalid_requests_match_oracle():
    t = wl.make_tree_mss(4, seed=11, B=8, N=16, V=1000, D=4, dtype=wl.F32)
    par, tok, coins, T, q = (t.parents.copy(), t.node_tokens.copy(), t.coins.copy(),
                             t.temperature.copy(), t.draft_probs.copy())
    lg = t.logits.copy()
    par[1, 5] = 7                          # parent after the child
    tok[2, 3] = t.V                        # token out of range
    T[3] = -1.0                            # bad temperature
    coins[4, 2] = 0.0                      # coin outside (0, 1]
    q[5, t.parents[5, 4], t.node_tokens[5, 4]] = np.nan   # q(token) not a probability
    lg[6, 0] = -np.inf                     # the root row has no finite logit
    par[7, 1:] = np.arange(0, t.N - 1)     # a chain deeper than D
    kw = dict(parents=par, tokens=tok, coins=coins, temperature=T, q=q, logits=lg)
    stats, g, o = check_mss(t, "invalid requests", **kw)
    assert (o["accept_len"][1:8] == -1).all() and o["accept_len"][0] >= 0
    np.testing.assert_array_equal(g["accept_len"], o["accept_len"])


def test_deterministic_bits():
    t = wl.make_tree_mss(4, seed=12, B=16, N=32, V=20000, D=5)
    a = gpu_mss(t)
    b = gpu_mss(t)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


@pytest.mark.parametrize("cluster", ["1", "2", "5"])
def test_cluster_sizes(cluster, launch):
    """The walk split over W workgroups per request (W set with the cluster option)
    matches the oracle for every W, including one workgroup per request and a W that does
    not divide the vocabulary evenly."""
    launch.update(cluster=int(cluster))
    t = wl.make_tree_mss(4, seed=13, B=16, N=40, V=30011, D=6, max_children=6, dtype=wl.BF16)
    check_mss(t, f"cluster cap {cluster}")


def test_first_token_law_with_iid_children():
    """Multi-step speculative sampling is lossless when a node's children are independent
    draws from its draft row: over 20000 trials, each drawing the root's three children
    afresh from q (duplicates allowed), the first emitted token follows the root's target
    row (chi-square on the GPU's tokens); the first 2000 trials are also compared with the
    oracle."""
    import scipy.special
    import scipy.stats
    rng = np.random.default_rng(909)
    V, N, D, trials = 20, 4, 1, 20000
    rows = (rng.standard_normal((N, V)) * 1.5).astype(np.float32)
    drafts = rows + rng.standard_normal((N, V)).astype(np.float32)
    q = scipy.special.softmax(drafts.astype(np.float64), axis=-1).astype(np.float32)
    parents = np.array([-1, 0, 0, 0], np.int32)
    tokens = np.zeros((trials, N), np.int32)
    qq = q[0].astype(np.float64) / q[0].astype(np.float64).sum()
    tokens[:, 1:] = rng.choice(V, size=(trials, 3), p=qq)
    t = wl.TreeMssInputs(name="law tree", B=trials, N=N, V=V, D=D, dtype=wl.F32,
                         logits=np.ascontiguousarray(np.broadcast_to(rows, (trials, N, V))),
                         draft_probs=np.ascontiguousarray(np.broadcast_to(q, (trials, N, V))),
                         node_tokens=tokens,
                         parents=np.ascontiguousarray(np.broadcast_to(parents, (trials, N))),
                         coins=wl.draw_coins(rng, (trials, N)),
                         temperature=np.ones(trials, np.float32))
    say("mss first-token law, 20000 trials")
    g = gpu_mss(t)
    assert (g["accept_len"] >= 0).all()
    p0 = scipy.special.softmax(rows[0].astype(np.float64))
    counts = np.bincount(g["out_tokens"][:, 0], minlength=V)
    exp = p0 * trials
    keep = exp >= 5
    obs, ex = counts[keep], exp[keep]
    if (~keep).any():  # the rare tokens pooled into one bin
        obs, ex = np.append(obs, counts[~keep].sum()), np.append(ex, exp[~keep].sum())
    assert scipy.stats.chisquare(obs, ex).pvalue > 1e-3
    head = {k: v for k, v in dict(logits=t.logits[:2000], q=t.draft_probs[:2000],
                                   tokens=t.node_tokens[:2000], parents=t.parents[:2000],
                                   coins=t.coins[:2000], temperature=t.temperature[:2000]).items()}
    o = oracle_mss(t, **head)
    compare({k: v[:2000] for k, v in g.items()}, o,
            ["accept_len", "out_tokens", "accepted_nodes"], o["margin"], label="mss law tree")
