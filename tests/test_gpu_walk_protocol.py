"""The walks' hand-off protocol on the GPU: bounded waits that run out, determinism over
many calls, and results that do not depend on the launch options.

The waits between a request's workgroups are bounded; a bound of one poll (set from the
host with the spin_limit option, so every kernel still runs to its end) makes most
requests give up.  Such a request must report SPEC_ROW_RETRY (-2), never a wrong result;
the requests that completed must still match the oracle; and the next call on the same
workspace, with the default bound, must match the oracle everywhere (the call counter
that tags the hand-off words advanced only after every workgroup of the forced call had
finished).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from lossless_rejection_sampling_verify_amd import _lib as L
from lossless_rejection_sampling_verify_amd import workloads as wl

from test_gpu_parity import (_api, compare, dev, dev_logits, launch, say, torch,  # noqa: F401
                             chain_cfg, BAND)
# one call each, no retry: these tests force give-ups and check how they are reported
from test_gpu_parity import (_gpu_chain_once as gpu_chain, _gpu_greedy_once as gpu_greedy,
                             _gpu_tree_once as gpu_tree)

pytestmark = pytest.mark.gpu

RETRY = L.SPEC_ROW_RETRY


def _completed_match(g, o, keys, margin, label):
    """Requests that did not give up match the oracle (outside the near-tie band)."""
    done = g["accept_len"] != RETRY
    sub_g = {k: np.asarray(v)[done] for k, v in g.items()}
    sub_o = {k: np.asarray(v)[done] for k, v in o.items() if k in keys or k == "accept_len"}
    compare(sub_g, sub_o, keys, None if margin is None else margin[done], probs=False,
            label=label,
            accept_margin=None if margin is None else np.asarray(o["accept_margin"])[done])
    return int((~done).sum())


def test_chain_and_greedy_give_up_then_recover(launch):
    c = wl.make_chain(5, seed=21, B=64, G=4, V=152064)
    o = oracle.verify_chain(c.logits, c.dtype, c.draft_probs, c.draft_tokens, c.coins,
                            c.temperature)
    oa, oo = oracle.verify_greedy(c.logits, c.dtype, c.greedy_tokens)
    for rnd, spin in enumerate((1, 1, 200)):
        launch.clear()
        launch.update(spin_limit=spin)
        say(f"chain, {spin} polls per wait, round {rnd}")
        g = gpu_chain(c.logits, c.dtype, c.draft_probs, c.draft_tokens, c.coins, c.temperature)
        gave_up = _completed_match(g, o, ["accept_len", "out_tokens"], o["margin"],
                                   f"chain spin {spin} (completed) r{rnd}")
        if spin == 1:
            assert gave_up > 0, "a one-poll bound should make some request give up"
        assert set(np.unique(g["accept_len"])) <= set(range(-2, c.G + 1))
        say(f"greedy, {spin} polls per wait, round {rnd}: chain gave up on {gave_up}")
        ga, go = gpu_greedy(c.logits, c.dtype, c.greedy_tokens)
        gave_up_g = _completed_match(dict(accept_len=ga, out_tokens=go),
                                     dict(accept_len=oa, out_tokens=oo),
                                     ["accept_len", "out_tokens"], None,
                                     f"greedy spin {spin} (completed) r{rnd}")
        say(f"greedy gave up on {gave_up_g}")
        if spin == 1:
            assert gave_up_g > 0
        launch.clear()      # the default bound, same cached workspaces
        say(f"chain and greedy after the forced give-ups, round {rnd}")
        g = gpu_chain(c.logits, c.dtype, c.draft_probs, c.draft_tokens, c.coins, c.temperature)
        assert (g["accept_len"] != RETRY).all()
        compare(g, o, ["accept_len", "out_tokens"], o["margin"], label=f"chain after give-ups r{rnd}")
        ga, go = gpu_greedy(c.logits, c.dtype, c.greedy_tokens)
        np.testing.assert_array_equal(ga, oa)
        np.testing.assert_array_equal(go, oo)


@pytest.mark.parametrize("mode", [oracle.TREE_GREEDY, oracle.TREE_SAMPLING])
def test_tree_gives_up_then_recovers(mode, launch):
    t = wl.make_tree(4, seed=22, B=16, N=40, V=60000, D=5, max_children=5)
    o = oracle.verify_tree(t.logits, t.dtype, t.node_tokens, t.parents, t.coins, t.temperature,
                           t.D, mode)
    margin = o["margin"] if mode == oracle.TREE_SAMPLING else None
    keys = ["accept_len", "out_tokens", "accepted_nodes"]
    launch.update(spin_limit=1)
    say(f"tree mode {mode}, one poll per wait")
    g = gpu_tree(t, mode)
    assert _completed_match(g, o, keys, margin, f"tree {mode} spin 1 (completed)") > 0
    launch.clear()
    say(f"tree mode {mode} after the forced give-ups")
    g = gpu_tree(t, mode)
    assert (g["accept_len"] != RETRY).all()
    if mode == oracle.TREE_GREEDY:
        g["probs"] = np.zeros_like(g["probs"])
        o["probs"] = np.zeros_like(o["probs"])
    compare(g, o, keys, margin, label=f"tree {mode} after give-ups")


def test_multi_step_tree_gives_up_then_recovers(launch):
    from test_gpu_mss import gpu_mss, oracle_mss
    t = wl.make_tree_mss(4, seed=23, B=16, N=32, V=40000, D=5, max_children=4)
    o = oracle_mss(t)
    keys = ["accept_len", "out_tokens", "accepted_nodes"]
    launch.update(spin_limit=1)
    say("multi-step tree, one poll per wait")
    g = gpu_mss(t)
    assert _completed_match(g, o, keys, o["margin"], "mss spin 1 (completed)") > 0
    launch.clear()
    say("multi-step tree after the forced give-ups")
    g = gpu_mss(t)
    assert (g["accept_len"] != RETRY).all()
    compare(g, o, keys, o["margin"], label="mss after give-ups")


@pytest.fixture(scope="module")
def large_batch():
    c = chain_cfg(5)
    o = oracle.verify_chain(c.logits, c.dtype, c.draft_probs, c.draft_tokens, c.coins,
                            c.temperature)
    oa, oo = oracle.verify_greedy(c.logits, c.dtype, c.greedy_tokens)
    return c, o, oa, oo


def test_large_batch_is_deterministic_over_100_calls(large_batch):
    """The large-batch workload (B=256, gamma=4, V=152064, bf16) in the benchmark's launch
    configuration: 100 chain calls and 100 greedy calls on one set of device inputs give
    bitwise-identical outputs, equal to the oracle's."""
    c, o, oa, oo = large_batch
    api = _api()
    lg, q = dev_logits(c.logits, c.dtype), dev(c.draft_probs)
    x, xg, u, T = dev(c.draft_tokens), dev(c.greedy_tokens), dev(c.coins), dev(c.temperature)
    say("large batch, 100 chain + 100 greedy calls")
    outs_c, outs_g = [], []
    for _ in range(100):
        acc, toks, probs = api.spec_verify_chain(lg, q, x, u, T, want_probs=True)
        outs_c.append((acc.clone(), toks.clone(), probs.clone()))
        ga, go = api.spec_verify_greedy(lg, xg)
        outs_g.append((ga.clone(), go.clone()))
    torch.cuda.synchronize()
    ref_c = [t.cpu().numpy() for t in outs_c[0]]
    ref_g = [t.cpu().numpy() for t in outs_g[0]]
    for i in range(1, 100):
        for a, r in zip(outs_c[i], ref_c):
            assert np.array_equal(a.cpu().numpy(), r), f"chain call {i}"
        for a, r in zip(outs_g[i], ref_g):
            assert np.array_equal(a.cpu().numpy(), r), f"greedy call {i}"
    compare(dict(accept_len=ref_c[0], out_tokens=ref_c[1], probs=ref_c[2]), o,
            ["accept_len", "out_tokens"], o["margin"], label="workload 5 chain x100 (first)")
    np.testing.assert_array_equal(ref_g[0], oa)
    np.testing.assert_array_equal(ref_g[1], oo)


@pytest.mark.parametrize("opts", [dict(cluster=1), dict(cluster=2), dict(cluster=3),
                                  dict(cluster=16), dict(row_loads="streaming"),
                                  dict(path="eager"), dict(path="eager", splits=1),
                                  dict(path="eager", splits=5), dict(path="eager", splits=64)],
                         ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_large_batch_across_launch_options(large_batch, opts, launch):
    """The same batch under other cluster widths (clamped to what the device holds), load
    kinds, and the eager passes at several split counts: greedy bit-exact, chain equal to
    the oracle outside the near-tie band."""
    c, o, oa, oo = large_batch
    launch.update(opts)
    say(f"large batch with {opts}")
    g = gpu_chain(c.logits, c.dtype, c.draft_probs, c.draft_tokens, c.coins, c.temperature)
    compare(g, o, ["accept_len", "out_tokens"], o["margin"], label=f"workload 5 chain {opts}")
    ga, go = gpu_greedy(c.logits, c.dtype, c.greedy_tokens)
    np.testing.assert_array_equal(ga, oa)
    np.testing.assert_array_equal(go, oo)
