"""CPU checks of the GPU parity helpers' near-tie recheck and retry (no GPU): outputs that
the band allows are accepted, others are not.  The 'GPU outputs' here are the oracle's own
results for coins moved across their decision boundaries."""
import numpy as np
import pytest

import oracle
from test_gpu_parity import BAND, RETRY, _retrying, chain_recheck


def _two_near_decisions():
    """One request, G = 3, V = 8, fp32 logits at T = 1: at positions 0 and 1 the draft row
    equals the target except at the drafted token, where q is one part in 1e7 above p, so
    p/q lies just below 1.  Coin 0 lies just above p/q (the oracle rejects at 0) and coin 1
    just below it (it would accept at 1): two decisions within the band."""
    rng = np.random.default_rng(7)
    G, V = 3, 8
    logits = rng.normal(0.0, 1.0, (1, G + 1, V)).astype(np.float32)
    T = np.ones(1, np.float32)
    q = np.zeros((1, G, V), np.float32)
    x = np.zeros((1, G), np.int32)
    r = np.zeros(G)
    for j in range(G):
        z = logits[0, j].astype(np.float64)
        p = np.exp(z - z.max())
        p /= p.sum()
        x[0, j] = int(np.argmax(p))
        q[0, j] = p.astype(np.float32)
        q[0, j, x[0, j]] = np.float32(p[x[0, j]] * (1.0 + 1e-7))
        r[j] = p[x[0, j]] / float(q[0, j, x[0, j]])
    assert r[0] < 1.0 and r[1] < 1.0

    def above(v):
        f = np.float32(v)
        while float(f) <= v:
            f = np.nextafter(f, np.float32(2.0))
        return f

    def below(v):
        f = np.float32(v)
        while float(f) > v:
            f = np.nextafter(f, np.float32(0.0))
        return f

    coins = np.array([[above(r[0]), below(r[1]), 0.5, 0.3]], np.float32)
    moved = np.array([[below(r[0]), above(r[1]), 0.5, 0.3]], np.float32)
    assert abs(float(coins[0, 0]) - r[0]) < BAND and abs(float(coins[0, 1]) - r[1]) < BAND
    return logits, q, x, coins, moved, T


def test_follow_reaches_two_moved_decisions():
    logits, q, x, coins, moved, T = _two_near_decisions()
    plain = oracle.verify_chain(logits, "f32", q, x, coins, T)
    gpu = oracle.verify_chain(logits, "f32", q, x, moved, T)
    assert int(plain["accept_len"][0]) == 0  # the oracle rejects at 0
    assert int(gpu["accept_len"][0]) == 1    # kept at 0, rejected at 1: two decisions moved
    assert chain_recheck(logits, "f32", q, x, coins, T, gpu)(0)


def test_follow_refuses_a_different_kept_token():
    logits, q, x, coins, moved, T = _two_near_decisions()
    gpu = oracle.verify_chain(logits, "f32", q, x, moved, T)
    bad = dict(gpu)
    bad["out_tokens"] = gpu["out_tokens"].copy()
    bad["out_tokens"][0, 0] = (int(x[0, 0]) + 1) % logits.shape[-1]
    assert not chain_recheck(logits, "f32", q, x, coins, T, bad)(0)


def test_follow_refuses_a_decision_outside_the_band():
    logits, q, x, coins, moved, T = _two_near_decisions()
    gpu = oracle.verify_chain(logits, "f32", q, x, moved, T)
    far = moved.copy()           # kept at 0, as on the GPU's path
    far[0, 1] = np.float32(0.5)  # far below p/q at 1: the oracle keeps x_1 and no nudge
    ref = oracle.verify_chain(logits, "f32", q, x, far, T)  # of the band rejects it
    assert int(ref["accept_len"][0]) >= 2
    assert not chain_recheck(logits, "f32", q, x, far, T, gpu)(0)


def test_retrying_calls_again_once():
    calls = []

    def fake(results):
        def call():
            calls.append(1)
            return results[len(calls) - 1]
        return call

    ok = {"accept_len": np.array([1, 2])}
    assert _retrying(fake([ok])) is ok and len(calls) == 1
    calls.clear()
    first = {"accept_len": np.array([1, RETRY])}
    assert _retrying(fake([first, ok])) is ok and len(calls) == 2
    calls.clear()
    with pytest.raises(AssertionError):
        _retrying(fake([first, first]))
    calls.clear()
    assert _retrying(fake([(np.array([0, 0]), None)]))[0].tolist() == [0, 0]
