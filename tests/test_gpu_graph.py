"""The verify calls captured into a HIP graph replay correctly.

A captured call keeps its kernel arguments, so anything that must change from one call
to the next -- the tags of the words a request's workgroups hand to each other -- has to
come from device state, which the library keeps in the workspace header.  Each test
captures one call, then replays it on several input sets copied into the captured
buffers (with eager work and synchronisation between replays), and checks every replay
against the oracle on that input set.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from lossless_rejection_sampling_verify_amd import workloads as wl

from test_gpu_parity import _api, compare, dev, dev_logits, say, torch

pytestmark = pytest.mark.gpu


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                      # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_chain_and_greedy_replays():
    api = _api()
    sets = [wl.make_chain(2, seed=s, B=16, G=4, V=32000) for s in (51, 52, 53)]
    c0 = sets[0]
    lg = dev_logits(c0.logits, c0.dtype)
    q, x, xg = dev(c0.draft_probs), dev(c0.draft_tokens), dev(c0.greedy_tokens)
    u, T = dev(c0.coins), dev(c0.temperature)
    B, R = c0.B, c0.R
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty(B, R, dtype=torch.int32, device="cuda")
    probs = torch.empty(B, R, dtype=torch.float32, device="cuda")
    gacc = torch.empty(B, dtype=torch.int32, device="cuda")
    gout = torch.empty(B, R, dtype=torch.int32, device="cuda")

    def call():
        api.spec_verify_chain(lg, q, x, u, T, out=(acc, out, probs))
        api.spec_verify_greedy(lg, xg, out=(gacc, gout))

    g = _capture(call)
    for rep in range(2):
        for k, c in enumerate(sets):
            say(f"graph replay {rep} of input set {k}")
            lg.copy_(dev_logits(c.logits, c.dtype))
            q.copy_(dev(c.draft_probs))
            x.copy_(dev(c.draft_tokens))
            xg.copy_(dev(c.greedy_tokens))
            u.copy_(dev(c.coins))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            o = oracle.verify_chain(c.logits, c.dtype, c.draft_probs, c.draft_tokens, c.coins,
                                    c.temperature)
            compare(dict(accept_len=acc.cpu().numpy(), out_tokens=out.cpu().numpy(),
                         probs=probs.cpu().numpy()), o, ["accept_len", "out_tokens"],
                    o["margin"], label=f"chain replay {rep}/{k}")
            oa, oo = oracle.verify_greedy(c.logits, c.dtype, c.greedy_tokens)
            np.testing.assert_array_equal(gacc.cpu().numpy(), oa)
            np.testing.assert_array_equal(gout.cpu().numpy(), oo)


@pytest.mark.parametrize("kind", ["tree", "mss"])
def test_tree_replays(kind):
    api = _api()
    if kind == "tree":
        sets = [wl.make_tree(4, seed=s, B=8, N=24, V=20000, D=4, max_children=4) for s in (61, 62, 63)]
    else:
        sets = [wl.make_tree_mss(4, seed=s, B=8, N=24, V=20000, D=4, max_children=4)
                for s in (61, 62, 63)]
    t0 = sets[0]
    lg = dev_logits(t0.logits, t0.dtype)
    tok, par, cn, T = dev(t0.node_tokens), dev(t0.parents), dev(t0.coins), dev(t0.temperature)
    qd = dev(t0.draft_probs) if kind == "mss" else None
    B, D = t0.B, t0.D
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty(B, D + 1, dtype=torch.int32, device="cuda")
    nodes = torch.empty(B, D, dtype=torch.int32, device="cuda")
    probs = torch.empty(B, D + 1, dtype=torch.float32, device="cuda")

    def call():
        if kind == "tree":
            api.spec_verify_tree(lg, tok, par, cn, T, D, oracle.TREE_SAMPLING,
                                 out=(acc, out, nodes, probs))
        else:
            api.spec_verify_tree_mss(lg, qd, tok, par, cn, T, D, out=(acc, out, nodes, probs))

    g = _capture(call)
    for rep in range(2):
        for k, t in enumerate(sets):
            say(f"graph replay {rep} of {kind} input set {k}")
            lg.copy_(dev_logits(t.logits, t.dtype))
            tok.copy_(dev(t.node_tokens))
            par.copy_(dev(t.parents))
            cn.copy_(dev(t.coins))
            if qd is not None:
                qd.copy_(dev(t.draft_probs))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            if kind == "tree":
                o = oracle.verify_tree(t.logits, t.dtype, t.node_tokens, t.parents, t.coins,
                                       t.temperature, D, oracle.TREE_SAMPLING)
            else:
                o = oracle.verify_tree_mss(t.logits, t.dtype, t.draft_probs, t.node_tokens,
                                           t.parents, t.coins, t.temperature, D)
            compare(dict(accept_len=acc.cpu().numpy(), out_tokens=out.cpu().numpy(),
                         accepted_nodes=nodes.cpu().numpy(), probs=probs.cpu().numpy()), o,
                    ["accept_len", "out_tokens", "accepted_nodes"], o["margin"],
                    label=f"{kind} replay {rep}/{k}")


def test_filtered_chain_replays():
    """The chain verify from draft logits with top-k / top-p, captured once and replayed on
    input sets whose rows, drafts and coins differ (the knobs stay those of the capture)."""
    api = _api()
    sets = [wl.make_chain_logits(2, seed=s, B=12, G=3, V=20000, top_k=40, top_p=0.85)
            for s in (71, 72, 73)]
    c0 = sets[0]
    lg, dl = dev_logits(c0.logits, c0.dtype), dev_logits(c0.draft_logits, c0.dtype)
    x, u, T = dev(c0.draft_tokens), dev(c0.coins), dev(c0.temperature)
    B, R = c0.B, c0.R
    tk = dev(np.asarray(np.broadcast_to(c0.top_k, (B,)), np.int32).copy())
    tp = dev(np.asarray(np.broadcast_to(c0.top_p, (B,)), np.float32).copy())
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty(B, R, dtype=torch.int32, device="cuda")
    probs = torch.empty(B, R, dtype=torch.float32, device="cuda")

    def call():
        api.spec_verify_chain_filtered(lg, dl, x, u, T, tk, tp, out=(acc, out, probs))

    g = _capture(call)
    for rep in range(2):
        for k, c in enumerate(sets):
            say(f"graph replay {rep} of filtered input set {k}")
            lg.copy_(dev_logits(c.logits, c.dtype))
            dl.copy_(dev_logits(c.draft_logits, c.dtype))
            x.copy_(dev(c.draft_tokens))
            u.copy_(dev(c.coins))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            o = oracle.verify_chain_filtered(c.logits, c.draft_logits, c.dtype, c.draft_tokens,
                                             c.coins, c.temperature, c.top_k, c.top_p)
            compare(dict(accept_len=acc.cpu().numpy(), out_tokens=out.cpu().numpy(),
                         probs=probs.cpu().numpy()), o, ["accept_len", "out_tokens"],
                    o["margin"], label=f"filtered replay {rep}/{k}")
