"""spec_verify_chain_filtered (HIP) vs the oracle on identical seeded inputs.

Bar per request: accept_len and emitted tokens bit-exact unless the oracle's decision
trace (acceptance tests, the top-p boundaries, the final draw) passes within 1e-6 of a
threshold; probabilities of emitted tokens within 1e-5 relative.  Covers the large-batch
shape (bf16, V=152064) with top-k, top-p, both and neither, top-k = 1, fp32 rows, a
ragged vocabulary (scalar head/tail and a partial last chunk), tie-heavy bf16 rows, and
invalid knobs.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from lossless_rejection_sampling_verify_amd import workloads as wl

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
BAND = 1e-6


def _api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_rejection_sampling_verify_amd import api
    return api


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_logits(a, dtype):
    a = np.ascontiguousarray(a)
    if dtype == wl.BF16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def check(c, label, top_k=None, top_p=None):
    api = _api()
    tk = c.top_k if top_k is None else top_k
    tp = c.top_p if top_p is None else top_p
    print(f"[gpu-case] filtered {label} B={c.B} G={c.G} V={c.V} {c.dtype}", flush=True)
    acc, out, probs = api.spec_verify_chain_filtered(
        dev_logits(c.logits, c.dtype), dev_logits(c.draft_logits, c.dtype), dev(c.draft_tokens),
        dev(c.coins), dev(c.temperature), dev(np.asarray(tk, np.int32)),
        dev(np.asarray(tp, np.float32)), want_probs=True)
    torch.cuda.synchronize()
    g = dict(accept_len=acc.cpu().numpy(), out_tokens=out.cpu().numpy(), probs=probs.cpu().numpy())
    o = oracle.verify_chain_filtered(c.logits, c.draft_logits, c.dtype, c.draft_tokens, c.coins,
                                     c.temperature, tk, tp)
    near = o["margin"] <= BAND
    mism = (g["accept_len"] != o["accept_len"]) | (g["out_tokens"] != o["out_tokens"]).any(1)
    bad = mism & ~near
    assert not bad.any(), (f"{label}: {int(bad.sum())} requests differ outside the band; first "
                           f"b={int(np.nonzero(bad)[0][0])}")
    ok = ~mism
    gp, op = g["probs"][ok].astype(np.float64), o["probs"][ok]
    big = np.abs(op) >= 1e-30
    rel = np.abs(gp[big] - op[big]) / np.abs(op[big])
    assert rel.size == 0 or rel.max() <= 1e-5, f"{label}: prob rel err {rel.max():.3g}"
    print(f"[gpu-case] {label}: near={int(near.sum())} near_mismatch={int((mism & near).sum())}",
          flush=True)
    return g, o


@pytest.mark.parametrize("k,p", [(0, 1.0), (50, 1.0), (0, 0.9), (20, 0.8), (1000, 0.95)])
def test_large_batch_shape(k, p):
    c = wl.make_chain_logits(5, seed=k + int(p * 100), B=24, top_k=k, top_p=p)
    check(c, f"V=152064 k={k} p={p}")


def test_top1_is_greedy():
    c = wl.make_chain_logits(5, seed=3, B=16, V=50000, dtype=wl.F32, top_k=1)
    g, _ = check(c, "top-1 fp32")
    dl = c.draft_logits.astype(np.float32)
    ga, go = oracle.verify_greedy(c.logits, c.dtype, np.argmax(dl, -1).astype(np.int32))
    np.testing.assert_array_equal(g["accept_len"], ga)


@pytest.mark.parametrize("dtype,V", [(wl.F32, 4099), (wl.BF16, 4099), (wl.BF16, 9), (wl.F32, 1)])
def test_ragged(dtype, V):
    c = wl.make_chain_logits(2, seed=V, B=12, G=3, V=V, dtype=dtype,
                             top_k=np.array([0, 3, 7, 1] * 3), top_p=np.array([1.0, 0.5, 0.9] * 4))
    check(c, f"ragged {dtype} V={V}")


def test_bf16_ties_and_mixed_knobs():
    c = wl.make_chain_logits(3, seed=11, B=32, G=6, V=30000, T=0.7,
                             top_k=np.arange(32) * 7, top_p=np.linspace(0.3, 1.0, 32))
    check(c, "boosted bf16, per-request knobs")


def test_invalid_knobs():
    c = wl.make_chain_logits(2, seed=2, B=6, G=2, V=2000, top_k=5, top_p=0.7)
    tp = np.array([0.7, 0.0, -1.0, np.nan, 1.5, 0.7], np.float32)
    g, o = check(c, "invalid top_p", top_p=tp)
    assert (g["accept_len"][[1, 2, 3]] == -1).all() and (g["accept_len"][[0, 4, 5]] >= 0).all()


@pytest.mark.parametrize("dtype", [wl.BF16, wl.F32])
def test_candidate_overflow_and_plateaus(dtype):
    """Rows whose top-k boundary sits on a wide plateau.  With 3000 tokens tied at the top,
    more candidates reach the lanes' lower bound than LDS holds, so the row is selected by
    the radix walk instead.  With 1500 tied tokens the direct selection keeps them all
    (ties at the k-th key are kept).  Target and draft plateaus either differ (every
    draft is rejected and the correction comes from the residual) or coincide, with the
    drafts on them (every draft is accepted).  Both must match the oracle."""
    import dataclasses
    c = wl.make_chain_logits(2, seed=21, B=8, G=3, V=40000, dtype=dtype, top_k=100, top_p=0.9)
    rng = np.random.default_rng(5)
    tl = wl.logits_as_f32(c.logits, dtype)
    dl = wl.logits_as_f32(c.draft_logits, dtype)
    enc = (lambda f: wl.f32_to_bf16_bits(f)) if dtype == wl.BF16 else (lambda f: f)
    for width in (3000, 1500):
        for shared in (False, True):
            t2, d2, x2 = tl.copy(), dl.copy(), c.draft_tokens.copy()
            for b in range(c.B):
                for i in range(c.R):
                    ids = rng.choice(c.V, size=width, replace=False)
                    t2[b, i, ids] = t2[b, i].max() + 1.0
                    if i < c.G:
                        dids = ids if shared else rng.choice(c.V, size=width, replace=False)
                        d2[b, i, dids] = d2[b, i].max() + 1.0
                        if shared:
                            x2[b, i] = ids[rng.integers(width)]
            c2 = dataclasses.replace(c, logits=enc(t2), draft_logits=enc(d2), draft_tokens=x2)
            g, o = check(c2, f"plateau of {width}, shared={shared}, {dtype}")
            if shared:
                assert (o["accept_len"] == c.G).all()


@pytest.mark.parametrize("dtype", [wl.BF16, wl.F32])
def test_top_keys_crowded_in_one_lane(dtype):
    """The row's eight largest logits sit in lane 0's first two 16-byte vectors (its first
    batch of the first pass): the lanes' maxima then bound the top-k loosely, and the
    second pass must still read that batch back (its recorded maximum reaches the bound)
    and match the oracle."""
    import dataclasses
    c = wl.make_chain_logits(2, seed=31, B=8, G=3, V=40000, dtype=dtype, top_k=50, top_p=0.9)
    kvec = 8 if dtype == wl.BF16 else 4
    ids = np.array([0, 1, 2, 3, 256 * kvec, 256 * kvec + 1, 256 * kvec + 2, 256 * kvec + 3])
    tl = wl.logits_as_f32(c.logits, dtype).copy()
    dl = wl.logits_as_f32(c.draft_logits, dtype).copy()
    enc = (lambda f: wl.f32_to_bf16_bits(f)) if dtype == wl.BF16 else (lambda f: f)
    for arr in (tl, dl):
        top = arr.max(axis=-1, keepdims=True)
        arr[..., ids] = top + np.arange(1, 9, dtype=np.float32)
    c2 = dataclasses.replace(c, logits=enc(tl), draft_logits=enc(dl))
    check(c2, f"top keys crowded in lane 0, {dtype}")


@pytest.mark.parametrize("dtype", [wl.BF16, wl.F32])
def test_signed_zero_at_the_top_k_boundary(dtype):
    """Rows whose top-k boundary is 0.0 with both signs of zero among the tied tokens:
    -0.0 and +0.0 compare equal, so every zero is kept (ties at the k-th logit), as in the
    oracle.  Target and draft share the plateau and the drafts sit on -0.0 tokens, so the
    kept set decides every acceptance."""
    import dataclasses
    c = wl.make_chain_logits(2, seed=41, B=8, G=3, V=4099, dtype=dtype, top_k=20, top_p=1.0)
    rng = np.random.default_rng(9)
    enc = (lambda f: wl.f32_to_bf16_bits(f)) if dtype == wl.BF16 else (lambda f: f)
    t = wl.logits_as_f32(c.logits, dtype)
    d = wl.logits_as_f32(c.draft_logits, dtype)
    t = (t - t.max(axis=-1, keepdims=True) - 1.0).astype(np.float32)  # every logit below 0
    d = (d - d.max(axis=-1, keepdims=True) - 1.0).astype(np.float32)
    x2 = c.draft_tokens.copy()
    for b in range(c.B):
        for i in range(c.R):
            ids = rng.choice(c.V, size=30, replace=False)
            t[b, i, ids[:18]] = 0.0
            t[b, i, ids[18:]] = -0.0
            if i < c.G:
                d[b, i, ids[:18]] = 0.0
                d[b, i, ids[18:]] = -0.0
                x2[b, i] = ids[20 + (b + i) % 10]                # a draft on a -0.0 token
    assert (np.signbit(t) & (t == 0)).sum() == c.B * c.R * 12
    c2 = dataclasses.replace(c, logits=enc(t), draft_logits=enc(d), draft_tokens=x2)
    g, o = check(c2, f"signed zeros at the top-k boundary, {dtype}")
    assert (o["accept_len"] >= 1).all()


@pytest.mark.parametrize("V", [152064, 131072 + 7])
def test_fp32_rows_beyond_the_batch_record(V):
    """fp32 rows of this length have more first-pass batches per lane than the record
    holds, so the second pass reads the whole row again."""
    c = wl.make_chain_logits(5, seed=V % 97, B=3, G=2, V=V, dtype=wl.F32, top_k=50, top_p=0.9)
    check(c, f"fp32 V={V} k=50 p=0.9")


@pytest.mark.parametrize("width", [200, 600, 1800])
def test_recorded_batches_beyond_the_list(width):
    """Long bf16 rows with `width` tied tokens at the top, scattered at random: every
    batch of the first pass that holds one of them is read back by the candidate pass.
    About 200 and 550 such batches fit the list that spreads their loads over the
    workgroup; about 1500 (width 1800) do not, and the lanes read their batches one by
    one instead.  200 candidates are ordered by rank, 600 and 1800 by the sorting
    network.  All must match the oracle."""
    import dataclasses
    c = wl.make_chain_logits(5, seed=width, B=4, G=2, top_k=100, top_p=0.9)
    rng = np.random.default_rng(width)
    tl = wl.logits_as_f32(c.logits, c.dtype).copy()
    dl = wl.logits_as_f32(c.draft_logits, c.dtype).copy()
    for b in range(c.B):
        for i in range(c.R):
            ids = rng.choice(c.V, size=width, replace=False)
            tl[b, i, ids] = tl[b, i].max() + 1.0
            if i < c.G:
                dids = rng.choice(c.V, size=width, replace=False)
                dl[b, i, dids] = dl[b, i].max() + 1.0
    c2 = dataclasses.replace(c, logits=wl.f32_to_bf16_bits(tl), draft_logits=wl.f32_to_bf16_bits(dl))
    check(c2, f"{width} tied top tokens scattered over V={c.V}")


def test_bench_shape():
    """The benchmark's filtered workload itself: B=256, G=4, V=152064 bf16, top-k 50 and
    top-p 0.9 for every request, at the launch configuration the benchmark times."""
    c = wl.make_chain_logits(5, top_k=50, top_p=0.9)
    assert c.B == 256
    check(c, "bench shape B=256 k=50 p=0.9")


def test_repeated_calls_are_bit_identical():
    """The candidates and the kept-token lists are filled in the order the atomics land, and
    the draw from a list sorts it by token id first: 20 calls on the same inputs (top-k 50
    with and without top-p, and top-k off, which takes the full draw) give the same bits."""
    api = _api()
    c = wl.make_chain_logits(5, seed=7, B=64, top_k=np.where(np.arange(64) % 3 == 2, 0, 50),
                             top_p=np.where(np.arange(64) % 2 == 0, 0.9, 1.0))
    args = (dev_logits(c.logits, c.dtype), dev_logits(c.draft_logits, c.dtype),
            dev(c.draft_tokens), dev(c.coins), dev(c.temperature),
            dev(np.asarray(c.top_k, np.int32)), dev(np.asarray(c.top_p, np.float32)))
    first = None
    for _ in range(20):
        out = [x.cpu().numpy() for x in api.spec_verify_chain_filtered(*args, want_probs=True)]
        if first is None:
            first = out
            continue
        for a, b in zip(first, out):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    check(c, "repeated calls, mixed knobs")
