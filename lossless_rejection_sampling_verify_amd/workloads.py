"""Seeded synthetic inputs for the batched speculative-decoding verify step.

This module only *draws* inputs, the way a serving system would hand them to the
verifier: target logits for every verified position (or every tree node), the draft
distribution q and the drafted tokens, a token tree as a parent array, uniform coins
and a per-request temperature.  It holds none of the verify arithmetic (no acceptance
test, no residual, no inverse-CDF draw, no tree walk); both the fp64 CPU oracle and
the HIP library consume exactly the arrays produced here.

The five named workloads follow the verify problem as the pages state it: target logits
over gamma+1 positions from one target forward (atlas "Speculative Decoding", section 0)
and draft tokens x ~ q with the draft distribution q (ricardokevins "Speculative
Decoding", section on correction sampling; zdszero spec_origins, "Speculative Decoding",
acceptance rule).  The trees are flattened token trees described by a parent relation
(zdszero spec_origins, SpecInfer, tree attention mask), with drafts taken as the top-k
of perturbed logits, as EAGLE-style drafters emit (spec_origins, "in SGLang").

Value distributions: logits ~ N(0, sigma^2), optionally with a block of boosted ids per
row; draft logits = target logits + N(0, var); q = softmax(draft / T) computed in fp64
and stored as fp32; x ~ q drawn by numpy's categorical sampler.  bf16 logits are the
fp32 draws rounded to nearest-even and stored as raw uint16 bit patterns.  Coins are
(k+1)/2^24 with k uniform in [0, 2^24): every coin lies in (0, 1] and is exact in fp32.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F32 = "f32"
BF16 = "bf16"

# Named workloads.  Shapes and distributions follow the five configurations the
# verify path is measured on; "G" is the speculation length gamma, "N" counts tree
# nodes including the root, "D" is the maximum tree depth.
CONFIGS = {
    1: dict(kind="chain", name="tiny-chain B=1 G=4 V=32 fp32",
            B=1, G=4, V=32, dtype=F32, sigma=2.0, boost=None, draft_var=1.0, T=1.0),
    2: dict(kind="chain", name="chain B=8 G=4 V=32000 fp32",
            B=8, G=4, V=32000, dtype=F32, sigma=3.0, boost=None, draft_var=1.0, T=1.0),
    3: dict(kind="chain", name="chain B=64 G=8 V=128256 bf16 T=0.7 boosted",
            B=64, G=8, V=128256, dtype=BF16, sigma=3.0, boost=(32, 8.0), draft_var=1.5, T=0.7),
    4: dict(kind="tree", name="tree B=32 N=64 D=6 V=128256 bf16",
            B=32, N=64, D=6, max_children=8, V=128256, dtype=BF16, sigma=3.0, T=1.0),
    5: dict(kind="chain", name="large-batch B=256 G=4 V=152064 bf16",
            B=256, G=4, V=152064, dtype=BF16, sigma=3.0, boost=None, draft_var=1.0, T=1.0),
}

COIN_BITS = 24


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def logits_as_f32(logits: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(logits) if dtype == BF16 else np.asarray(logits, dtype=np.float32)


def draw_coins(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform coins on the lattice (k+1)/2^24, k in [0, 2^24): all in (0, 1], exact in fp32."""
    k = rng.integers(0, 1 << COIN_BITS, size=shape, dtype=np.int64)
    return ((k + 1).astype(np.float64) / float(1 << COIN_BITS)).astype(np.float32)


def _streams(tag: int, seed: int, n: int):
    ss = np.random.SeedSequence([int(tag), int(seed)])
    return [np.random.default_rng(s) for s in ss.spawn(n)]


def _draft_distribution(draft_logits: np.ndarray, T: float) -> np.ndarray:
    """The draft model's distribution at temperature T, fp64 (input synthesis only)."""
    z = draft_logits.astype(np.float64) / float(T)
    z -= z.max(axis=-1, keepdims=True)
    np.exp(z, out=z)
    z /= z.sum(axis=-1, keepdims=True)
    return z


@dataclass
class ChainInputs:
    name: str
    B: int
    G: int
    V: int
    dtype: str
    logits: np.ndarray          # [B][G+1][V] float32, or uint16 bf16 bits
    draft_probs: np.ndarray     # [B][G][V] float32
    draft_tokens: np.ndarray    # [B][G] int32, x_i ~ q_i
    greedy_tokens: np.ndarray   # [B][G] int32, x_i = argmax of the draft logits
    coins: np.ndarray           # [B][G+1] float32 in (0, 1]
    temperature: np.ndarray     # [B] float32
    meta: dict = field(default_factory=dict)

    @property
    def R(self) -> int:
        return self.G + 1


@dataclass
class TreeInputs:
    name: str
    B: int
    N: int
    V: int
    D: int
    dtype: str
    logits: np.ndarray          # [B][N][V]; row j = target distribution after node j
    node_tokens: np.ndarray     # [B][N] int32; [b][0] is the root (unused)
    parents: np.ndarray         # [B][N] int32; [b][0] = -1, parents[b][i] < i
    coins: np.ndarray           # [B][D+1] float32 in (0, 1]
    temperature: np.ndarray     # [B] float32
    meta: dict = field(default_factory=dict)


def _target_rows(rng, rows: int, V: int, sigma: float, boost, dtype: str, chunk: int = 256):
    """Target logits ~ N(0, sigma^2) (+ boost on a few distinct ids per row), as stored dtype."""
    out = np.empty((rows, V), dtype=np.uint16 if dtype == BF16 else np.float32)
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        x = rng.standard_normal((r1 - r0, V), dtype=np.float32)
        x *= np.float32(sigma)
        if boost is not None:
            nb, amount = boost
            for r in range(r1 - r0):
                ids = rng.choice(V, size=nb, replace=False)
                x[r, ids] += np.float32(amount)
        out[r0:r1] = f32_to_bf16_bits(x) if dtype == BF16 else x
    return out


def make_chain(cfg_id: int = 2, seed: int = 0, *, B: int | None = None, G: int | None = None,
               V: int | None = None, dtype: str | None = None, T: float | None = None,
               sigma: float | None = None, draft_var: float | None = None,
               boost="cfg") -> ChainInputs:
    """Chain-verify inputs for workload ``cfg_id``; keyword overrides give scaled variants."""
    c = dict(CONFIGS[cfg_id])
    if c["kind"] != "chain":
        raise ValueError(f"workload {cfg_id} is not a chain workload")
    B = c["B"] if B is None else B
    G = c["G"] if G is None else G
    V = c["V"] if V is None else V
    dtype = c["dtype"] if dtype is None else dtype
    T = c["T"] if T is None else T
    sigma = c["sigma"] if sigma is None else sigma
    draft_var = c["draft_var"] if draft_var is None else draft_var
    boost = c["boost"] if boost == "cfg" else boost
    if boost is not None:
        boost = (min(boost[0], V), boost[1])
    r_logits, r_noise, r_draft, r_coins, _ = _streams(cfg_id, seed, 5)

    R = G + 1
    logits = _target_rows(r_logits, B * R, V, sigma, boost, dtype).reshape(B, R, V)
    draft_probs = np.empty((B, G, V), dtype=np.float32)
    draft_tokens = np.empty((B, G), dtype=np.int32)
    greedy_tokens = np.empty((B, G), dtype=np.int32)
    sd = np.float32(np.sqrt(draft_var))
    for b in range(B):
        tgt = logits_as_f32(logits[b, :G], dtype)                  # [G][V]
        d = tgt + r_noise.standard_normal((G, V), dtype=np.float32) * sd
        greedy_tokens[b] = np.argmax(d, axis=-1)
        q64 = _draft_distribution(d, T)
        draft_probs[b] = q64.astype(np.float32)
        for i in range(G):
            draft_tokens[b, i] = r_draft.choice(V, p=q64[i])
    coins = draw_coins(r_coins, (B, R))
    temperature = np.full((B,), T, dtype=np.float32)
    return ChainInputs(name=c["name"] if (B, G, V) == (c["B"], c["G"], c["V"]) else
                       f"chain B={B} G={G} V={V} {dtype} (from workload {cfg_id})",
                       B=B, G=G, V=V, dtype=dtype, logits=logits, draft_probs=draft_probs,
                       draft_tokens=draft_tokens, greedy_tokens=greedy_tokens, coins=coins,
                       temperature=temperature,
                       meta=dict(cfg=cfg_id, seed=seed, sigma=sigma, draft_var=draft_var,
                                 boost=boost, T=T))


def _random_tree(rng, N: int, D: int, max_children: int):
    """Parent array of an N-node tree (node 0 = root) with depth exactly D (when N > D).

    Nodes 1..D form a spine so the tree reaches depth D; every other node attaches to a
    uniformly chosen existing node of depth < D with fewer than ``max_children``
    children.  The result is renumbered breadth-first, children in creation order, so
    siblings are contiguous and parents[i] < i.
    """
    parent = [-1]
    depth = [0]
    nchild = [0]
    spine = min(D, N - 1)
    for i in range(1, spine + 1):
        parent.append(i - 1)
        depth.append(depth[i - 1] + 1)
        nchild.append(0)
        nchild[i - 1] += 1
    while len(parent) < N:
        cand = [j for j in range(len(parent)) if depth[j] < D and nchild[j] < max_children]
        if not cand:
            raise ValueError("tree shape cannot hold N nodes")
        p = cand[int(rng.integers(0, len(cand)))]
        parent.append(p)
        depth.append(depth[p] + 1)
        nchild.append(0)
        nchild[p] += 1
    children = [[] for _ in range(N)]
    for i in range(1, N):
        children[parent[i]].append(i)
    order = [0]
    for j in order:
        order.extend(children[j])
    new_id = {old: new for new, old in enumerate(order)}
    parents = np.full(N, -1, dtype=np.int32)
    for old in range(1, N):
        parents[new_id[old]] = new_id[parent[old]]
    return parents


def make_tree(cfg_id: int = 4, seed: int = 0, *, B: int | None = None, N: int | None = None,
              V: int | None = None, D: int | None = None, max_children: int | None = None,
              dtype: str | None = None, T: float | None = None,
              sigma: float | None = None) -> TreeInputs:
    """Token-tree verify inputs; node j's children carry the top-k tokens of row j + N(0,1)."""
    c = dict(CONFIGS[cfg_id])
    if c["kind"] != "tree":
        raise ValueError(f"workload {cfg_id} is not a tree workload")
    B = c["B"] if B is None else B
    N = c["N"] if N is None else N
    V = c["V"] if V is None else V
    D = c["D"] if D is None else D
    max_children = c["max_children"] if max_children is None else max_children
    dtype = c["dtype"] if dtype is None else dtype
    T = c["T"] if T is None else T
    sigma = c["sigma"] if sigma is None else sigma
    r_logits, r_noise, _, r_coins, r_tree = _streams(cfg_id, seed, 5)

    logits = _target_rows(r_logits, B * N, V, sigma, None, dtype).reshape(B, N, V)
    parents = np.empty((B, N), dtype=np.int32)
    node_tokens = np.full((B, N), -1, dtype=np.int32)
    for b in range(B):
        par = _random_tree(r_tree, N, D, max_children)
        parents[b] = par
        for j in range(N):
            kids = np.nonzero(par == j)[0]
            if len(kids) == 0:
                continue
            if len(kids) > V:
                raise ValueError("more children than vocabulary entries")
            pert = logits_as_f32(logits[b, j], dtype) + r_noise.standard_normal(V, dtype=np.float32)
            top = np.argpartition(-pert, len(kids) - 1)[: len(kids)]
            top = top[np.argsort(-pert[top], kind="stable")]
            node_tokens[b, kids] = top.astype(np.int32)
    coins = draw_coins(r_coins, (B, D + 1))
    temperature = np.full((B,), T, dtype=np.float32)
    full = (B, N, V, D) == (c["B"], c["N"], c["V"], c["D"])
    return TreeInputs(name=c["name"] if full else f"tree B={B} N={N} D={D} V={V} {dtype}",
                      B=B, N=N, V=V, D=D, dtype=dtype, logits=logits, node_tokens=node_tokens,
                      parents=parents, coins=coins, temperature=temperature,
                      meta=dict(cfg=cfg_id, seed=seed, sigma=sigma, T=T,
                                max_children=max_children))


@dataclass
class TreeMssInputs:
    name: str
    B: int
    N: int
    V: int
    D: int
    dtype: str
    logits: np.ndarray          # [B][N][V]; row j = target distribution after node j
    draft_probs: np.ndarray     # [B][N][V] float32; row j = draft distribution after node j
    node_tokens: np.ndarray     # [B][N] int32; children of j drawn i.i.d. from row j of q
    parents: np.ndarray         # [B][N] int32; [b][0] = -1, parents[b][i] < i
    coins: np.ndarray           # [B][N] float32 in (0, 1]; [c-1] tests node c, [N-1] final
    temperature: np.ndarray     # [B] float32
    meta: dict = field(default_factory=dict)


def make_tree_mss(cfg_id: int = 4, seed: int = 0, *, B: int | None = None, N: int | None = None,
                  V: int | None = None, D: int | None = None, max_children: int | None = None,
                  dtype: str | None = None, T: float | None = None, sigma: float | None = None,
                  draft_var: float = 1.0) -> TreeMssInputs:
    """Token-tree inputs with draft distributions: the tree workload's shapes, target rows
    and parent arrays, plus a draft row per node, q_j = softmax((row j + N(0, draft_var)) / T),
    from which the children of node j are drawn independently (with replacement)."""
    c = dict(CONFIGS[cfg_id])
    if c["kind"] != "tree":
        raise ValueError(f"workload {cfg_id} is not a tree workload")
    B = c["B"] if B is None else B
    N = c["N"] if N is None else N
    V = c["V"] if V is None else V
    D = c["D"] if D is None else D
    max_children = c["max_children"] if max_children is None else max_children
    dtype = c["dtype"] if dtype is None else dtype
    T = c["T"] if T is None else T
    sigma = c["sigma"] if sigma is None else sigma
    r_logits, r_noise, r_draft, r_coins, r_tree = _streams(100 + cfg_id, seed, 5)

    logits = _target_rows(r_logits, B * N, V, sigma, None, dtype).reshape(B, N, V)
    parents = np.empty((B, N), dtype=np.int32)
    node_tokens = np.full((B, N), -1, dtype=np.int32)
    q = np.empty((B, N, V), dtype=np.float32)
    sd = np.float32(np.sqrt(draft_var))
    for b in range(B):
        par = _random_tree(r_tree, N, D, max_children)
        parents[b] = par
        for j in range(N):
            d = logits_as_f32(logits[b, j], dtype) + sd * r_noise.standard_normal(V, dtype=np.float32)
            qj = _draft_distribution(d, T)
            q[b, j] = qj
            kids = np.nonzero(par == j)[0]
            if len(kids):
                cdf = np.cumsum(qj)
                u = r_draft.random(len(kids)) * cdf[-1]
                node_tokens[b, kids] = np.minimum(np.searchsorted(cdf, u, side="right"),
                                                  V - 1).astype(np.int32)
    coins = draw_coins(r_coins, (B, N))
    temperature = np.full((B,), T, dtype=np.float32)
    full = (B, N, V, D) == (c["B"], c["N"], c["V"], c["D"])
    return TreeMssInputs(name=(c["name"] + " with draft rows") if full
                         else f"tree B={B} N={N} D={D} V={V} {dtype} with draft rows",
                         B=B, N=N, V=V, D=D, dtype=dtype, logits=logits, draft_probs=q,
                         node_tokens=node_tokens, parents=parents, coins=coins,
                         temperature=temperature,
                         meta=dict(cfg=cfg_id, seed=seed, sigma=sigma, T=T,
                                   max_children=max_children, draft_var=draft_var))


@dataclass
class ChainLogitsInputs:
    name: str
    B: int
    G: int
    V: int
    dtype: str
    logits: np.ndarray          # [B][G+1][V] target logits (float32 or bf16 bits)
    draft_logits: np.ndarray    # [B][G][V] draft logits, same dtype
    draft_tokens: np.ndarray    # [B][G] int32, drawn by the drafter from its filtered q
    coins: np.ndarray           # [B][G+1] float32 in (0, 1]
    temperature: np.ndarray     # [B] float32
    top_k: np.ndarray           # [B] int32 (0: off)
    top_p: np.ndarray           # [B] float32 (1: off)

    @property
    def R(self) -> int:
        return self.G + 1


def _drafter_sample(rng, d_row: np.ndarray, T: float, k: int, top_p: float) -> int:
    """How a drafter with top-k / top-p sampling picks its token (input synthesis)."""
    z = d_row.astype(np.float64) / T
    z -= z.max()
    p = np.exp(z)
    if 0 < k < len(p):
        p[d_row < np.sort(d_row)[::-1][k - 1]] = 0.0
    p /= p.sum()
    if top_p < 1.0:
        order = np.sort(p)[::-1]
        tau = order[np.searchsorted(np.cumsum(order), top_p)]
        p[p < tau] = 0.0
        p /= p.sum()
    return int(rng.choice(len(p), p=p))


def make_chain_logits(cfg_id: int = 5, seed: int = 0, *, B: int | None = None,
                      G: int | None = None, V: int | None = None, dtype: str | None = None,
                      T: float | None = None, top_k=0, top_p=1.0) -> ChainLogitsInputs:
    """Chain inputs with the draft as logits (draft = target + N(0, var) noise, stored in the
    target's dtype) and drafts sampled with the given top-k / top-p (scalars or [B])."""
    c = dict(CONFIGS[cfg_id])
    B = c["B"] if B is None else B
    G = c["G"] if G is None else G
    V = c["V"] if V is None else V
    dtype = c["dtype"] if dtype is None else dtype
    T = c["T"] if T is None else T
    r_logits, r_noise, r_draft, r_coins, _ = _streams(100 + cfg_id, seed, 5)
    R = G + 1
    logits = _target_rows(r_logits, B * R, V, c["sigma"], c.get("boost"), dtype).reshape(B, R, V)
    top_k = np.broadcast_to(np.asarray(top_k, np.int32), (B,)).copy()
    top_p = np.broadcast_to(np.asarray(top_p, np.float32), (B,)).copy()
    sd = np.float32(np.sqrt(c["draft_var"]))
    draft_logits = np.empty((B, G, V), dtype=logits.dtype)
    draft_tokens = np.empty((B, G), np.int32)
    for b in range(B):
        d = logits_as_f32(logits[b, :G], dtype) + r_noise.standard_normal((G, V), dtype=np.float32) * sd
        draft_logits[b] = f32_to_bf16_bits(d) if dtype == BF16 else d
        dw = logits_as_f32(draft_logits[b], dtype)
        for i in range(G):
            draft_tokens[b, i] = _drafter_sample(r_draft, dw[i], T, int(top_k[b]), float(top_p[b]))
    return ChainLogitsInputs(name=f"chain from draft logits B={B} G={G} V={V} {dtype}", B=B, G=G,
                             V=V, dtype=dtype, logits=logits, draft_logits=draft_logits,
                             draft_tokens=draft_tokens, coins=draw_coins(r_coins, (B, R)),
                             temperature=np.full((B,), T, np.float32), top_k=top_k, top_p=top_p)
