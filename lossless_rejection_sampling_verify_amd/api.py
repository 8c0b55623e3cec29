"""Torch-facing binding of the verify library: same names as the C ABI.

PyTorch provides device memory and the current stream; every step of the verify runs in
the HIP kernels of ``libspecverify.so``.  Inputs must already be contiguous device tensors
of the documented dtypes (fp32 or bf16 logits, fp32 draft probabilities / coins /
temperatures, int32 tokens and parents); nothing is converted or computed here.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib as L

_WORKSPACES: dict = {}


def _check(t: torch.Tensor, name: str, dtype, dims: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dimensions, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _logit_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return L.SPEC_F32
    if t.dtype == torch.bfloat16:
        return L.SPEC_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _torch_stream(device, stream):
    return torch.cuda.current_stream(device) if stream is None else stream


def _stream(device, stream):
    return _torch_stream(device, stream).cuda_stream


def _opts(opts):
    o = L.options(opts)
    return None if o is None else ctypes.byref(o)


def workspace(op: int, B: int, R: int, V: int, device, stream=None) -> torch.Tensor:
    """A workspace big enough for the call, cached per device, kind and stream.

    Calls that may run at the same time need separate workspaces, and calls issued in
    order on one stream can share one, so the cache keeps one buffer per stream.  A buffer
    is allocated on the stream it serves and zero-filled there (the library keeps a call
    counter and per-request exit words in its header and leaves them ready for the next
    call).  When a call needs a larger one, the old buffer is released to torch's caching
    allocator, which hands that memory out again only in that stream's order, after the
    calls already enqueued on it."""
    need = L.workspace_bytes(op, B, R, V)
    if need == 0:
        raise ValueError("unsupported sizes")
    dev = torch.device(device)
    s = _torch_stream(dev, stream)
    key = (dev, op, s.cuda_stream)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < need:
        with torch.cuda.stream(s):
            ws = torch.zeros(max(need, 1 << 20), dtype=torch.uint8, device=dev)
        _WORKSPACES[key] = ws
    return ws


def spec_verify_greedy(logits: torch.Tensor, draft_tokens: torch.Tensor, *, ws=None,
                       stream=None, out=None, opts=None):
    """Greedy chain verify.  logits [B][G+1][V] fp32/bf16, draft_tokens [B][G] int32.
    ``opts``: launch options (a dict of spec_options fields, or None for the defaults).

    Returns (accept_len [B] int32, out_tokens [B][G+1] int32)."""
    _check(logits, "logits", (torch.float32, torch.bfloat16), 3)
    _check(draft_tokens, "draft_tokens", torch.int32, 2)
    B, R, V = logits.shape
    G = R - 1
    if draft_tokens.shape != (B, G):
        raise ValueError("draft_tokens must be [B][G]")
    dev = logits.device
    ws = workspace(L.SPEC_OP_GREEDY, B, R, V, dev, stream) if ws is None else ws
    if out is None:
        acc = torch.empty(B, dtype=torch.int32, device=dev)
        toks = torch.empty(B, R, dtype=torch.int32, device=dev)
    else:
        acc, toks = out
    rc = L.lib().spec_verify_greedy_opt(_ptr(logits), _logit_dtype(logits), _ptr(draft_tokens), B,
                                        G, V, _ptr(acc), _ptr(toks), _ptr(ws), ws.numel(),
                                        _stream(dev, stream), _opts(opts))
    if rc != L.SPEC_OK:
        raise L.SpecVerifyError("spec_verify_greedy", rc)
    return acc, toks


def spec_verify_chain(logits: torch.Tensor, draft_probs: torch.Tensor, draft_tokens: torch.Tensor,
                      coins: torch.Tensor, temperature: torch.Tensor, *, want_probs: bool = False,
                      ws=None, stream=None, out=None, opts=None):
    """Chain rejection sampling.  logits [B][G+1][V], draft_probs [B][G][V] fp32,
    draft_tokens [B][G] int32, coins [B][G+1] fp32, temperature [B] fp32.
    ``opts``: launch options (a dict of spec_options fields, or None for the defaults).

    Returns (accept_len [B], out_tokens [B][G+1], probs [B][G+1] or None)."""
    _check(logits, "logits", (torch.float32, torch.bfloat16), 3)
    _check(draft_probs, "draft_probs", torch.float32, 3)
    _check(draft_tokens, "draft_tokens", torch.int32, 2)
    _check(coins, "coins", torch.float32, 2)
    _check(temperature, "temperature", torch.float32, 1)
    B, R, V = logits.shape
    G = R - 1
    if draft_probs.shape != (B, G, V) or draft_tokens.shape != (B, G) or \
            coins.shape != (B, R) or temperature.shape != (B,):
        raise ValueError("inconsistent shapes")
    dev = logits.device
    ws = workspace(L.SPEC_OP_CHAIN, B, R, V, dev, stream) if ws is None else ws
    if out is None:
        acc = torch.empty(B, dtype=torch.int32, device=dev)
        toks = torch.empty(B, R, dtype=torch.int32, device=dev)
        probs = torch.empty(B, R, dtype=torch.float32, device=dev) if want_probs else None
    else:
        acc, toks, probs = out
    rc = L.lib().spec_verify_chain_opt(_ptr(logits), _logit_dtype(logits), _ptr(draft_probs),
                                       _ptr(draft_tokens), _ptr(coins), _ptr(temperature), B, G,
                                       V, _ptr(acc), _ptr(toks), _ptr(probs), _ptr(ws),
                                       ws.numel(), _stream(dev, stream), _opts(opts))
    if rc != L.SPEC_OK:
        raise L.SpecVerifyError("spec_verify_chain", rc)
    return acc, toks, probs


def spec_verify_chain_filtered(logits: torch.Tensor, draft_logits: torch.Tensor,
                               draft_tokens: torch.Tensor, coins: torch.Tensor,
                               temperature: torch.Tensor, top_k=None, top_p=None, *,
                               want_probs: bool = False, ws=None, stream=None, out=None):
    """Chain rejection sampling from draft logits with top-k / top-p filtering.
    logits [B][G+1][V] and draft_logits [B][G][V] (same dtype, fp32 or bf16),
    draft_tokens [B][G] int32, coins [B][G+1] fp32, temperature [B] fp32,
    top_k [B] int32 or None, top_p [B] fp32 or None.

    Returns (accept_len [B], out_tokens [B][G+1], probs [B][G+1] or None)."""
    _check(logits, "logits", (torch.float32, torch.bfloat16), 3)
    _check(draft_logits, "draft_logits", logits.dtype, 3)
    _check(draft_tokens, "draft_tokens", torch.int32, 2)
    _check(coins, "coins", torch.float32, 2)
    _check(temperature, "temperature", torch.float32, 1)
    B, R, V = logits.shape
    G = R - 1
    if draft_logits.shape != (B, G, V) or draft_tokens.shape != (B, G) or \
            coins.shape != (B, R) or temperature.shape != (B,):
        raise ValueError("inconsistent shapes")
    if top_k is not None:
        _check(top_k, "top_k", torch.int32, 1)
    if top_p is not None:
        _check(top_p, "top_p", torch.float32, 1)
    dev = logits.device
    ws = workspace(L.SPEC_OP_CHAIN_FILTERED, B, R, V, dev, stream) if ws is None else ws
    if out is None:
        acc = torch.empty(B, dtype=torch.int32, device=dev)
        toks = torch.empty(B, R, dtype=torch.int32, device=dev)
        probs = torch.empty(B, R, dtype=torch.float32, device=dev) if want_probs else None
    else:
        acc, toks, probs = out
    rc = L.lib().spec_verify_chain_filtered(_ptr(logits), _ptr(draft_logits), _logit_dtype(logits),
                                            _ptr(draft_tokens), _ptr(coins), _ptr(temperature),
                                            _ptr(top_k), _ptr(top_p), B, G, V, _ptr(acc),
                                            _ptr(toks), _ptr(probs), _ptr(ws), ws.numel(),
                                            _stream(dev, stream))
    if rc != L.SPEC_OK:
        raise L.SpecVerifyError("spec_verify_chain_filtered", rc)
    return acc, toks, probs


def spec_verify_tree(logits: torch.Tensor, node_tokens: torch.Tensor, parents: torch.Tensor,
                     coins, temperature, D: int, mode: int, threshold_single: float = 1.0,
                     threshold_acc: float = 1.0, *, want_probs: bool = False, ws=None,
                     stream=None, out=None, opts=None):
    """Token-tree verify.  logits [B][N][V], node_tokens/parents [B][N] int32,
    coins [B][D+1] fp32 and temperature [B] fp32 (sampling mode; None in greedy mode).
    ``opts``: launch options (a dict of spec_options fields, or None for the defaults).

    Returns (accept_len [B], out_tokens [B][D+1], accepted_nodes [B][D], probs or None)."""
    _check(logits, "logits", (torch.float32, torch.bfloat16), 3)
    _check(node_tokens, "node_tokens", torch.int32, 2)
    _check(parents, "parents", torch.int32, 2)
    B, N, V = logits.shape
    if node_tokens.shape != (B, N) or parents.shape != (B, N):
        raise ValueError("node_tokens / parents must be [B][N]")
    if coins is not None:
        _check(coins, "coins", torch.float32, 2)
        if coins.shape != (B, D + 1):
            raise ValueError("coins must be [B][D+1]")
    if temperature is not None:
        _check(temperature, "temperature", torch.float32, 1)
    dev = logits.device
    ws = workspace(L.SPEC_OP_TREE, B, N, V, dev, stream) if ws is None else ws
    if out is None:
        acc = torch.empty(B, dtype=torch.int32, device=dev)
        toks = torch.empty(B, D + 1, dtype=torch.int32, device=dev)
        nodes = torch.empty(B, D, dtype=torch.int32, device=dev)
        probs = torch.empty(B, D + 1, dtype=torch.float32, device=dev) if want_probs else None
    else:
        acc, toks, nodes, probs = out
    rc = L.lib().spec_verify_tree_opt(_ptr(logits), _logit_dtype(logits), _ptr(node_tokens),
                                      _ptr(parents), _ptr(coins), _ptr(temperature), B, N, V, D,
                                      int(mode), float(threshold_single), float(threshold_acc),
                                      _ptr(acc), _ptr(toks), _ptr(nodes), _ptr(probs), _ptr(ws),
                                      ws.numel(), _stream(dev, stream), _opts(opts))
    if rc != L.SPEC_OK:
        raise L.SpecVerifyError("spec_verify_tree", rc)
    return acc, toks, nodes, probs


def spec_verify_tree_mss(logits: torch.Tensor, draft_probs: torch.Tensor,
                         node_tokens: torch.Tensor, parents: torch.Tensor, coins: torch.Tensor,
                         temperature: torch.Tensor, D: int, *, want_probs: bool = False, ws=None,
                         stream=None, out=None, opts=None):
    """Token-tree verify by multi-step speculative sampling.  logits [B][N][V],
    draft_probs [B][N][V] fp32 (row j: the distribution node j's children were drawn from),
    node_tokens/parents [B][N] int32, coins [B][N] fp32 (coins[b][c-1] tests node c,
    coins[b][N-1] the final draw), temperature [B] fp32.

    Returns (accept_len [B], out_tokens [B][D+1], accepted_nodes [B][D], probs or None)."""
    _check(logits, "logits", (torch.float32, torch.bfloat16), 3)
    _check(draft_probs, "draft_probs", torch.float32, 3)
    _check(node_tokens, "node_tokens", torch.int32, 2)
    _check(parents, "parents", torch.int32, 2)
    _check(coins, "coins", torch.float32, 2)
    _check(temperature, "temperature", torch.float32, 1)
    B, N, V = logits.shape
    if draft_probs.shape != (B, N, V):
        raise ValueError("draft_probs must be [B][N][V]")
    if node_tokens.shape != (B, N) or parents.shape != (B, N) or coins.shape != (B, N):
        raise ValueError("node_tokens / parents / coins must be [B][N]")
    if temperature.shape != (B,):
        raise ValueError("temperature must be [B]")
    dev = logits.device
    ws = workspace(L.SPEC_OP_TREE_MSS, B, N, V, dev, stream) if ws is None else ws
    if out is None:
        acc = torch.empty(B, dtype=torch.int32, device=dev)
        toks = torch.empty(B, D + 1, dtype=torch.int32, device=dev)
        nodes = torch.empty(B, D, dtype=torch.int32, device=dev)
        probs = torch.empty(B, D + 1, dtype=torch.float32, device=dev) if want_probs else None
    else:
        acc, toks, nodes, probs = out
    rc = L.lib().spec_verify_tree_mss_opt(_ptr(logits), _logit_dtype(logits), _ptr(draft_probs),
                                          _ptr(node_tokens), _ptr(parents), _ptr(coins),
                                          _ptr(temperature), B, N, V, D, _ptr(acc), _ptr(toks),
                                          _ptr(nodes), _ptr(probs), _ptr(ws), ws.numel(),
                                          _stream(dev, stream), _opts(opts))
    if rc != L.SPEC_OK:
        raise L.SpecVerifyError("spec_verify_tree_mss", rc)
    return acc, toks, nodes, probs


def spec_tree_mask(parents: torch.Tensor, base_pos=None, *, want_positions: bool = True,
                   stream=None, out=None):
    """Tree attention mask.  parents [B][N] int32, base_pos [B] int32 or None.

    Returns (mask [B][N][ceil(N/32)] int32 holding the uint32 bit rows,
    positions [B][N] int32 or None)."""
    _check(parents, "parents", torch.int32, 2)
    B, N = parents.shape
    if base_pos is not None:
        _check(base_pos, "base_pos", torch.int32, 1)
        if base_pos.shape != (B,):
            raise ValueError("base_pos must be [B]")
    dev = parents.device
    W = (N + 31) // 32
    if out is None:
        mask = torch.empty(B, N, W, dtype=torch.int32, device=dev)
        pos = torch.empty(B, N, dtype=torch.int32, device=dev) if want_positions else None
    else:
        mask, pos = out
    rc = L.lib().spec_tree_mask(_ptr(parents), _ptr(base_pos), B, N, _ptr(mask), _ptr(pos),
                                _stream(dev, stream))
    if rc != L.SPEC_OK:
        raise L.SpecVerifyError("spec_tree_mask", rc)
    return mask, pos


def spec_tree_commit_kv(accepted_nodes: torch.Tensor, accept_len: torch.Tensor,
                        kv_tree: torch.Tensor, kv_out: torch.Tensor, *, want_slots: bool = True,
                        stream=None, slots=None):
    """Commit the accepted tree path.  accepted_nodes [B][D], accept_len [B] int32;
    kv_tree [B][N][...] and kv_out [B][D+1][...] contiguous, same dtype and row size
    (kv_out is written in place).  Returns slots [B][D+1] int32 or None."""
    _check(accepted_nodes, "accepted_nodes", torch.int32, 2)
    _check(accept_len, "accept_len", torch.int32, 1)
    if not (kv_tree.is_contiguous() and kv_out.is_contiguous()):
        raise ValueError("kv_tree and kv_out must be contiguous")
    if kv_tree.device.type != "cuda" or kv_out.device.type != "cuda":
        raise ValueError("kv_tree and kv_out must be device tensors")
    B, D = accepted_nodes.shape
    if accept_len.shape != (B,) or kv_tree.dim() < 2 or kv_out.dim() < 2 or \
            kv_tree.shape[0] != B or kv_out.shape[:2] != (B, D + 1) or kv_tree.dtype != kv_out.dtype:
        raise ValueError("inconsistent shapes")
    N = kv_tree.shape[1]
    row_bytes = kv_tree[0, 0].numel() * kv_tree.element_size()
    if kv_out[0, 0].numel() * kv_out.element_size() != row_bytes:
        raise ValueError("kv_tree and kv_out rows differ in size")
    dev = accepted_nodes.device
    if slots is None and want_slots:
        slots = torch.empty(B, D + 1, dtype=torch.int32, device=dev)
    rc = L.lib().spec_tree_commit_kv(_ptr(accepted_nodes), _ptr(accept_len), B, D, N,
                                     _ptr(kv_tree), _ptr(kv_out), row_bytes, _ptr(slots),
                                     _stream(dev, stream))
    if rc != L.SPEC_OK:
        raise L.SpecVerifyError("spec_tree_commit_kv", rc)
    return slots


def spec_calib_read(data: torch.Tensor, sink: torch.Tensor, *, stream=None):
    """Read-bandwidth calibration: streams every byte of the contiguous device tensor
    `data` (16-byte aligned, nbytes a multiple of 16).  `sink` is a one-element fp32
    device tensor the kernel writes only on an impossible sentinel."""
    if data.device.type != "cuda" or not data.is_contiguous():
        raise ValueError("data must be a contiguous device tensor")
    _check(sink, "sink", torch.float32, 1)
    rc = L.lib().spec_calib_read(_ptr(data), data.numel() * data.element_size(), _ptr(sink),
                                 _stream(data.device, stream))
    if rc != L.SPEC_OK:
        raise L.SpecVerifyError("spec_calib_read", rc)


def spec_calib_exp(blocks: int, iters: int, sink: torch.Tensor, *, stream=None):
    """Exponential-throughput calibration: blocks * 256 * iters * 8 v_exp_f32."""
    _check(sink, "sink", torch.float32, 1)
    rc = L.lib().spec_calib_exp(int(blocks), int(iters), _ptr(sink), _stream(sink.device, stream))
    if rc != L.SPEC_OK:
        raise L.SpecVerifyError("spec_calib_exp", rc)
