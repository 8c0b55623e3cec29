#!/usr/bin/env python3
"""Benchmark of the batched speculative-decoding verify step on one MI355X.

One step = one pass of the whole chain/greedy verify path over the large-batch workload
(B=256 requests, gamma=4, V=152064, bf16 target logits ~ N(0, 3^2), draft = target +
N(0,1), T=1): spec_verify_greedy and spec_verify_chain on the same batch.  Inputs are
synthetic, seeded, and resident in HBM before timing starts; three copies rotate so
consecutive steps never find the logits in the 256 MB Infinity Cache.

Prints ONE JSON line: verified positions/s (whole step), the roofline of the dominant
call (spec_verify_chain: algorithmic HBM bytes per call / call time measured with HIP
events on the launch stream), and the CPU oracle timed on a bounded sample of the same
workload.

Both calls walk each request position by position and stop at the first rejection (or
mismatch), so the algorithmic bytes of a call are the rows the method consults: for
request b, rows 0..k_b of its logits, plus the fp32 draft row at k_b when the chain
rejected there.  The eager passes (every row streamed), selected with
SPEC_VERIFY_EAGER=1, are timed after the main region and reported under
modes.*_eager with their own bytes (every row once).

HBM traffic: two rocprofv3 counter passes over this script (FETCH_SIZE, then WRITE_SIZE,
with --calib-copy-mib so that a plain device copy of known size runs after the timed
region) are reduced by ``bench.py --traffic-from FETCH_DIR WRITE_DIR``, which scales each
counter by what it reads for the copy and writes profiles/traffic.json; later runs report
that traffic while the kernel source is unchanged (its hash is stored with it).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, AMD published peak
CHAIN_KERNELS = ["k_chain_walk"]  # the final draw runs inside the walk (k_draw only past 64 chunks a slice)
GREEDY_KERNELS = ["k_greedy_walk"]
EAGER_CHAIN_KERNELS = ["k_rows<sampling>", "k_chain_accept", "k_mass", "k_draw"]
EAGER_GREEDY_KERNELS = ["k_rows<greedy>", "k_greedy_merge"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=5, choices=[2, 3, 5])
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--tree", action="store_true", help="also time the tree workload")
    ap.add_argument("--filtered", action="store_true",
                    help="also time chain verify from draft logits with top-k 50 / top-p 0.9")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"))
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, copy a buffer of this many MiB 3 times (counter scale)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="reduce two rocprofv3 --pmc runs (csv) into --traffic-json and exit")
    return ap.parse_args()


def main():
    args = parse()
    if args.traffic_from:
        _traffic_from(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the verify path is single-GPU here)", file=sys.stderr)
        sys.exit(2)

    import torch

    import lossless_rejection_sampling_verify_amd as pkg
    from lossless_rejection_sampling_verify_amd import _lib as L
    from lossless_rejection_sampling_verify_amd import api
    from lossless_rejection_sampling_verify_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    c = wl.make_chain(args.workload)
    gen_s = time.time() - t0
    B, G, V, R = c.B, c.G, c.V, c.R
    esize = 2 if c.dtype == wl.BF16 else 4

    def logits_dev(a):
        a = np.ascontiguousarray(a)
        if c.dtype == wl.BF16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    base = dict(logits=logits_dev(c.logits), q=torch.from_numpy(c.draft_probs).to(dev),
                x=torch.from_numpy(c.draft_tokens).to(dev), xg=torch.from_numpy(c.greedy_tokens).to(dev),
                u=torch.from_numpy(c.coins).to(dev), T=torch.from_numpy(c.temperature).to(dev))
    copies = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(args.copies - 1)]
    ws_g = api.workspace(L.SPEC_OP_GREEDY, B, R, V, dev)
    ws_c = api.workspace(L.SPEC_OP_CHAIN, B, R, V, dev)
    out_g = (torch.empty(B, dtype=torch.int32, device=dev), torch.empty(B, R, dtype=torch.int32, device=dev))
    out_c = (torch.empty(B, dtype=torch.int32, device=dev), torch.empty(B, R, dtype=torch.int32, device=dev),
             torch.empty(B, R, dtype=torch.float32, device=dev))
    stream = torch.cuda.current_stream(dev)

    def step(i, ev=None):
        d = copies[i % len(copies)]
        if ev is not None:
            ev[0].record(stream)
        api.spec_verify_greedy(d["logits"], d["xg"], ws=ws_g, out=out_g)
        if ev is not None:
            ev[1].record(stream)
        api.spec_verify_chain(d["logits"], d["q"], d["x"], d["u"], d["T"], ws=ws_c, out=out_c)
        if ev is not None:
            ev[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, synchronised on both sides
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start

    greedy_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    chain_ms = np.array([e[1].elapsed_time(e[2]) for e in events])
    acc_c = out_c[0].cpu().numpy()
    acc_g = out_g[0].cpu().numpy()
    rejected = int((acc_c < G).sum())

    small_g = B * G * 4 + B * 4 + B * R * 4                          # drafts, outputs
    small_c = (B * (G + R + 1) * 4 + B * G * 4 +                     # tokens, coins, T, q gathers
               B * 4 + 2 * B * R * 4)                                # outputs
    # the rows each request consults, and the draft row where the chain rejected
    greedy_bytes = int((acc_g + 1).sum()) * V * esize + small_g
    chain_bytes = int((acc_c + 1).sum()) * V * esize + rejected * V * 4 + small_c
    positions = 2 * B * R
    value = positions * args.steps / elapsed

    chain_gbs = chain_bytes / (chain_ms.mean() * 1e-3) / 1e9
    greedy_gbs = greedy_bytes / (greedy_ms.mean() * 1e-3) / 1e9

    # the eager passes, for comparison (outside the timed region)
    os.environ["SPEC_VERIFY_EAGER"] = "1"
    for i in range(3):
        step(i)
    torch.cuda.synchronize()
    ev_e = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(20)]
    for i in range(20):
        step(i, ev_e[i])
    torch.cuda.synchronize()
    del os.environ["SPEC_VERIFY_EAGER"]
    greedy_e = np.array([e[0].elapsed_time(e[1]) for e in ev_e])
    chain_e = np.array([e[1].elapsed_time(e[2]) for e in ev_e])
    eager_g_bytes = B * R * V * esize + small_g
    eager_c_bytes = B * R * V * esize + rejected * V * 4 + small_c

    traffic = None
    if os.path.exists(args.traffic_json):
        tj = json.load(open(args.traffic_json))
        if tj.get("workload") == c.name and tj.get("kernel_source_sha") == _source_sha():
            traffic = tj.get("calls", {}).get("spec_verify_chain", {}).get("bytes")

    result = {
        "metric": "verified positions/sec and logit-read GB/s (% of HBM peak), 1 MI355X",
        "value": value,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if c.dtype == wl.BF16 else "f32",
        "data": "synthetic (seeded; shapes and distributions of the large-batch workload)",
        "config": {"workload": c.name, "B": B, "gamma": G, "V": V, "positions_per_step": positions,
                   "step": "spec_verify_greedy + spec_verify_chain", "input_copies": args.copies},
        "roofline": {
            "bound": "hbm",
            "kernel": "spec_verify_chain call: " + " + ".join(CHAIN_KERNELS) +
                      " (bytes: rows consulted up to the first rejection, plus its draft row)",
            "achieved": chain_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": chain_gbs / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": chain_bytes,
            "avg_launch_ms": float(chain_ms.mean()),
        },
        "modes": {
            "greedy": {"avg_ms": float(greedy_ms.mean()), "p90_ms": float(np.percentile(greedy_ms, 90)),
                       "GB/s": greedy_gbs, "frac": greedy_gbs / HBM_PEAK_GBS,
                       "positions/s": B * R / (greedy_ms.mean() * 1e-3),
                       "rows_consulted": int((acc_g + 1).sum()),
                       "tokens/s": float((acc_g + 1).sum()) / (greedy_ms.mean() * 1e-3)},
            "chain": {"avg_ms": float(chain_ms.mean()), "p90_ms": float(np.percentile(chain_ms, 90)),
                      "GB/s": chain_gbs, "frac": chain_gbs / HBM_PEAK_GBS,
                      "positions/s": B * R / (chain_ms.mean() * 1e-3),
                      "rejected_requests": rejected,
                      "rows_consulted": int((acc_c + 1).sum()),
                      "tokens/s": float((acc_c + 1).sum()) / (chain_ms.mean() * 1e-3)},
            "greedy_eager": {"avg_ms": float(greedy_e.mean()), "bytes": eager_g_bytes,
                             "GB/s": eager_g_bytes / (greedy_e.mean() * 1e-3) / 1e9,
                             "frac": eager_g_bytes / (greedy_e.mean() * 1e-3) / 1e9 / HBM_PEAK_GBS},
            "chain_eager": {"avg_ms": float(chain_e.mean()), "bytes": eager_c_bytes,
                            "GB/s": eager_c_bytes / (chain_e.mean() * 1e-3) / 1e9,
                            "frac": eager_c_bytes / (chain_e.mean() * 1e-3) / 1e9 / HBM_PEAK_GBS},
        },
        "input_generation_s": gen_s,
    }

    # exponentials per chain call: one per element of every consulted row and of the row
    # the last token is drawn from
    result["calibration"] = _calibration(torch, dev, api,
                                         exps_chain=(int((acc_c + 1).sum()) + B) * V)
    if args.tree:
        result["modes"].update(_tree_modes(args, torch, dev, api, wl))
    if args.filtered:
        result["modes"].update(_filtered_mode(args, torch, dev, api, wl))

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["calib_copy_bytes"] = n
        del src, dst

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = _cpu_baseline(c, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def _kernel_key(name):
    """Short kernel name as used in CHAIN_KERNELS / GREEDY_KERNELS."""
    if "copyBuffer" in name:
        return "copy"
    base = name.split("::")[1].split("(")[0] if "::" in name else name
    if base.startswith("k_rows<"):
        return "k_rows<sampling>" if base.rstrip(">").endswith("true") else "k_rows<greedy>"
    return base.split("<")[0]


def _read_counter_csv(d, counter):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    rows = []
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    return rows


def _traffic_from(args):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of each kernel of the timed calls, scaled
    by the ratio of known bytes to what the same counter reads for the calibration copy
    (the last three device copies of the run)."""
    out = {"kernel_source_sha": _source_sha(), "unit": "bytes per dispatch"}
    per = {}
    for counter, d in (("FETCH_SIZE", args.traffic_from[0]), ("WRITE_SIZE", args.traffic_from[1])):
        rows = _read_counter_csv(d, counter)
        copies = [v for _, n, v in rows if _kernel_key(n) == "copy"][-3:]
        lines = [ln for ln in open(os.path.join(d, "bench.json")) if ln.startswith("{")]
        meta = json.loads(lines[-1])
        known = meta["calib_copy_bytes"] / 1024.0
        scale = known / (sum(copies) / len(copies))
        out.setdefault("workload", meta["config"]["workload"])
        out[f"{counter}_copy_KiB"] = sum(copies) / len(copies)
        out[f"{counter}_scale"] = scale
        for _, n, v in rows:
            k = _kernel_key(n)
            if k != "copy":
                per.setdefault(k, {}).setdefault(counter, []).append(v)
    kernels = {}
    for k, cv in per.items():
        f = float(np.mean(cv.get("FETCH_SIZE", [0.0]))) * 1024 * out["FETCH_SIZE_scale"]
        w = float(np.mean(cv.get("WRITE_SIZE", [0.0]))) * 1024 * out["WRITE_SIZE_scale"]
        kernels[k] = {"fetch_bytes": f, "write_bytes": w, "dispatches": len(cv.get("FETCH_SIZE", []))}
    out["kernels"] = kernels
    out["calls"] = {
        name: {"bytes": sum(kernels[k]["fetch_bytes"] + kernels[k]["write_bytes"] for k in ks),
               "kernels": ks}
        for name, ks in (("spec_verify_chain", CHAIN_KERNELS), ("spec_verify_greedy", GREEDY_KERNELS),
                         ("spec_verify_chain eager", EAGER_CHAIN_KERNELS),
                         ("spec_verify_greedy eager", EAGER_GREEDY_KERNELS))
        if all(k in kernels for k in ks)}
    os.makedirs(os.path.dirname(args.traffic_json), exist_ok=True)
    json.dump(out, open(args.traffic_json, "w"), indent=1)
    print(json.dumps(out, indent=1))


def _source_sha():
    import hashlib
    p = os.path.join(ROOT, "lossless_rejection_sampling_verify_amd", "csrc", "spec_verify.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def _tree_modes(args, torch, dev, api, wl):
    t = wl.make_tree(4)
    lg = torch.from_numpy(np.ascontiguousarray(t.logits).view(np.int16)).view(torch.bfloat16).to(dev)
    copies = [lg] + [lg.clone() for _ in range(args.copies - 1)]
    tok, par = torch.from_numpy(t.node_tokens).to(dev), torch.from_numpy(t.parents).to(dev)
    cn, tp = torch.from_numpy(t.coins).to(dev), torch.from_numpy(t.temperature).to(dev)
    out = {}
    stream = torch.cuda.current_stream(dev)
    def timed(mode):
        for i in range(5):
            api.spec_verify_tree(copies[i % len(copies)], tok, par, cn, tp, t.D, mode)
        torch.cuda.synchronize()
        ms = []
        for i in range(20):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            acc, _, _, _ = api.spec_verify_tree(copies[i % len(copies)], tok, par, cn, tp, t.D, mode)
            e1.record(stream)
            ms.append((e0, e1, acc))
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b, _ in ms]), ms[-1][2].cpu().numpy()

    for mode, name in ((0, "tree_greedy"), (1, "tree_sampling")):
        d, acc = timed(mode)
        os.environ["SPEC_VERIFY_EAGER"] = "1"
        de, _ = timed(mode)
        del os.environ["SPEC_VERIFY_EAGER"]
        eager = t.B * t.N * t.V * 2
        path = int((acc + 1).sum()) * t.V * 2   # the rows of the nodes the walk reaches
        out[name] = {"workload": t.name, "avg_ms": float(d.mean()),
                     "positions/s": t.B * t.N / (d.mean() * 1e-3),
                     "path_only_bytes": path,
                     "GB/s_path_only": path / (d.mean() * 1e-3) / 1e9,
                     "eager_avg_ms": float(de.mean()), "eager_bytes": eager,
                     "GB/s_eager": eager / (de.mean() * 1e-3) / 1e9,
                     "frac_eager": eager / (de.mean() * 1e-3) / 1e9 / HBM_PEAK_GBS}
    out["tree_mss"] = _tree_mss_mode(torch, dev, api, wl, stream)
    # committing the accepted paths' KV (the step after verify): 128 KiB per token, the KV
    # of 32 layers x 8 KV heads x 128 dims x (K, V) in bf16
    row = 128 * 1024
    acc, _, nodes, _ = api.spec_verify_tree(copies[0], tok, par, cn, tp, t.D, 1)
    kv_tree = torch.empty(t.B, t.N, row, dtype=torch.uint8, device=dev).fill_(3)
    kv_out = torch.empty(t.B, t.D + 1, row, dtype=torch.uint8, device=dev)
    slots = torch.empty(t.B, t.D + 1, dtype=torch.int32, device=dev)
    for _ in range(5):
        api.spec_tree_commit_kv(nodes, acc, kv_tree, kv_out, slots=slots)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(20)]
    for e0, e1 in ev:
        e0.record(stream)
        api.spec_tree_commit_kv(nodes, acc, kv_tree, kv_out, slots=slots)
        e1.record(stream)
    torch.cuda.synchronize()
    d = np.array([a.elapsed_time(b) for a, b in ev])
    moved = int((acc.cpu().numpy() + 1).sum()) * row * 2
    out["tree_commit_kv"] = {"workload": t.name + ", 128 KiB KV per token",
                             "avg_ms": float(d.mean()), "bytes_moved": moved,
                             "GB/s": moved / (d.mean() * 1e-3) / 1e9}
    del kv_tree, kv_out
    # the tree attention mask and positions of the same trees (the step before verify)
    base = torch.arange(t.B, dtype=torch.int32, device=dev)
    W = (t.N + 31) // 32
    outs = (torch.empty(t.B, t.N, W, dtype=torch.int32, device=dev),
            torch.empty(t.B, t.N, dtype=torch.int32, device=dev))
    for _ in range(5):
        api.spec_tree_mask(par, base, out=outs)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(20)]
    for e0, e1 in ev:
        e0.record(stream)
        api.spec_tree_mask(par, base, out=outs)
        e1.record(stream)
    torch.cuda.synchronize()
    d = np.array([a.elapsed_time(b) for a, b in ev])
    nbytes = t.B * t.N * 4 + t.B * 4 + t.B * t.N * W * 4 + t.B * t.N * 4
    out["tree_mask"] = {"workload": t.name, "avg_ms": float(d.mean()),
                        "nodes/s": t.B * t.N / (d.mean() * 1e-3), "bytes": nbytes,
                        "bound": "latency (one workgroup per request)"}
    return out


def _mss_path_bytes(t, acc, nodes, wl):
    """The method's own bytes for a multi-step sampling walk: every row the walk reaches
    once, plus the draft row of every node where a child was rejected."""
    es = 2 if t.dtype == wl.BF16 else 4
    total = 0
    for b in range(t.B):
        k = int(acc[b])
        path = [0] + [int(n) for n in nodes[b, :k]]
        par = t.parents[b]
        total += len(path) * t.V * es
        for i, v in enumerate(path):
            kids = [c for c in range(v + 1, t.N) if par[c] == v]
            rejected = (kids.index(path[i + 1]) > 0) if i + 1 < len(path) else bool(kids)
            if rejected:
                total += t.V * 4
    return total


def _tree_mss_mode(torch, dev, api, wl, stream):
    """spec_verify_tree_mss on the tree workload with a draft row per node.  The walk
    touches only ~100 MB per call, so a 1 GiB buffer is rewritten between timed calls
    (untimed) to keep earlier calls' rows out of the memory-side cache."""
    t = wl.make_tree_mss(4)
    lg = torch.from_numpy(np.ascontiguousarray(t.logits).view(np.int16)).view(torch.bfloat16).to(dev)
    q = torch.from_numpy(t.draft_probs).to(dev)
    tok, par = torch.from_numpy(t.node_tokens).to(dev), torch.from_numpy(t.parents).to(dev)
    cn, tp = torch.from_numpy(t.coins).to(dev), torch.from_numpy(t.temperature).to(dev)
    flush = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    for _ in range(5):
        api.spec_verify_tree_mss(lg, q, tok, par, cn, tp, t.D)
    torch.cuda.synchronize()
    ev = []
    for _ in range(20):
        flush.add_(1.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        acc, _, nodes, _ = api.spec_verify_tree_mss(lg, q, tok, par, cn, tp, t.D)
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    d = np.array([a.elapsed_time(b) for a, b in ev])
    acc, nodes = acc.cpu().numpy(), nodes.cpu().numpy()
    path = _mss_path_bytes(t, acc, nodes, wl)
    del flush, lg, q
    return {"workload": t.name, "avg_ms": float(d.mean()),
            "positions/s": t.B * t.N / (d.mean() * 1e-3),
            "accepted_mean": float(acc.mean()), "path_only_bytes": path,
            "GB/s_path_only": path / (d.mean() * 1e-3) / 1e9}


def _filtered_mode(args, torch, dev, api, wl):
    """spec_verify_chain_filtered on the large-batch shape, draft as bf16 logits, top-k 50
    and top-p 0.9 for every request."""
    c = wl.make_chain_logits(args.workload, top_k=50, top_p=0.9)

    def lg(a):
        a = np.ascontiguousarray(a)
        if c.dtype == wl.BF16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    base = dict(l=lg(c.logits), d=lg(c.draft_logits), x=torch.from_numpy(c.draft_tokens).to(dev),
                u=torch.from_numpy(c.coins).to(dev), T=torch.from_numpy(c.temperature).to(dev),
                k=torch.from_numpy(c.top_k).to(dev), p=torch.from_numpy(c.top_p).to(dev))
    copies = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(args.copies - 1)]
    stream = torch.cuda.current_stream(dev)
    for i in range(5):
        d = copies[i % len(copies)]
        api.spec_verify_chain_filtered(d["l"], d["d"], d["x"], d["u"], d["T"], d["k"], d["p"])
    torch.cuda.synchronize()
    ev = []
    for i in range(20):
        d = copies[i % len(copies)]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        acc, _, _ = api.spec_verify_chain_filtered(d["l"], d["d"], d["x"], d["u"], d["T"], d["k"], d["p"])
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    es = 2 if c.dtype == wl.BF16 else 4
    once = (c.B * c.R + c.B * c.G) * c.V * es
    return {"chain_filtered": {"workload": c.name + ", top-k 50, top-p 0.9",
                               "avg_ms": float(t.mean()),
                               "positions/s": c.B * c.R / (t.mean() * 1e-3),
                               "row_bytes_once": once,
                               "GB/s_rows_once": once / (t.mean() * 1e-3) / 1e9,
                               "accepted_mean": float(acc.float().mean().item())}}


def _calibration(torch, dev, api, exps_chain):
    """This device's own ceilings, measured after the timed region: the read bandwidth
    of the row passes' access pattern (16-byte non-temporal loads over 2 GiB) and the
    v_exp_f32 throughput, with the time the chain call's exponentials alone would take."""
    stream = torch.cuda.current_stream(dev)
    sink = torch.zeros(1, dtype=torch.float32, device=dev)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            ms.append(e0.elapsed_time(e1))
        return float(np.median(ms))

    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    read_ms = timed(lambda: api.spec_calib_read(buf, sink), 7)
    del buf
    blocks, iters = 4096, 1024
    exp_ms = timed(lambda: api.spec_calib_exp(blocks, iters, sink), 5)
    exp_rate = blocks * 256 * iters * 8 / (exp_ms * 1e-3)
    read_gbs = nbytes / (read_ms * 1e-3) / 1e9
    return {"read_GB/s": read_gbs, "read_frac_of_peak": read_gbs / HBM_PEAK_GBS,
            "read_bytes": nbytes, "exp_per_s": exp_rate,
            "chain_exps_per_call": exps_chain,
            "chain_exp_floor_ms": exps_chain / exp_rate * 1e3}


def _cpu_baseline(c, seconds):
    """The fp64 oracle on a bounded sample (the first 64 requests), greedy + chain, repeated
    for about `seconds` seconds on the host's cores."""
    import oracle
    nb = min(64, c.B)
    lg = np.ascontiguousarray(c.logits[:nb])
    q = np.ascontiguousarray(c.draft_probs[:nb])
    x, xg = np.ascontiguousarray(c.draft_tokens[:nb]), np.ascontiguousarray(c.greedy_tokens[:nb])
    u, T = np.ascontiguousarray(c.coins[:nb]), np.ascontiguousarray(c.temperature[:nb])
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.verify_greedy(lg, c.dtype, xg)
        oracle.verify_chain(lg, c.dtype, q, x, u, T)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    pos = reps * 2 * nb * c.R
    return {"value": pos / el, "unit": "positions/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"first {nb} of {c.B} requests of '{c.name}', greedy + chain verify, "
                      f"{reps} repetitions in {el:.1f} s (fp64 C oracle, OpenMP over requests)"}


if __name__ == "__main__":
    main()
