#!/usr/bin/env python3
"""Benchmark of the batched speculative-decoding verify step on one MI355X.

One step = one pass of the whole chain/greedy verify path over the large-batch workload
(B=256 requests, gamma=4, V=152064, bf16 target logits ~ N(0, 3^2), draft = target +
N(0,1), T=1): spec_verify_greedy and spec_verify_chain.  Inputs are synthetic, seeded,
and resident in HBM before timing starts.  Four copies of them rotate, and the greedy and
chain calls of a step read different copies, so no call finds the rows the previous call
read in the 256 MB memory-side cache.

Prints ONE JSON line: verified positions/s (whole step: both calls' B * (gamma+1)
positions), the roofline of the dominant call (spec_verify_chain: algorithmic HBM bytes
per call / call time measured with HIP events on the launch stream), and the CPU oracle
timed on a bounded sample of the same workload (1 thread and all host threads), with a
parity check of the timed outputs against it.

Both calls walk each request position by position and stop at the first rejection (or
mismatch), so the algorithmic bytes of a call are the rows the method consults: for
request b, rows 0..k_b of its logits, plus the fp32 draft row at k_b when the chain
rejected there.  The eager passes (every row streamed), selected with the launch option
path = eager, are timed after the main region and reported under modes.*_eager with
their own bytes (every row once).  modes.workloads times the tiny, small and boosted
chain workloads; modes.alpha_sweep times the large batch at draft acceptance rates of
about 0.4, 0.65 and 0.9 and with q = p (every row read).

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
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=5, choices=[2, 3, 5])
    ap.add_argument("--copies", type=int, default=4,
                    help="input copies in rotation; the greedy and chain calls of a step use "
                         "different copies (at least 4 keeps every call's rows out of the "
                         "256 MB memory-side cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip timing the tiny, small and boosted chain workloads")
    ap.add_argument("--no-alpha-sweep", action="store_true",
                    help="skip the sweep over draft acceptance rates")
    ap.add_argument("--tree", action="store_true", help="also time the tree workload")
    ap.add_argument("--filtered", action="store_true",
                    help="also time chain verify from draft logits with top-k 50 / top-p 0.9")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"))
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, copy a buffer of this many MiB 3 times (counter scale)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="reduce two rocprofv3 --pmc runs (csv) into --traffic-json and exit")
    return ap.parse_args()


def _say(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class _Dev:
    """Device copies of one chain workload's inputs."""

    def __init__(self, torch, dev, c, copies):
        def lg(a):
            a = np.ascontiguousarray(a)
            if c.dtype == "bf16":
                return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(a).to(dev)
        base = dict(logits=lg(c.logits), q=torch.from_numpy(c.draft_probs).to(dev),
                    x=torch.from_numpy(c.draft_tokens).to(dev),
                    xg=torch.from_numpy(c.greedy_tokens).to(dev),
                    u=torch.from_numpy(c.coins).to(dev), T=torch.from_numpy(c.temperature).to(dev))
        self.copies = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(copies - 1)]


def _path_bytes(c, acc_g, acc_c, esize):
    """The method's own bytes of the greedy and chain calls: for request b, rows 0..k_b of its
    logits, plus (chain) the fp32 draft row at k_b where it rejected, plus tokens, coins,
    temperatures, gathers and outputs."""
    B, G, V, R = c.B, c.G, c.V, c.G + 1
    small_g = B * G * 4 + B * 4 + B * R * 4
    small_c = B * (G + R + 1) * 4 + B * G * 4 + B * 4 + 2 * B * R * 4
    rejected = int((acc_c < G).sum())
    greedy = int((acc_g + 1).sum()) * V * esize + small_g
    chain = int((acc_c + 1).sum()) * V * esize + rejected * V * 4 + small_c
    eager_g = B * R * V * esize + small_g
    eager_c = B * R * V * esize + rejected * V * 4 + small_c
    return greedy, chain, eager_g, eager_c, rejected


def _timed_pair(torch, api, d, stream, reps, opts=None, warm=3):
    """Event-timed greedy and chain calls, each call on its own input copy (the greedy call
    of round i on copy 2i, the chain call on copy 2i + 1, modulo the copies)."""
    n = len(d.copies)
    outs = {}

    def one(i, ev=None):
        dg, dc = d.copies[(2 * i) % n], d.copies[(2 * i + 1) % n]
        if ev is not None:
            ev[0].record(stream)
        outs["g"] = api.spec_verify_greedy(dg["logits"], dg["xg"], opts=opts)
        if ev is not None:
            ev[1].record(stream)
        outs["c"] = api.spec_verify_chain(dc["logits"], dc["q"], dc["x"], dc["u"], dc["T"],
                                          opts=opts)
        if ev is not None:
            ev[2].record(stream)
    for i in range(warm):
        one(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for i in range(reps):
        one(i, evs[i])
    torch.cuda.synchronize()
    g_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    c_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    return g_ms, c_ms, outs["g"][0].cpu().numpy(), outs["c"][0].cpu().numpy()


def _stats(ms):
    return {"avg_us": float(ms.mean() * 1e3), "median_us": float(np.median(ms) * 1e3),
            "p90_us": float(np.percentile(ms, 90) * 1e3)}


def main():
    args = parse()
    if args.traffic_from:
        _traffic_from(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the verify path is single-GPU here)", file=sys.stderr)
        sys.exit(2)
    if args.copies < 2:
        print("--copies must be at least 2 (the greedy and chain calls of a step read "
              "different copies)", file=sys.stderr)
        sys.exit(2)

    import torch

    import lossless_rejection_sampling_verify_amd as pkg  # noqa: F401
    from lossless_rejection_sampling_verify_amd import _lib as L
    from lossless_rejection_sampling_verify_amd import api
    from lossless_rejection_sampling_verify_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    c = wl.make_chain(args.workload)
    gen_s = time.time() - t0
    _say(f"generated {c.name} in {gen_s:.1f} s")
    B, G, V, R = c.B, c.G, c.V, c.R
    esize = 2 if c.dtype == wl.BF16 else 4

    d = _Dev(torch, dev, c, args.copies)
    copies = d.copies
    ws_g = api.workspace(L.SPEC_OP_GREEDY, B, R, V, dev)
    ws_c = api.workspace(L.SPEC_OP_CHAIN, B, R, V, dev)
    out_g = (torch.empty(B, dtype=torch.int32, device=dev), torch.empty(B, R, dtype=torch.int32, device=dev))
    out_c = (torch.empty(B, dtype=torch.int32, device=dev), torch.empty(B, R, dtype=torch.int32, device=dev),
             torch.empty(B, R, dtype=torch.float32, device=dev))
    stream = torch.cuda.current_stream(dev)
    n = len(copies)

    # Each HIP event recorded between two kernels costs about 5.5 us of GPU time here (the
    # step took 130.9 / 125.5 / 119.7 us with 3 / 2 / 0 events per step), so the timed region
    # times the chain call on every `every`-th step and the greedy call on the steps halfway
    # between, rather than every call of every step.
    every = 4 if args.steps >= 8 else 1

    def step(i, ev=None):
        # the greedy call reads copy 2i, the chain call copy 2i + 1: no call finds the rows
        # the call before it read in the memory-side cache
        dg, dc = copies[(2 * i) % n], copies[(2 * i + 1) % n]
        tg = ev is not None and i % every == every // 2
        tc = ev is not None and i % every == 0
        if tg:
            ev[0].record(stream)
        api.spec_verify_greedy(dg["logits"], dg["xg"], ws=ws_g, out=out_g)
        if tg:
            ev[1].record(stream)
        if tc:
            ev[2].record(stream)
        api.spec_verify_chain(dc["logits"], dc["q"], dc["x"], dc["u"], dc["T"], ws=ws_c, out=out_c)
        if tc:
            ev[3].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, synchronised on both sides
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    _say(f"timed {args.steps} steps in {elapsed * 1e3:.2f} ms")

    greedy_ms = np.array([e[0].elapsed_time(e[1]) for i, e in enumerate(events)
                          if i % every == every // 2])
    chain_ms = np.array([e[2].elapsed_time(e[3]) for i, e in enumerate(events) if i % every == 0])
    # the last step's outputs (every copy holds the same inputs), for the parity check
    acc_g, toks_g = out_g[0].cpu().numpy(), out_g[1].cpu().numpy()
    acc_c, toks_c = out_c[0].cpu().numpy(), out_c[1].cpu().numpy()
    probs_c = out_c[2].cpu().numpy()

    greedy_bytes, chain_bytes, eager_g_bytes, eager_c_bytes, rejected = _path_bytes(c, acc_g, acc_c, esize)
    positions = 2 * B * R
    value = positions * args.steps / elapsed

    chain_gbs = chain_bytes / (chain_ms.mean() * 1e-3) / 1e9
    greedy_gbs = greedy_bytes / (greedy_ms.mean() * 1e-3) / 1e9

    # the eager passes, for comparison (outside the timed region), same copy rotation
    ge, ce, _, _ = _timed_pair(torch, api, d, stream, 20, opts={"path": "eager"})

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
                   "step": "spec_verify_greedy + spec_verify_chain, each on its own input copy",
                   "input_copies": args.copies},
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
            "launches_timed": int(len(chain_ms)),
            "timed_every_steps": every,
        },
        "modes": {
            "greedy": {"avg_ms": float(greedy_ms.mean()), "median_ms": float(np.median(greedy_ms)), "p90_ms": float(np.percentile(greedy_ms, 90)),
                       "GB/s": greedy_gbs, "frac": greedy_gbs / HBM_PEAK_GBS,
                       "bytes": greedy_bytes,
                       "positions/s": B * R / (greedy_ms.mean() * 1e-3),
                       "rows_consulted": int((acc_g + 1).sum()),
                       "tokens/s": float((acc_g + 1).sum()) / (greedy_ms.mean() * 1e-3)},
            "chain": {"avg_ms": float(chain_ms.mean()), "median_ms": float(np.median(chain_ms)), "p90_ms": float(np.percentile(chain_ms, 90)),
                      "GB/s": chain_gbs, "frac": chain_gbs / HBM_PEAK_GBS,
                      "bytes": chain_bytes,
                      "positions/s": B * R / (chain_ms.mean() * 1e-3),
                      "rejected_requests": rejected,
                      "rows_consulted": int((acc_c + 1).sum()),
                      "tokens/s": float((acc_c + 1).sum()) / (chain_ms.mean() * 1e-3)},
            "greedy_eager": {"avg_ms": float(ge.mean()), "median_ms": float(np.median(ge)), "bytes": eager_g_bytes,
                             "GB/s": eager_g_bytes / (ge.mean() * 1e-3) / 1e9,
                             "frac": eager_g_bytes / (ge.mean() * 1e-3) / 1e9 / HBM_PEAK_GBS},
            "chain_eager": {"avg_ms": float(ce.mean()), "median_ms": float(np.median(ce)), "bytes": eager_c_bytes,
                            "GB/s": eager_c_bytes / (ce.mean() * 1e-3) / 1e9,
                            "frac": eager_c_bytes / (ce.mean() * 1e-3) / 1e9 / HBM_PEAK_GBS},
        },
        "input_generation_s": gen_s,
    }
    _say("main workload done")

    # exponentials per chain call: one per element of every consulted row and of the row
    # the last token is drawn from
    result["calibration"] = _calibration(torch, dev, api,
                                         exps_chain=(int((acc_c + 1).sum()) + B) * V)
    del d, copies
    sweep_inputs = {}
    if not args.no_workloads:
        result["modes"]["workloads"] = _workload_modes(torch, dev, api, wl, stream)
        _say("workloads done")
    if not args.no_alpha_sweep and args.workload == 5:
        result["modes"]["alpha_sweep"] = _alpha_sweep(torch, dev, api, wl, stream, c, sweep_inputs)
        _say("alpha sweep done")
    if args.tree:
        result["modes"].update(_tree_modes(args, torch, dev, api, wl))
    if args.filtered:
        result["modes"].update(_filtered_mode(args, torch, dev, api, wl))

    if args.calib_copy_mib > 0:
        nb = args.calib_copy_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["calib_copy_bytes"] = nb
        del src, dst

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = _cpu_baseline(
            c, args.cpu_seconds, dict(accept_len=acc_g, out_tokens=toks_g),
            dict(accept_len=acc_c, out_tokens=toks_c, probs=probs_c), sweep_inputs)
        _say("cpu baseline done")
    print(json.dumps(result), flush=True)


# the draft noise variances of the sweep, with the acceptance rate each gives on the
# large-batch target rows (target logits ~ N(0, 9), T = 1), and q = p
ALPHA_SWEEP = (("alpha~0.40", 2.6), ("alpha~0.65", 0.8), ("alpha~0.90", 0.05), ("q=p", 0.0))


def _alpha_sweep(torch, dev, api, wl, stream, c0, keep):
    """The large-batch call at other draft acceptance rates: the same target rows, drafts
    d = target + N(0, var) (q = softmax(d), x ~ q; greedy drafts argmax d), var from
    ALPHA_SWEEP; var = 0 gives q = p, so every draft is accepted and every row is read.
    For each point: walk and eager times of both calls, rows consulted, path-only and
    all-row bandwidth, and the acceptance rate seen in the GPU's outputs (accepted tests
    over tested positions).  The oracle's exact alpha (mean beta) on a sample of each
    point is in the CPU-baseline block."""
    out = {}
    esize = 2 if c0.dtype == wl.BF16 else 4
    for name, var in ALPHA_SWEEP:
        t0 = time.time()
        c = wl.make_chain(5, draft_var=var)
        assert np.array_equal(c.logits[:2], c0.logits[:2]), "the sweep keeps the target rows"
        d = _Dev(torch, dev, c, 4)
        g_ms, c_ms, acc_g, acc_c = _timed_pair(torch, api, d, stream, 20)
        ge, ce, _, _ = _timed_pair(torch, api, d, stream, 10, opts={"path": "eager"})
        gb, cb, egb, ecb, rej = _path_bytes(c, acc_g, acc_c, esize)
        tested = np.minimum(acc_c + 1, c.G).sum()
        out[name] = {
            "draft_noise_var": var,
            "alpha_observed_chain": float(acc_c.sum() / tested),
            "mean_accept_len": {"chain": float(acc_c.mean()), "greedy": float(acc_g.mean())},
            "rows_consulted": {"chain": int((acc_c + 1).sum()), "greedy": int((acc_g + 1).sum()),
                               "of": c.B * c.R},
            "chain": {"walk_us": float(c_ms.mean() * 1e3), "eager_us": float(ce.mean() * 1e3),
                      "path_bytes": cb, "frac_path": cb / (c_ms.mean() * 1e-3) / 1e9 / HBM_PEAK_GBS,
                      "eager_bytes": ecb,
                      "frac_eager": ecb / (ce.mean() * 1e-3) / 1e9 / HBM_PEAK_GBS,
                      "positions/s_walk": c.B * c.R / (c_ms.mean() * 1e-3)},
            "greedy": {"walk_us": float(g_ms.mean() * 1e3), "eager_us": float(ge.mean() * 1e3),
                       "path_bytes": gb, "frac_path": gb / (g_ms.mean() * 1e-3) / 1e9 / HBM_PEAK_GBS,
                       "eager_bytes": egb,
                       "frac_eager": egb / (ge.mean() * 1e-3) / 1e9 / HBM_PEAK_GBS,
                       "positions/s_walk": c.B * c.R / (g_ms.mean() * 1e-3)},
        }
        keep[name] = dict(logits=c.logits[:16].copy(), q=c.draft_probs[:16].copy(),
                          x=c.draft_tokens[:16].copy(), u=c.coins[:16].copy(),
                          T=c.temperature[:16].copy(), dtype=c.dtype)
        del d, c
        torch.cuda.empty_cache()
        _say(f"alpha sweep {name}: {time.time() - t0:.1f} s")
    return out


def _workload_modes(torch, dev, api, wl, stream):
    """The tiny chain, the small chain and the boosted chain workloads, greedy and chain
    calls (walks): latency, and for the boosted workload the path-only bandwidth."""
    out = {}
    for cfg, reps in ((1, 200), (2, 200), (3, 50)):
        c = wl.make_chain(cfg)
        d = _Dev(torch, dev, c, 4 if cfg == 3 else 2)
        g_ms, c_ms, acc_g, acc_c = _timed_pair(torch, api, d, stream, reps, warm=10)
        esize = 2 if c.dtype == wl.BF16 else 4
        gb, cb, egb, ecb, rej = _path_bytes(c, acc_g, acc_c, esize)
        # medians: these calls are a few microseconds, and a stray slow launch skews a mean
        gm, cm = float(np.median(g_ms)), float(np.median(c_ms))
        out[c.name] = {
            "greedy": dict(_stats(g_ms), path_bytes=gb,
                           frac_path=gb / (gm * 1e-3) / 1e9 / HBM_PEAK_GBS,
                           positions_per_s=c.B * c.R / (gm * 1e-3),
                           tokens_per_s=int((acc_g + 1).sum()) / (gm * 1e-3),
                           rows_consulted=int((acc_g + 1).sum()), of=c.B * c.R),
            "chain": dict(_stats(c_ms), path_bytes=cb,
                          frac_path=cb / (cm * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          positions_per_s=c.B * c.R / (cm * 1e-3),
                          tokens_per_s=int((acc_c + 1).sum()) / (cm * 1e-3),
                          rows_consulted=int((acc_c + 1).sum()), of=c.B * c.R),
            "bound": "latency (a few rows per request)" if cfg < 3 else "hbm + latency tail",
        }
        del d
    return out


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
    def timed(mode, opts=None):
        for i in range(5):
            api.spec_verify_tree(copies[i % len(copies)], tok, par, cn, tp, t.D, mode, opts=opts)
        torch.cuda.synchronize()
        ms = []
        for i in range(20):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            acc, _, _, _ = api.spec_verify_tree(copies[i % len(copies)], tok, par, cn, tp, t.D, mode,
                                                opts=opts)
            e1.record(stream)
            ms.append((e0, e1, acc))
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b, _ in ms]), ms[-1][2].cpu().numpy()

    for mode, name in ((0, "tree_greedy"), (1, "tree_sampling")):
        d, acc = timed(mode)
        de, _ = timed(mode, {"path": "eager"})
        eager = t.B * t.N * t.V * 2
        path = int((acc + 1).sum()) * t.V * 2   # the rows of the nodes the walk reaches
        # medians: under a profiler the first calls of each kernel run much longer
        md, mde = float(np.median(d)), float(np.median(de))
        out[name] = {"workload": t.name, "avg_ms": float(d.mean()), "median_ms": md,
                     "positions/s": t.B * t.N / (md * 1e-3),
                     "path_only_bytes": path,
                     "GB/s_path_only": path / (md * 1e-3) / 1e9,
                     "frac_path_only": path / (md * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "levels_walked_max": int(acc.max()) + 1,
                     "us_per_level_longest": md * 1e3 / (int(acc.max()) + 1),
                     "eager_median_ms": mde, "eager_bytes": eager,
                     "GB/s_eager": eager / (mde * 1e-3) / 1e9,
                     "frac_eager": eager / (mde * 1e-3) / 1e9 / HBM_PEAK_GBS}
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
    md = float(np.median(d))
    return {"workload": t.name, "avg_ms": float(d.mean()), "median_ms": md,
            "positions/s": t.B * t.N / (md * 1e-3),
            "accepted_mean": float(acc.mean()), "path_only_bytes": path,
            "GB/s_path_only": path / (md * 1e-3) / 1e9,
            "frac_path_only": path / (md * 1e-3) / 1e9 / HBM_PEAK_GBS}


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
    md = float(np.median(t))
    return {"chain_filtered": {"workload": c.name + ", top-k 50, top-p 0.9",
                               "avg_ms": float(t.mean()), "median_ms": md,
                               "positions/s": c.B * c.R / (md * 1e-3),
                               "row_bytes_once": once,
                               "GB/s_rows_once": once / (md * 1e-3) / 1e9,
                               "frac_rows_once": once / (md * 1e-3) / 1e9 / HBM_PEAK_GBS,
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


def _cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_baseline(c, seconds, gpu_greedy, gpu_chain, sweep):
    """The fp64 oracle as it stands, on a bounded sample of the same workload (its first 64
    requests), greedy + chain, timed at 1 thread and at every host thread: three blocks
    of about seconds/6 each per thread count, the median block rate reported.  The same
    oracle results are compared with the GPU's outputs of the last timed step for those
    requests (parity block), and the oracle's acceptance-rate diagnostic gives the exact
    alpha (mean beta) of the sample, and of a 16-request sample of each alpha-sweep point."""
    import oracle
    nb = min(64, c.B)
    lg = np.ascontiguousarray(c.logits[:nb])
    q = np.ascontiguousarray(c.draft_probs[:nb])
    x, xg = np.ascontiguousarray(c.draft_tokens[:nb]), np.ascontiguousarray(c.greedy_tokens[:nb])
    u, T = np.ascontiguousarray(c.coins[:nb]), np.ascontiguousarray(c.temperature[:nb])
    all_threads = oracle.num_threads()

    def rate(threads):
        oracle.set_num_threads(threads)
        blocks = []
        for _ in range(3):
            reps, t0 = 0, time.perf_counter()
            while True:
                oracle.verify_greedy(lg, c.dtype, xg)
                oracle.verify_chain(lg, c.dtype, q, x, u, T)
                reps += 1
                el = time.perf_counter() - t0
                if el >= seconds / 6:
                    break
            blocks.append(reps * 2 * nb * c.R / el)
        return float(np.median(blocks)), blocks

    one, one_blocks = rate(1)
    full, full_blocks = rate(all_threads)
    oracle.set_num_threads(all_threads)
    # parity of the timed outputs on the sample, and the exact alpha
    oa, oo = oracle.verify_greedy(lg, c.dtype, xg)
    o = oracle.verify_chain(lg, c.dtype, q, x, u, T, beta=True)
    mism = (gpu_chain["accept_len"][:nb] != o["accept_len"]) | \
        (gpu_chain["out_tokens"][:nb] != o["out_tokens"]).any(1)
    near = o["margin"] <= 1e-6
    ok = ~mism
    rel = np.abs(gpu_chain["probs"][:nb][ok].astype(np.float64) - o["probs"][ok]) / \
        np.maximum(np.abs(o["probs"][ok]), 1e-30)
    parity = {
        "requests": nb,
        "greedy_mismatch": int(((gpu_greedy["accept_len"][:nb] != oa) |
                                (gpu_greedy["out_tokens"][:nb] != oo).any(1)).sum()),
        "chain": {"near": int(near.sum()), "near_accept": int((o["accept_margin"] <= 1e-6).sum()),
                  "near_mismatch": int((mism & near).sum()),
                  "mismatch_outside_band": int((mism & ~near).sum()),
                  "max_prob_rel_err": float(rel.max()) if rel.size else 0.0},
    }
    alpha = {"large-batch sample": float(o["beta"].mean())}
    for name, inp in sweep.items():
        r = oracle.verify_chain(inp["logits"], inp["dtype"], inp["q"], inp["x"], inp["u"],
                                inp["T"], beta=True)
        alpha[name] = float(r["beta"].mean())
    return {"value": full, "unit": "positions/s", "cores": all_threads, "kind": "oracle",
            "value_1_thread": one, "blocks": {"1": one_blocks, str(all_threads): full_blocks},
            "cpu_model": _cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"first {nb} of {c.B} requests of '{c.name}', greedy + chain verify, "
                      f"fp64 C oracle (OpenMP over requests); median of 3 blocks of "
                      f"~{seconds / 6:.1f} s at 1 and at {all_threads} threads",
            "parity_of_timed_outputs": parity, "alpha_exact": alpha}


if __name__ == "__main__":
    main()
