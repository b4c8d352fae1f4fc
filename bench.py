#!/usr/bin/env python3
"""Throughput of the verify + commit step on one MI355X.

One step = one decode step of one GDN layer at batch 1 (16 q/k heads, 48
value heads, d_k = d_v = 128, bf16 q/k/v, fp32 state, f16 persisted node
states, fp32 outputs and final state): gdn_commit_verify_chain commits the
previous step's accepted node into the state cache and verifies the next
16-node draft, in one launch.  The metric is verified draft tokens per second
per GDN layer: 16 nodes per step per layer.

Timing.  Inputs are resident in device memory before the timed region, and
steps rotate over enough independent buffer sets (> 256 MB in total) that the
256 MB Infinity Cache cannot hold one step's data from its previous visit.
Every call is marshalled once (binding ``prepare=True``), so a step costs the
host one C call.  After the warm-up an untimed settling phase of fixed
duration runs the same steps; each timed region then starts behind a short
device-side spacer (a memory-bound fill) so that the host has enqueued the
region's launches before the device reaches them, and the device-side events
measure the launches back to back, not the host.  Reported: the mean over
the K steps of one region (the value), the median of per-step event pairs
over a second region, and, as a launch-overhead measurement only, the same
steps replayed from a captured HIP graph.

Printed: one JSON line with the metric, the roofline of the step kernel
(algorithmic bytes per launch / average launch time from HIP events over the
timed region), the oracle timed on this host's cores (all of them and one),
and secondary measurements (tree, batched, replay, index-table commit,
prefill).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK = 2.5e15
PROFILES = os.path.join(ROOT, "profiles")
VERIFY_SOURCES = ["gated_deltanet_recurrence_gdn_amd/csrc/verify.hip",
                  "gated_deltanet_recurrence_gdn_amd/csrc/verify_body.h",
                  "gated_deltanet_recurrence_gdn_amd/csrc/gdn_device.h",
                  "gated_deltanet_recurrence_gdn_amd/csrc/gdn_internal.h"]
METRIC = "verified draft tokens/s per GDN layer (48 v-heads, d=128) + % HBM roofline"
SETTLE_S = 0.25  # untimed settling phase before the timed regions


def source_sha(paths) -> str:
    import hashlib

    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key: str, sha: str):
    """HBM bytes per launch of a kernel from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a copy kernel of known size), or None
    when there is none for the current kernel source."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel_key)
    if not rec or rec.get("source_sha") != sha:
        return None
    return rec.get("bytes_per_launch")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------
class Timer:
    """Device-side timing of a list of prepared steps (called round robin) on
    torch's current stream, the stream every prepared call launches on."""

    def __init__(self, torch, dev):
        self.torch = torch
        # spacer: in-place passes over 256 MiB (~0.1 ms of device time each), one per 10 steps to be
        # enqueued (a prepared step costs the host well under 10 us)
        self.spacer_buf = torch.ones(64 << 20, device=dev)

    def spacer(self, steps: int):
        for _ in range(2 + steps // 10):
            self.spacer_buf.mul_(1.0)

    def settle(self, calls, seconds: float):
        t_end = time.perf_counter() + seconds
        i = 0
        while time.perf_counter() < t_end:
            calls[i % len(calls)]()
            i += 1
        self.torch.cuda.synchronize()
        return i

    def region(self, calls, steps: int) -> float:
        """Mean device time per step (ms) of `steps` steps launched back to back."""
        torch = self.torch
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        self.spacer(steps)
        calls[-1]()  # one untimed step between the spacer and the timed ones
        t0.record()
        for i in range(steps):
            calls[i % len(calls)]()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    def per_step(self, calls, steps: int) -> list:
        """Device time of each step (ms) from an event pair around it."""
        torch = self.torch
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        self.spacer(steps)
        ev[0].record()
        for i in range(steps):
            calls[i % len(calls)]()
            ev[i + 1].record()
        torch.cuda.synchronize()
        return [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]

    def graph(self, make_calls, steps: int, replays: int = 5):
        """Mean time per step (ms) of `steps` steps captured in one HIP graph and
        replayed; make_calls(stream) prepares the steps on the capture stream."""
        torch = self.torch
        s = torch.cuda.Stream()
        calls = make_calls(s)
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                calls[i % len(calls)]()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(replays):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / (replays * steps)


def measure(timer, calls, steps, warmup, settle=0.0):
    for i in range(warmup):
        calls[i % len(calls)]()
    timer.torch.cuda.synchronize()
    if settle > 0:
        timer.settle(calls, settle)
    mean = timer.region(calls, steps)
    per = timer.per_step(calls, steps)
    return mean, statistics.median(per), per


# ---------------------------------------------------------------------------
# inputs
# ---------------------------------------------------------------------------
def dev_set(torch, d, dev):
    t = {n: torch.from_numpy(np.ascontiguousarray(d[n + "_bits"]).view(np.int16)).to(dev).view(torch.bfloat16)
         for n in ("q", "k", "v")}
    for n in ("alpha", "beta", "state0"):
        t[n] = torch.from_numpy(np.ascontiguousarray(d[n])).to(dev)
    t["accepted"] = torch.from_numpy(d["accepted"]).to(dev)
    return t


def make_sets(torch, wl, w, nsets, dev, tree=False):
    sets = []
    for i in range(nsets):
        d = wl.make_inputs(w, seed=wl.WORKLOAD_SEEDS[w.name] + 7919 * i)
        t = dev_set(torch, d, dev)
        B, N = w.batch, w.n_nodes
        t["out"] = torch.empty(B, N, w.h_v, w.d_v, device=dev)
        t["persist"] = torch.empty(B, N, w.h_v, w.d_v, w.d_k, device=dev, dtype=torch.float16)
        t["final"] = None if tree else torch.empty(B, w.h_v, w.d_v, w.d_k, device=dev)
        t["parent"] = d["parent"]
        sets.append(t)
    return sets


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--sets", type=int, default=12, help="rotating buffer sets (chain and tree)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU work of the oracle baseline (all cores)")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--skip-secondary", action="store_true")
    ap.add_argument("--only-prefill", action="store_true",
                    help="run only the chunked prefill leg and print its measurement (for counter profiles)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB (reads and writes MIB MiB), to scale "
                         "memory counters in a profile")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} (WORLD_SIZE={world}) is not supported: the path "
              "has no cross-GPU step (each (sequence, head) recurrence is independent).", file=sys.stderr)
        return 2

    import torch

    from gated_deltanet_recurrence_gdn_amd import binding as gb
    from gated_deltanet_recurrence_gdn_amd import workloads as wl

    gb.lib()
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)  # one elementwise kernel: n*4 bytes read, n*4 written
        torch.cuda.synchronize()
        del src, dst
    timer = Timer(torch, dev)
    if args.only_prefill:
        print(json.dumps({"prefill": bench_prefill(torch, gb, wl, dev, timer, max(10, args.steps // 5))}),
              flush=True)
        return 0
    w = wl.WORKLOADS["chain"]
    ledger = wl.algorithmic_bytes_verify(w)
    sets = make_sets(torch, wl, w, args.sets, dev)
    set_bytes = ledger["total"]
    log(f"chain: {args.sets} buffer sets, {set_bytes * args.sets / 1e6:.0f} MB rotated")

    def verify_call(s, stream=None):
        return gb.gdn_verify_chain(s["q"], s["k"], s["v"], s["alpha"], s["beta"], s["state0"], out=s["out"],
                                   persist=s["persist"], final_state=s["final"], stream=stream, prepare=True)

    def commit_call(s, stream=None):
        return gb.gdn_commit(s["accepted"], s["persist"], s["state0"], final_state=s["final"], stream=stream,
                             prepare=True)

    def fused_call(s, stream=None):  # commit this set's previous accepted node, then verify
        return gb.gdn_commit_verify_chain(s["accepted"], s["persist"], s["q"], s["k"], s["v"], s["alpha"],
                                          s["beta"], s["state0"], final_prev=s["final"], out=s["out"],
                                          persist=s["persist"], final_state=s["final"], stream=stream,
                                          prepare=True)

    for s in sets:  # every set has a verified block to commit before the first fused step
        verify_call(s)()
    fused = [fused_call(s) for s in sets]
    verify = [verify_call(s) for s in sets]
    commit = [commit_call(s) for s in sets]

    def two_launch(i):
        def step():
            verify[i]()
            commit[i]()
        return step

    step2 = [two_launch(i) for i in range(len(sets))]
    step_ms, med_ms, per = measure(timer, fused, args.steps, args.warmup, settle=SETTLE_S)
    graph_ms = timer.graph(lambda st: [fused_call(s, st) for s in sets], min(args.steps, 240))
    step2_ms, step2_med, _ = measure(timer, step2, args.steps, args.warmup)
    verify_ms, verify_med, _ = measure(timer, verify, args.steps, args.warmup)
    tokens_per_step = w.batch * w.n_nodes
    value = tokens_per_step / (step_ms * 1e-3)
    achieved = ledger["fused_total"] / (step_ms * 1e-3) / 1e9
    log(f"chain fused step {step_ms * 1e3:.2f} us mean, {med_ms * 1e3:.2f} us median of per-step events, "
        f"{graph_ms * 1e3:.2f} us graph-replayed ({achieved:.0f} GB/s); two-launch step {step2_ms * 1e3:.2f} us, "
        f"verify kernel {verify_ms * 1e3:.2f} us")

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "chain verify + commit: batch 1, 16 q/k heads, 48 value heads, d_k=d_v=128, "
                        "16-node draft, bf16 q/k/v, fp32 state, f16 persisted node states, fp32 outputs; "
                        "one launch per step (gdn_commit_verify_chain commits the previous step's accepted "
                        "node and verifies the next block)",
            "batch": w.batch, "nodes": w.n_nodes, "h_qk": w.h_qk, "h_v": w.h_v, "d_k": w.d_k, "d_v": w.d_v,
            "buffer_sets": args.sets, "rotated_bytes": set_bytes * args.sets,
            "step_bytes": ledger["fused_total"],
            "timing": {"step_us_mean": step_ms * 1e3, "step_us_median": med_ms * 1e3,
                       "step_us_min": min(per) * 1e3, "step_us_max": max(per) * 1e3,
                       "graph_replayed_step_us": graph_ms * 1e3,
                       "settle_s": SETTLE_S,
                       "how": "mean: one region of K back-to-back steps behind a device-side spacer "
                              "(the value); median: per-step event pairs over a second region; "
                              "graph: the same steps captured in one HIP graph and replayed "
                              "(launch-overhead measurement only)"},
            "two_launch_step": {"ms_per_step": step2_ms, "median_ms": step2_med,
                                "tokens_per_s_per_layer": tokens_per_step / (step2_ms * 1e-3),
                                "step_bytes": set_bytes, "verify_kernel_us": verify_ms * 1e3,
                                "verify_kernel_us_median": verify_med * 1e3,
                                "verify_gbs": ledger["verify_total"] / (verify_ms * 1e-3) / 1e9},
        },
        "roofline": {
            "kernel": "commit_verify_chain_kernel<128,1,f16 persist,f32 out,nt>",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic("commit_verify_chain_batch1", source_sha(VERIFY_SOURCES)),
            "algorithmic_bytes_per_launch": ledger["fused_total"],
            "avg_launch_us": step_ms * 1e3,
        },
    }
    del sets, fused, verify, commit, step2
    torch.cuda.empty_cache()

    if not args.skip_secondary:
        result["secondary"] = secondary(torch, gb, wl, dev, timer, args)

    if not args.skip_cpu:
        result["cpu_baseline"] = cpu_baseline(wl, w, args.cpu_seconds)

    print(json.dumps(result), flush=True)
    return 0


def secondary(torch, gb, wl, dev, timer, args):
    out = {}
    # tree: 22 nodes, batch 1
    w = wl.WORKLOADS["tree"]
    led = wl.algorithmic_bytes_verify(w)
    sets = make_sets(torch, wl, w, args.sets, dev, tree=True)
    tverify = [gb.gdn_verify_tree(s["parent"], s["q"], s["k"], s["v"], s["alpha"], s["beta"], s["state0"],
                                  out=s["out"], persist=s["persist"], prepare=True) for s in sets]
    tcommit = [gb.gdn_commit(s["accepted"], s["persist"], s["state0"], prepare=True) for s in sets]

    def tstep(i):
        def step():
            tverify[i]()
            tcommit[i]()
        return step

    sm, smed, _ = measure(timer, [tstep(i) for i in range(len(sets))], args.steps, args.warmup)
    km, kmed, _ = measure(timer, tverify, args.steps, args.warmup)
    # one launch per step: commit this set's previous accepted node, then verify its tree
    tfused = [gb.gdn_commit_verify_tree(s["accepted"], s["persist"], s["parent"], s["q"], s["k"], s["v"],
                                        s["alpha"], s["beta"], s["state0"], out=s["out"], persist=s["persist"],
                                        prepare=True) for s in sets]
    fm, fmed, _ = measure(timer, tfused, args.steps, args.warmup)
    out["tree"] = {"nodes_per_s_per_layer": w.n_nodes / (fm * 1e-3), "ms_per_step": fm, "median_ms": fmed,
                   "step_bytes": led["fused_total"],
                   "step_gbs": led["fused_total"] / (fm * 1e-3) / 1e9,
                   "step_hbm_frac": led["fused_total"] / (fm * 1e-3) / 1e9 / HBM_PEAK_GBS,
                   "how": "one launch per step (gdn_commit_verify_tree)",
                   "two_launch": {"nodes_per_s_per_layer": w.n_nodes / (sm * 1e-3), "ms_per_step": sm,
                                  "median_ms": smed, "step_bytes": led["total"]},
                   "verify_us": km * 1e3, "verify_us_median": kmed * 1e3,
                   "verify_gbs": led["verify_total"] / (km * 1e-3) / 1e9,
                   "verify_hbm_frac": led["verify_total"] / (km * 1e-3) / 1e9 / HBM_PEAK_GBS,
                   "verify_bytes": led["verify_total"]}
    log("tree", out["tree"])
    del sets, tverify, tcommit, tfused
    torch.cuda.empty_cache()
    # batched: 8 sequences x 48 layers in one launch
    w = wl.WORKLOADS["batched_chain"]
    led = wl.algorithmic_bytes_verify(w)
    (s,) = make_sets(torch, wl, w, 1, dev)
    bverify = gb.gdn_verify_chain(s["q"], s["k"], s["v"], s["alpha"], s["beta"], s["state0"], out=s["out"],
                                  persist=s["persist"], final_state=s["final"], prepare=True)
    bcommit = gb.gdn_commit(s["accepted"], s["persist"], s["state0"], final_state=s["final"], prepare=True)
    bfused = gb.gdn_commit_verify_chain(s["accepted"], s["persist"], s["q"], s["k"], s["v"], s["alpha"], s["beta"],
                                        s["state0"], final_prev=s["final"], out=s["out"], persist=s["persist"],
                                        final_state=s["final"], prepare=True)

    def bstep():
        bverify()
        bcommit()

    n = max(5, args.steps // 50)
    wb = max(2, args.warmup // 25)
    sm, smed, _ = measure(timer, [bstep], n, wb)
    km, _, _ = measure(timer, [bverify], n, wb)
    fm, fmed, _ = measure(timer, [bfused], n, wb)
    out["batched_chain"] = {"tokens_per_s_per_layer": w.batch * w.n_nodes / (sm * 1e-3),
                            "ms_per_step": sm, "median_ms": smed, "verify_ms": km, "step_bytes": led["total"],
                            "step_hbm_gbs": led["total"] / (sm * 1e-3) / 1e9,
                            "verify_gbs": led["verify_total"] / (km * 1e-3) / 1e9,
                            "commit_ms": sm - km,
                            "fused": {"ms_per_step": fm, "median_ms": fmed,
                                      "tokens_per_s_per_layer": w.batch * w.n_nodes / (fm * 1e-3),
                                      "step_bytes": led["fused_total"],
                                      "step_hbm_gbs": led["fused_total"] / (fm * 1e-3) / 1e9,
                                      "hbm_frac": led["fused_total"] / (fm * 1e-3) / 1e9 / HBM_PEAK_GBS}}
    log("batched_chain", out["batched_chain"])
    del s, bverify, bcommit, bfused
    torch.cuda.empty_cache()
    out["replay_chain"] = bench_replay(torch, gb, wl, dev, timer, args)
    log("replay_chain", out["replay_chain"])
    out["replay_batched_chain"] = bench_replay(torch, gb, wl, dev, timer, args, "batched_chain", 1, n, wb)
    log("replay_batched_chain", out["replay_batched_chain"])
    out["index_chain"] = bench_index(torch, gb, wl, dev, timer, args)
    log("index_chain", out["index_chain"])
    out["prefill"] = bench_prefill(torch, gb, wl, dev, timer, max(10, args.steps // 5))
    log("prefill", out["prefill"])
    out["prefill_varlen"] = bench_prefill_varlen(torch, gb, wl, dev, timer, max(3, args.steps // 100))
    log("prefill_varlen", out["prefill_varlen"])
    return out


def bench_replay(torch, gb, wl, dev, timer, args, name="chain", n_sets=None, steps=None, warmup=None):
    """Decode step with commit by replay: one launch replays the previous
    block's accepted prefix from the cached fp32 state, writes the committed
    state and verifies the next block (outputs only, no persisted node
    states).  At the chain workload the same rotation over buffer sets as the
    headline; at the batched workload one set."""
    w = wl.WORKLOADS[name]
    led = wl.algorithmic_bytes_replay(w)
    calls = []
    for i in range(args.sets if n_sets is None else n_sets):
        base = wl.WORKLOAD_SEEDS[w.name] + 7919 * i
        p = dev_set(torch, wl.make_inputs(w, seed=base), dev)
        s = dev_set(torch, wl.make_inputs(w, seed=base + 1), dev)
        s["out"] = torch.empty(w.batch, w.n_nodes, w.h_v, w.d_v, device=dev)
        calls.append(gb.gdn_replay_verify_chain(p["accepted"], p["q"], p["k"], p["v"], p["alpha"], p["beta"],
                                                s["q"], s["k"], s["v"], s["alpha"], s["beta"], s["state0"],
                                                out=s["out"], prepare=True))
    sm, smed, _ = measure(timer, calls, args.steps if steps is None else steps,
                          args.warmup if warmup is None else warmup)
    res = {"tokens_per_s_per_layer": w.batch * w.n_nodes / (sm * 1e-3), "ms_per_step": sm, "median_ms": smed,
           "kernel_us": sm * 1e3, "step_bytes": led["total"],
           "achieved_gbs": led["total"] / (sm * 1e-3) / 1e9,
           "hbm_frac": led["total"] / (sm * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "kernel": ("replay_verify_chain_kernel<128,1,no persist,f32 out,nt>" if w.batch == 1 else
                      "replay_verify_chain_kernel<128,2,no persist,f32 out>")}
    del calls
    torch.cuda.empty_cache()
    return res


def bench_index(torch, gb, wl, dev, timer, args):
    """Decode step with the index-table commit at the chain workload: verify
    through the index table with fp32 node states persisted into the pool's
    draft rows, then gdn_commit_index (two launches, no state copy).  Each
    buffer set is one pool: the canonical row and 16 draft rows."""
    w = wl.WORKLOADS["chain"]
    led = wl.algorithmic_bytes_index(w)
    N = w.n_nodes
    verify, steps = [], []
    for i in range(args.sets):
        s = dev_set(torch, wl.make_inputs(w, seed=wl.WORKLOAD_SEEDS[w.name] + 7919 * i), dev)
        pool = torch.empty(1 + N, w.h_v, w.d_v, w.d_k, device=dev)
        pool[0] = s["state0"][0]
        slot = torch.zeros(1, dtype=torch.int32, device=dev)
        out = torch.empty(1, N, w.h_v, w.d_v, device=dev)
        v = gb.gdn_verify_chain(s["q"], s["k"], s["v"], s["alpha"], s["beta"], pool, out=out,
                                persist=pool[1:].view(1, N, w.h_v, w.d_v, w.d_k), state_slot=slot, prepare=True)
        c = gb.gdn_commit_index(s["accepted"], slot, N, 1, 1 + N, prepare=True)

        def step(v=v, c=c):
            v()
            c()

        verify.append(v)
        steps.append(step)
    sm, smed, _ = measure(timer, steps, args.steps, args.warmup)
    km, _, _ = measure(timer, verify, args.steps, args.warmup)
    res = {"tokens_per_s_per_layer": w.batch * N / (sm * 1e-3), "ms_per_step": sm, "median_ms": smed,
           "verify_us": km * 1e3, "step_bytes": led["total"], "step_gbs": led["total"] / (sm * 1e-3) / 1e9,
           "verify_gbs": (led["total"] - led["commit"]) / (km * 1e-3) / 1e9,
           "kernel": "verify_chain_kernel<128,1,8,fp32 persist,f32 out,nt> + commit_index_kernel"}
    del verify, steps
    torch.cuda.empty_cache()
    return res


def prefill_flops(w) -> float:
    """Algorithmic matrix FLOPs of the chunked form (full C x C tiles): per
    (chunk, value head) W, U', W H, Q H, P U, K^T U; per (chunk, q/k head)
    K K^T and Q K^T."""
    C, dk, dv = w.chunk, w.d_k, w.d_v
    nch = (w.n_nodes + C - 1) // C
    per_vh = 2 * C * C * dk + 2 * C * C * dv + 3 * 2 * C * dk * dv + 2 * C * C * dv
    per_qk = 2 * 2 * C * C * dk
    return float(w.batch * nch * (w.h_v * per_vh + w.h_qk * per_qk))


def bench_prefill(torch, gb, wl, dev, timer, reps):
    """The 4096-token chunked prefill (out f16).  The state is advanced in
    place by every call (its values do not change the work)."""
    w = wl.WORKLOADS["prefill"]
    t = dev_set(torch, wl.make_inputs(w), dev)
    out = torch.empty(w.batch, w.n_nodes, w.h_v, w.d_v, device=dev, dtype=torch.float16)
    call = gb.gdn_prefill_chunked(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["state0"], out, prepare=True)
    ms, med, _ = measure(timer, [call], reps, 3, settle=SETTLE_S)
    fl = prefill_flops(w)
    return {"ms": ms, "median_ms": med, "tokens_per_s": w.batch * w.n_nodes / (ms * 1e-3),
            "algorithmic_gflop": fl / 1e9, "tflops": fl / (ms * 1e-3) / 1e12,
            "mfma_frac_f16_peak": fl / (ms * 1e-3) / MFMA_F16_PEAK, "out_dtype": "f16"}


def bench_prefill_varlen(torch, gb, wl, dev, timer, reps, n_seq=8):
    """Supplementary batched point: n_seq prompts of the prefill workload's
    shape (4096 tokens each) in one gdn_prefill_varlen call, boundary states
    every 26 chunks (1664 tokens); the graded prefill number is batch 1."""
    w = wl.WORKLOADS["prefill"]
    t = dev_set(torch, wl.make_inputs(w), dev)
    T = w.n_nodes
    q, k, v = (t[n][0].repeat(n_seq, 1, 1) for n in ("q", "k", "v"))
    alpha, beta = (t[n][0].repeat(n_seq, 1) for n in ("alpha", "beta"))
    st = t["state0"].repeat(n_seq, 1, 1, 1)
    out = torch.empty(n_seq * T, w.h_v, w.d_v, device=dev, dtype=torch.float16)
    cu = np.arange(0, (n_seq + 1) * T, T, dtype=np.int32)
    ncs = gb.gdn_prefill_boundary_states(cu, 26)
    cs = torch.empty(ncs, w.h_v, w.d_v, w.d_k, device=dev)
    ws = torch.empty(gb.gdn_prefill_varlen_workspace_bytes(cu, q, v, st, out), dtype=torch.uint8, device=dev)
    call = gb.gdn_prefill_varlen(cu, q, k, v, alpha, beta, st, out, chunk_states=cs, state_interval=26,
                                 workspace=ws, prepare=True)
    ms, med, _ = measure(timer, [call], reps, 2, settle=SETTLE_S)
    fl = prefill_flops(w) * n_seq
    return {"sequences": n_seq, "tokens": n_seq * T, "ms": ms, "median_ms": med,
            "tokens_per_s": n_seq * T / (ms * 1e-3), "tflops": fl / (ms * 1e-3) / 1e12,
            "mfma_frac_f16_peak": fl / (ms * 1e-3) / MFMA_F16_PEAK, "boundary_states": ncs, "out_dtype": "f16"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_baseline(wl, w, seconds):
    """The fp64 oracle on this host: the full step (chain with every node state
    kept, then the commit) on one input set of the workload, repeated for about
    `seconds` with every available core (at most 16), then for a third of that
    on one core."""
    import oracle

    d = wl.make_inputs(w)
    args = [d[n].astype(np.float64) for n in ("q", "k", "v", "alpha", "beta", "state0")]

    def run(nthreads, secs):
        reps, t_total = 0, 0.0
        while t_total < secs or reps == 0:
            t0 = time.perf_counter()
            ref = oracle.chain(*args, nthreads=nthreads)
            oracle.commit(args[5], ref["nodes"], d["accepted"], final=ref["final"])
            t_total += time.perf_counter() - t0
            reps += 1
        return reps, t_total

    nthreads = oracle.default_threads()
    reps, t_total = run(nthreads, seconds)
    reps1, t1 = run(1, seconds / 3)
    return {"value": w.batch * w.n_nodes * reps / t_total, "unit": "tokens/s/layer", "cores": nthreads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "one_core": {"value": w.batch * w.n_nodes * reps1 / t1, "unit": "tokens/s/layer", "cores": 1,
                         "sample": f"{reps1} repetitions, {t1:.1f} s"},
            "sample": f"{reps} repetitions of the full step on one input set of the same workload "
                      f"(48 heads x 16 nodes, fp64, every node state kept, then the commit), {t_total:.1f} s "
                      f"on {nthreads} threads"}


if __name__ == "__main__":
    sys.exit(main())
