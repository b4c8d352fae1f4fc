#!/usr/bin/env python3
"""Throughput of the verify + commit step on one MI355X.

One step = gdn_verify_chain over a 16-node draft (batch 1, 16 q/k heads,
48 value heads, d_k = d_v = 128, bf16 q/k/v, fp32 state, f16 persisted node
states, fp32 outputs and final state) followed by gdn_commit of a seeded
accepted length.  The metric is verified draft tokens per second per GDN
layer: 16 nodes per step per layer.

Inputs are resident in device memory before the timed region.  Steps rotate
over enough independent buffer sets (> 256 MB in total) that the 256 MB
Infinity Cache cannot hold one step's data from the previous visit, so every
step streams its state and writes its node states to HBM.

Printed: one JSON line with the metric, the roofline of the verify kernel
(algorithmic bytes per launch / average launch time from HIP events), the
oracle timed on this host's cores, and secondary measurements of the tree
and batched workloads.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
VERIFY_SOURCES = ["gated_deltanet_recurrence_gdn_amd/csrc/verify.hip",
                  "gated_deltanet_recurrence_gdn_amd/csrc/gdn_device.h",
                  "gated_deltanet_recurrence_gdn_amd/csrc/gdn_internal.h"]


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
METRIC = "verified draft tokens/s per GDN layer (48 v-heads, d=128) + % HBM roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


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


def time_steps(torch, sets, step_fn, kernel_fn, steps, warmup):
    """Whole-step time and verify-kernel time, both from HIP events on the
    launching stream (torch's current stream).  The step region times K
    verify + commit steps; the kernel region times K verify launches back to
    back over the same rotating sets, so its per-launch average is the
    kernel's duration including its launch and drain, as a kernel trace
    reports it."""
    for i in range(warmup):
        step_fn(sets[i % len(sets)])
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        step_fn(sets[i % len(sets)])
    t1.record()
    torch.cuda.synchronize()
    step_ms = t0.elapsed_time(t1) / steps
    t0.record()
    for i in range(steps):
        kernel_fn(sets[i % len(sets)])
    t1.record()
    torch.cuda.synchronize()
    kern_ms = t0.elapsed_time(t1) / steps
    return step_ms, kern_ms


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--sets", type=int, default=12, help="rotating buffer sets (chain and tree)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU work of the oracle baseline")
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
    if args.only_prefill:
        print(json.dumps({"prefill": bench_prefill(torch, gb, wl, dev, max(5, args.steps // 25))}), flush=True)
        return 0
    w = wl.WORKLOADS["chain"]
    ledger = wl.algorithmic_bytes_verify(w)
    sets = make_sets(torch, wl, w, args.sets, dev)
    set_bytes = ledger["total"]
    log(f"chain: {args.sets} buffer sets, {set_bytes * args.sets / 1e6:.0f} MB rotated")

    def verify_fn(s):
        gb.gdn_verify_chain(s["q"], s["k"], s["v"], s["alpha"], s["beta"], s["state0"], out=s["out"],
                            persist=s["persist"], final_state=s["final"])

    def step2(s):  # two launches: verify, then commit
        verify_fn(s)
        gb.gdn_commit(s["accepted"], s["persist"], s["state0"], final_state=s["final"])

    def fused(s):  # one launch: commit this set's previous accepted node, then verify
        gb.gdn_commit_verify_chain(s["accepted"], s["persist"], s["q"], s["k"], s["v"], s["alpha"], s["beta"],
                                   s["state0"], final_prev=s["final"], out=s["out"], persist=s["persist"],
                                   final_state=s["final"])

    for s in sets:  # every set has a verified block to commit before the first fused step
        verify_fn(s)
    step_ms, kern_ms = time_steps(torch, sets, fused, fused, args.steps, args.warmup)
    step2_ms, verify_ms = time_steps(torch, sets, step2, verify_fn, args.steps, args.warmup)
    tokens_per_step = w.batch * w.n_nodes
    value = tokens_per_step / (step_ms * 1e-3)
    achieved = ledger["fused_total"] / (kern_ms * 1e-3) / 1e9
    log(f"chain fused step {step_ms * 1e3:.2f} us ({achieved:.0f} GB/s); two-launch step {step2_ms * 1e3:.2f} us, "
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
            "step_hbm_gbs": ledger["fused_total"] / (step_ms * 1e-3) / 1e9,
            "step_hbm_frac": ledger["fused_total"] / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "two_launch_step": {"ms_per_step": step2_ms, "tokens_per_s_per_layer": tokens_per_step / (step2_ms * 1e-3),
                                "step_bytes": set_bytes, "verify_kernel_us": verify_ms * 1e3,
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
            "avg_launch_us": kern_ms * 1e3,
        },
    }
    del sets
    torch.cuda.empty_cache()

    if not args.skip_secondary:
        result["secondary"] = secondary(torch, gb, wl, dev, args)

    if not args.skip_cpu:
        result["cpu_baseline"] = cpu_baseline(wl, w, args.cpu_seconds)

    print(json.dumps(result), flush=True)
    return 0


def secondary(torch, gb, wl, dev, args):
    out = {}
    # tree: 22 nodes, batch 1
    w = wl.WORKLOADS["tree"]
    led = wl.algorithmic_bytes_verify(w)
    sets = make_sets(torch, wl, w, args.sets, dev, tree=True)

    def tverify(s):
        gb.gdn_verify_tree(s["parent"], s["q"], s["k"], s["v"], s["alpha"], s["beta"], s["state0"], out=s["out"],
                           persist=s["persist"])

    def tstep(s, verify=True):
        if verify:
            tverify(s)
        gb.gdn_commit(s["accepted"], s["persist"], s["state0"])

    sm, km = time_steps(torch, sets, tstep, tverify, args.steps, args.warmup)
    out["tree"] = {"nodes_per_s_per_layer": w.n_nodes / (sm * 1e-3), "ms_per_step": sm, "verify_us": km * 1e3,
                   "verify_gbs": led["verify_total"] / (km * 1e-3) / 1e9, "step_bytes": led["total"]}
    log("tree", out["tree"])
    del sets
    torch.cuda.empty_cache()
    # batched: 8 sequences x 48 layers in one launch
    w = wl.WORKLOADS["batched_chain"]
    led = wl.algorithmic_bytes_verify(w)
    sets = make_sets(torch, wl, w, 1, dev)

    def bverify(s):
        gb.gdn_verify_chain(s["q"], s["k"], s["v"], s["alpha"], s["beta"], s["state0"], out=s["out"],
                            persist=s["persist"], final_state=s["final"])

    def bstep(s, verify=True):
        if verify:
            bverify(s)
        gb.gdn_commit(s["accepted"], s["persist"], s["state0"], final_state=s["final"])

    def bfused(s):
        gb.gdn_commit_verify_chain(s["accepted"], s["persist"], s["q"], s["k"], s["v"], s["alpha"], s["beta"],
                                   s["state0"], final_prev=s["final"], out=s["out"], persist=s["persist"],
                                   final_state=s["final"])

    n = max(5, args.steps // 50)
    sm, km = time_steps(torch, sets, bstep, bverify, n, max(2, args.warmup // 25))
    fm, _ = time_steps(torch, sets, bfused, bfused, n, 1)
    out["batched_chain"] = {"tokens_per_s_per_layer": w.batch * w.n_nodes / (sm * 1e-3),
                            "ms_per_step": sm, "verify_ms": km, "step_bytes": led["total"],
                            "step_hbm_gbs": led["total"] / (sm * 1e-3) / 1e9,
                            "verify_gbs": led["verify_total"] / (km * 1e-3) / 1e9,
                            "commit_ms": sm - km,
                            "fused": {"ms_per_step": fm, "tokens_per_s_per_layer": w.batch * w.n_nodes / (fm * 1e-3),
                                      "step_bytes": led["fused_total"],
                                      "step_hbm_gbs": led["fused_total"] / (fm * 1e-3) / 1e9}}
    log("batched_chain", out["batched_chain"])
    del sets
    torch.cuda.empty_cache()
    out["replay_chain"] = bench_replay(torch, gb, wl, dev, args)
    log("replay_chain", out["replay_chain"])
    out["replay_batched_chain"] = bench_replay(torch, gb, wl, dev, args, "batched_chain", 1, n,
                                               max(2, args.warmup // 25))
    log("replay_batched_chain", out["replay_batched_chain"])
    out["index_chain"] = bench_index(torch, gb, wl, dev, args)
    log("index_chain", out["index_chain"])
    out["prefill"] = bench_prefill(torch, gb, wl, dev, max(5, args.steps // 25))
    log("prefill", out["prefill"])
    out["prefill_varlen"] = bench_prefill_varlen(torch, gb, wl, dev, max(3, args.steps // 100))
    log("prefill_varlen", out["prefill_varlen"])
    return out


def bench_replay(torch, gb, wl, dev, args, name="chain", n_sets=None, steps=None, warmup=None):
    """Decode step with commit by replay: one launch replays the previous
    block's accepted prefix from the cached fp32 state, writes the committed
    state and verifies the next block (outputs only, no persisted node
    states).  At the chain workload the same rotation over buffer sets as the
    headline; at the batched workload one set."""
    w = wl.WORKLOADS[name]
    led = wl.algorithmic_bytes_replay(w)
    sets = []
    for i in range(args.sets if n_sets is None else n_sets):
        base = wl.WORKLOAD_SEEDS[w.name] + 7919 * i
        prev = dev_set(torch, wl.make_inputs(w, seed=base), dev)
        cur = dev_set(torch, wl.make_inputs(w, seed=base + 1), dev)
        cur["out"] = torch.empty(w.batch, w.n_nodes, w.h_v, w.d_v, device=dev)
        cur["prev"] = prev
        sets.append(cur)

    def step(s):
        p = s["prev"]
        gb.gdn_replay_verify_chain(p["accepted"], p["q"], p["k"], p["v"], p["alpha"], p["beta"], s["q"], s["k"],
                                   s["v"], s["alpha"], s["beta"], s["state0"], out=s["out"])

    sm, km = time_steps(torch, sets, step, step, args.steps if steps is None else steps,
                        args.warmup if warmup is None else warmup)
    res = {"tokens_per_s_per_layer": w.batch * w.n_nodes / (sm * 1e-3), "ms_per_step": sm,
           "kernel_us": km * 1e3, "step_bytes": led["total"],
           "achieved_gbs": led["total"] / (km * 1e-3) / 1e9,
           "hbm_frac": led["total"] / (km * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "kernel": ("replay_verify_chain_kernel<128,1,no persist,f32 out,nt>" if w.batch == 1 else
                      "replay_verify_chain_kernel<128,2,no persist,f32 out>")}
    del sets
    torch.cuda.empty_cache()
    return res


def bench_index(torch, gb, wl, dev, args):
    """Decode step with the index-table commit at the chain workload: verify
    through the index table with fp32 node states persisted into the pool's
    draft rows, then gdn_commit_index (two launches, no state copy).  Each
    buffer set is one pool: the canonical row and 16 draft rows."""
    w = wl.WORKLOADS["chain"]
    led = wl.algorithmic_bytes_index(w)
    N = w.n_nodes
    sets = []
    for i in range(args.sets):
        s = dev_set(torch, wl.make_inputs(w, seed=wl.WORKLOAD_SEEDS[w.name] + 7919 * i), dev)
        pool = torch.empty(1 + N, w.h_v, w.d_v, w.d_k, device=dev)
        pool[0] = s["state0"][0]
        s["pool"], s["persist"] = pool, pool[1:].view(1, N, w.h_v, w.d_v, w.d_k)
        s["slot"] = torch.zeros(1, dtype=torch.int32, device=dev)
        s["out"] = torch.empty(1, N, w.h_v, w.d_v, device=dev)
        sets.append(s)

    def verify(s):
        gb.gdn_verify_chain(s["q"], s["k"], s["v"], s["alpha"], s["beta"], s["pool"], out=s["out"],
                            persist=s["persist"], state_slot=s["slot"])

    def step(s):
        verify(s)
        gb.gdn_commit_index(s["accepted"], s["slot"], N, 1, 1 + N)

    sm, km = time_steps(torch, sets, step, verify, args.steps, args.warmup)
    res = {"tokens_per_s_per_layer": w.batch * N / (sm * 1e-3), "ms_per_step": sm, "verify_us": km * 1e3,
           "step_bytes": led["total"], "step_gbs": led["total"] / (sm * 1e-3) / 1e9,
           "verify_gbs": (led["total"] - led["commit"]) / (km * 1e-3) / 1e9,
           "kernel": "verify_chain_kernel<128,1,8,fp32 persist,f32 out,nt> + commit_index_kernel"}
    del sets
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


def bench_prefill(torch, gb, wl, dev, reps):
    w = wl.WORKLOADS["prefill"]
    d = wl.make_inputs(w)
    t = dev_set(torch, d, dev)
    out = torch.empty(w.batch, w.n_nodes, w.h_v, w.d_v, device=dev, dtype=torch.float16)
    st = t["state0"].clone()

    def run():
        st.copy_(t["state0"])
        gb.gdn_prefill_chunked(t["q"], t["k"], t["v"], t["alpha"], t["beta"], st, out)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    copy_ms = 0.0
    t0.record()
    for _ in range(reps):
        st.copy_(t["state0"])
    t1.record()
    torch.cuda.synchronize()
    copy_ms = t0.elapsed_time(t1) / reps
    t0.record()
    for _ in range(reps):
        run()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps - copy_ms
    fl = prefill_flops(w)
    return {"ms": ms, "tokens_per_s": w.batch * w.n_nodes / (ms * 1e-3), "algorithmic_gflop": fl / 1e9,
            "tflops": fl / (ms * 1e-3) / 1e12, "mfma_frac_f16_peak": fl / (ms * 1e-3) / 2.5e15,
            "out_dtype": "f16"}


def bench_prefill_varlen(torch, gb, wl, dev, reps, n_seq=8):
    """Supplementary batched point: n_seq prompts of the prefill workload's
    shape (4096 tokens each) in one gdn_prefill_varlen call, boundary states
    every 26 chunks (1664 tokens); the graded prefill number is batch 1."""
    w = wl.WORKLOADS["prefill"]
    d = wl.make_inputs(w)
    t = dev_set(torch, d, dev)
    T = w.n_nodes
    q, k, v = (t[n][0].repeat(n_seq, 1, 1) for n in ("q", "k", "v"))
    alpha, beta = (t[n][0].repeat(n_seq, 1) for n in ("alpha", "beta"))
    st0 = t["state0"].repeat(n_seq, 1, 1, 1)
    st = st0.clone()
    out = torch.empty(n_seq * T, w.h_v, w.d_v, device=dev, dtype=torch.float16)
    cu = np.arange(0, (n_seq + 1) * T, T, dtype=np.int32)
    ncs = gb.gdn_prefill_boundary_states(cu, 26)
    cs = torch.empty(ncs, w.h_v, w.d_v, w.d_k, device=dev)
    ws = torch.empty(gb.gdn_prefill_varlen_workspace_bytes(cu, q, v, st, out), dtype=torch.uint8, device=dev)

    def run():
        st.copy_(st0)
        gb.gdn_prefill_varlen(cu, q, k, v, alpha, beta, st, out, chunk_states=cs, state_interval=26, workspace=ws)

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        st.copy_(st0)
    t1.record()
    torch.cuda.synchronize()
    copy_ms = t0.elapsed_time(t1) / reps
    t0.record()
    for _ in range(reps):
        run()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps - copy_ms
    fl = prefill_flops(w) * n_seq
    return {"sequences": n_seq, "tokens": n_seq * T, "ms": ms, "tokens_per_s": n_seq * T / (ms * 1e-3),
            "tflops": fl / (ms * 1e-3) / 1e12, "mfma_frac_f16_peak": fl / (ms * 1e-3) / 2.5e15,
            "boundary_states": ncs, "out_dtype": "f16"}


def cpu_baseline(wl, w, seconds):
    import oracle

    d = wl.make_inputs(w)
    nthreads = oracle.default_threads()
    args = [d[n].astype(np.float64) for n in ("q", "k", "v", "alpha", "beta", "state0")]
    reps, t_total = 0, 0.0
    while t_total < seconds or reps == 0:
        t0 = time.perf_counter()
        ref = oracle.chain(*args, nthreads=nthreads)
        oracle.commit(args[5], ref["nodes"], d["accepted"], final=ref["final"])
        t_total += time.perf_counter() - t0
        reps += 1
    return {"value": w.batch * w.n_nodes * reps / t_total, "unit": "tokens/s/layer", "cores": nthreads,
            "kind": "oracle",
            "sample": f"{reps} repetitions of the full step on one input set of the same workload "
                      f"(48 heads x 16 nodes, fp64, every node state kept, then the commit), {t_total:.1f} s"}


if __name__ == "__main__":
    sys.exit(main())
