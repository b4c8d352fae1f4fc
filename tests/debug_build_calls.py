"""Calls of every entry point on the index-checked build of the library
(libgdn_debug.so, -DGDN_DEBUG), run as a child process of
tests/test_gpu_debug_build.py with GDN_LIBRARY pointing at it.  After each call
the status word must still read GDN_OK (an index past its array's end would
set GDN_ERR_INTERNAL); the results are checked against the fp64 oracle at the
parity bar.  Prints one line per call and 'debug build: all calls clean'."""
import os
import sys

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import oracle  # noqa: E402
from gated_deltanet_recurrence_gdn_amd import binding as gb  # noqa: E402
from gated_deltanet_recurrence_gdn_amd import workloads as wl  # noqa: E402
from helpers import DEV, OUT_TOL, PERSIST_TOL, STATE_TOL, dev_inputs, max_rel, to_host  # noqa: E402


def clean(status, what):
    torch.cuda.synchronize()
    code = int(status.item())
    print(what, "status", code, flush=True)
    assert code == 0, (what, gb.STATUS.get(code, code))


def check(x, ref, tol, what):
    e = max_rel(to_host(x), ref)
    assert e <= tol, (what, e)


def main():
    assert os.environ.get("GDN_LIBRARY", "").endswith("libgdn_debug.so"), "run with GDN_LIBRARY set"
    assert gb.lib()._name.endswith("libgdn_debug.so")
    st = torch.zeros(1, dtype=torch.int32, device=DEV)

    # chain verify + commit + fused commit-verify + replay, two shapes (bf16 and fp32 inputs)
    for (B, N, Hqk, Hv, dk, dv, bf16) in [(2, 16, 2, 6, 128, 128, True), (3, 7, 1, 3, 64, 32, False)]:
        w = wl.Workload("custom", B, N, Hqk, Hv, dk, dv, qkv_bf16=bf16)
        d = wl.make_inputs(w, seed=77)
        t = dev_inputs(d, bf16=bf16)
        ref = oracle.chain(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"])
        out = torch.empty(B, N, Hv, dv, device=DEV)
        per = torch.empty(B, N, Hv, dv, dk, device=DEV, dtype=torch.float16)
        fin = torch.empty(B, Hv, dv, dk, device=DEV)
        gb.gdn_verify_chain(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["state0"], out=out, persist=per,
                            final_state=fin, status=st)
        clean(st, f"verify_chain {w.batch}x{w.n_nodes} d_k={dk}")
        check(out, ref["out"], OUT_TOL, "chain out")
        check(per, ref["nodes"], PERSIST_TOL, "chain persist")
        check(fin, ref["final"], STATE_TOL, "chain final")
        acc = torch.from_numpy(d["accepted"]).to(DEV)
        cache = t["state0"].clone()
        gb.gdn_commit(acc, per, cache, final_state=fin, status=st)
        clean(st, "commit")
        cache2 = t["state0"].clone()
        out2 = torch.empty_like(out)
        per2 = torch.empty_like(per)
        fin2 = torch.empty_like(fin)
        gb.gdn_commit_verify_chain(acc, per, t["q"], t["k"], t["v"], t["alpha"], t["beta"], cache2, final_prev=fin,
                                   out=out2, persist=per2, final_state=fin2, status=st)
        clean(st, "commit_verify_chain")
        assert torch.equal(cache2, cache)
        cache3 = t["state0"].clone()
        gb.gdn_commit_replay(acc, t["q"], t["k"], t["v"], t["alpha"], t["beta"], cache3, status=st)
        clean(st, "commit_replay")
        cache4 = t["state0"].clone()
        gb.gdn_replay_verify_chain(acc, t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["q"], t["k"], t["v"],
                                   t["alpha"], t["beta"], cache4, out=out2, persist=per2, final_state=fin2, status=st)
        clean(st, "replay_verify_chain")
        assert torch.equal(cache4, cache3)

    # tree verify, fused tree step, tree replay, through state slots
    w = wl.WORKLOADS["tree"]
    w = wl.Workload("custom", 2, w.n_nodes, 2, 6, 128, 128, tree=True, max_depth=w.max_depth)
    d = wl.make_inputs(w, seed=78)
    t = dev_inputs(d)
    B, N, Hv = w.batch, w.n_nodes, w.h_v
    ref = oracle.tree(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], d["parent"])
    pool = torch.cat([t["state0"], t["state0"]])
    slot = torch.tensor([3, 0], dtype=torch.int32, device=DEV)
    pool[3] = t["state0"][0]
    pool[0] = t["state0"][1]
    out = torch.empty(B, N, Hv, 128, device=DEV)
    per = torch.empty(B, N, Hv, 128, 128, device=DEV, dtype=torch.float16)
    gb.gdn_verify_tree(d["parent"], t["q"], t["k"], t["v"], t["alpha"], t["beta"], pool, out=out, persist=per,
                       state_slot=slot, status=st)
    clean(st, "verify_tree (slots)")
    check(out, ref["out"], OUT_TOL, "tree out")
    acc = torch.from_numpy(d["accepted"]).to(DEV)
    gb.gdn_commit_verify_tree(acc, per, d["parent"], t["q"], t["k"], t["v"], t["alpha"], t["beta"], pool,
                              out=out, persist=torch.empty_like(per), state_slot=slot, status=st)
    clean(st, "commit_verify_tree (slots)")
    gb.gdn_commit_replay(acc, t["q"], t["k"], t["v"], t["alpha"], t["beta"], pool, parent=d["parent"],
                         state_slot=slot, status=st)
    clean(st, "commit_replay (tree, slots)")

    # index-table commit and the convolution history
    table = torch.tensor([0, 1], dtype=torch.int32, device=DEV)
    gb.gdn_commit_index(acc, table, N, 8, 8 + B * N, status=st)
    clean(st, "commit_index")
    x = torch.randn(B, N, 96, device=DEV)
    hist = torch.randn(B, 3, 96, device=DEV)
    gb.gdn_conv_commit(acc, x, hist, parent=d["parent"], status=st)
    clean(st, "conv_commit (tree)")

    # prefill: chunked (ragged), varlen with boundary states, the no-allocation call
    w = wl.Workload("custom", 2, 150, 2, 6, 128, 64)
    d = wl.make_inputs(w, seed=79)
    t = dev_inputs(d)
    ref = oracle.chain(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], nodes=False)
    s1 = t["state0"].clone()
    o1 = torch.empty(2, 150, 6, 64, device=DEV)
    gb.gdn_prefill_chunked(t["q"], t["k"], t["v"], t["alpha"], t["beta"], s1, o1, status=st)
    clean(st, "prefill_chunked")
    check(o1, ref["out"], OUT_TOL, "prefill out")
    check(s1, ref["final"], STATE_TOL, "prefill final")
    s2 = t["state0"].clone()
    o2 = torch.empty_like(o1)
    gb.gdn_prefill_chunked_noalloc(t["q"], t["k"], t["v"], t["alpha"], t["beta"], s2, o2, status=st)
    clean(st, "prefill_chunked_noalloc")
    assert torch.equal(o2, o1) and torch.equal(s2, s1)
    cu = np.array([0, 150, 300], dtype=np.int32)
    flat = {n: t[n].reshape(300, *t[n].shape[2:]) for n in ("q", "k", "v", "alpha", "beta")}
    s3 = t["state0"].clone()
    o3 = torch.empty(300, 6, 64, device=DEV)
    cs = torch.empty(gb.gdn_prefill_boundary_states(cu, 1), 6, 64, 128, device=DEV)
    gb.gdn_prefill_varlen(cu, flat["q"], flat["k"], flat["v"], flat["alpha"], flat["beta"], s3, o3,
                          chunk_states=cs, state_interval=1, status=st)
    clean(st, "prefill_varlen (boundary states)")
    assert torch.equal(o3.view(2, 150, 6, 64), o1) and torch.equal(s3, s1)
    print("debug build: all calls clean", flush=True)


if __name__ == "__main__":
    main()
