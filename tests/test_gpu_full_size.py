"""Full-size parity of the launches the benchmark times, in the benchmark's own
configuration, against the fp64 oracle through the C ABI.

- the fused commit + verify (one launch per decode step) at batch 1, 16 q/k
  and 48 value heads, d = 128, 16 nodes, committing from the very buffers it
  writes (the benchmark's aliasing);
- the same launch at 384 units (8 sequences x 48 layers), the instance with two
  row groups per wave and plain stores, on every unit;
- the 22-node tree step in one launch (fused commit + tree verify) at batch 1,
  with the same aliasing;
- two launches on two streams back to back.
Bars: max relative error <= 2e-3 on outputs and fp32 states, <= 1e-2 on the f16
persisted states; the committed state bit-exact with its source."""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_recurrence_gdn_amd import binding as gb
from gated_deltanet_recurrence_gdn_amd import workloads as wl
from helpers import (DEV, OUT_TOL, PERSIST_TOL, STATE_TOL, alloc_outputs, dev_inputs, max_rel, run_chain, run_tree,
                     say, small_inputs, to_host)

pytestmark = pytest.mark.gpu


def committed_source(persist, fin, acc):
    """What the commit must write for each sequence: the accepted node's
    persisted copy widened, or the exact final state on full acceptance."""
    a = acc.long()
    src = persist[torch.arange(persist.shape[0], device=DEV), a].float()
    full = a == persist.shape[1] - 1
    src[full] = fin[full]
    return src


def fused_step(w, seed_prev, seed_next):
    """Verify block 1 (plain launch), then one fused launch that commits block
    1's accepted node and verifies block 2 over the same out/persist/final
    buffers.  Returns the inputs, the saved block-1 results and block 2's."""
    d1 = wl.make_inputs(w, seed=seed_prev)
    d2 = wl.make_inputs(w, seed=seed_next)
    t1, t2 = dev_inputs(d1), dev_inputs(d2)
    out, per, fin = run_chain(t1, w.n_nodes)
    source = committed_source(per, fin, torch.from_numpy(d1["accepted"]).to(DEV))
    state = t1["state0"].clone()
    acc = torch.from_numpy(d1["accepted"]).to(DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    gb.gdn_commit_verify_chain(acc, per, t2["q"], t2["k"], t2["v"], t2["alpha"], t2["beta"], state,
                               final_prev=fin, out=out, persist=per, final_state=fin, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return d1, d2, t2, source, state, out, per, fin


def test_fused_step_at_batch_one_full_size():
    w = wl.WORKLOADS["chain"]
    seed = wl.WORKLOAD_SEEDS["chain"]
    d1, d2, t2, source, state, out, per, fin = fused_step(w, seed, seed + 7919)
    say("fused step, batch 1: accepted", d1["accepted"])
    # the commit: bit for bit the accepted node's persisted copy (or the final state)
    assert torch.equal(state, source)
    # block 2 from the committed state, against the oracle run from that state
    ref = oracle.chain(d2["q"], d2["k"], d2["v"], d2["alpha"], d2["beta"], to_host(state))
    e = (max_rel(to_host(out), ref["out"]), max_rel(to_host(fin), ref["final"]),
         max_rel(to_host(per), ref["nodes"]))
    say(f"fused step vs oracle from the committed state: out {e[0]:.2e} final {e[1]:.2e} persist {e[2]:.2e}")
    assert e[0] <= OUT_TOL and e[1] <= STATE_TOL and e[2] <= PERSIST_TOL
    # and against the oracle end to end (block 1 in fp64, commit in fp64, block 2 in fp64)
    ref1 = oracle.chain(d1["q"], d1["k"], d1["v"], d1["alpha"], d1["beta"], d1["state0"])
    st64, _ = oracle.commit(d1["state0"].astype(np.float64), ref1["nodes"], d1["accepted"], final=ref1["final"])
    assert max_rel(to_host(state), st64) <= STATE_TOL
    ref2 = oracle.chain(d2["q"], d2["k"], d2["v"], d2["alpha"], d2["beta"], st64)
    assert max_rel(to_host(out), ref2["out"]) <= OUT_TOL
    assert max_rel(to_host(fin), ref2["final"]) <= STATE_TOL
    # and bit for bit the two-launch step (commit, then verify)
    o2, p2, f2 = run_chain(t2, w.n_nodes, state=source.clone())
    assert torch.equal(out, o2) and torch.equal(per, p2) and torch.equal(fin, f2)


def test_fused_tree_step_at_batch_one_full_size():
    """The 22-node tree step in one launch, in the benchmark's configuration and aliasing: block 2's tree
    verified over the out/persist buffers block 1's accepted node is committed from."""
    w = wl.WORKLOADS["tree"]
    seed = wl.WORKLOAD_SEEDS["tree"]
    d1 = wl.make_inputs(w, seed=seed)
    d2 = wl.make_inputs(w, seed=seed + 7919)
    t1, t2 = dev_inputs(d1), dev_inputs(d2)
    out, per = run_tree(t1, d1["parent"], w.n_nodes)
    acc = torch.from_numpy(d1["accepted"]).to(DEV)
    source = per[torch.arange(w.batch, device=DEV), acc.long()].float()
    state = t1["state0"].clone()
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    gb.gdn_commit_verify_tree(acc, per, d2["parent"], t2["q"], t2["k"], t2["v"], t2["alpha"], t2["beta"], state,
                              out=out, persist=per, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    say("fused tree step, batch 1: accepted", d1["accepted"])
    assert torch.equal(state, source)
    ref = oracle.tree(d2["q"], d2["k"], d2["v"], d2["alpha"], d2["beta"], to_host(state), d2["parent"])
    e = (max_rel(to_host(out), ref["out"]), max_rel(to_host(per), ref["nodes"]))
    say(f"fused tree step vs oracle from the committed state: out {e[0]:.2e} persist {e[1]:.2e}")
    assert e[0] <= OUT_TOL and e[1] <= PERSIST_TOL
    # end to end in fp64: block 1's tree, the commit of its accepted node, block 2's tree
    ref1 = oracle.tree(d1["q"], d1["k"], d1["v"], d1["alpha"], d1["beta"], d1["state0"], d1["parent"])
    st64, _ = oracle.commit(d1["state0"].astype(np.float64), ref1["nodes"], d1["accepted"])
    assert max_rel(to_host(state), st64) <= PERSIST_TOL  # the commit source is the f16 copy
    ref2 = oracle.tree(d2["q"], d2["k"], d2["v"], d2["alpha"], d2["beta"], st64, d2["parent"])
    assert max_rel(to_host(out), ref2["out"]) <= OUT_TOL
    # and bit for bit the two-launch step (commit, then tree verify)
    o2, p2 = run_tree({**t2, "state0": source.clone()}, d2["parent"], w.n_nodes)
    assert torch.equal(out, o2) and torch.equal(per, p2)


def test_fused_step_at_384_units_every_unit():
    w = wl.WORKLOADS["batched_chain"]
    seed = wl.WORKLOAD_SEEDS["batched_chain"]
    d1, d2, t2, source, state, out, per, fin = fused_step(w, seed, seed + 7919)
    assert torch.equal(state, source)
    # bit for bit the two-launch step
    o2, p2, f2 = run_chain(t2, w.n_nodes, state=source.clone())
    assert torch.equal(out, o2) and torch.equal(fin, f2) and torch.equal(per, p2)
    del o2, p2, f2
    # every unit's outputs and final state against the oracle, 48 units per call
    st_host = to_host(state)
    worst = [0.0, 0.0]
    for b0 in range(0, w.batch, 48):
        sl = slice(b0, b0 + 48)
        ref = oracle.chain(d2["q"][sl], d2["k"][sl], d2["v"][sl], d2["alpha"][sl], d2["beta"][sl], st_host[sl],
                           nodes=False)
        worst[0] = max(worst[0], max_rel(to_host(out[sl]), ref["out"]))
        worst[1] = max(worst[1], max_rel(to_host(fin[sl]), ref["final"]))
    say(f"384 units, worst batch of 48: out {worst[0]:.2e} final {worst[1]:.2e}")
    assert worst[0] <= OUT_TOL and worst[1] <= STATE_TOL
    # persisted states of a spread of units (each unit's 16 node states whole)
    for b in (0, 47, 100, 191, 255, 383):
        sl = slice(b, b + 1)
        ref = oracle.chain(d2["q"][sl], d2["k"][sl], d2["v"][sl], d2["alpha"][sl], d2["beta"][sl], st_host[sl])
        ep = max_rel(to_host(per[sl]), ref["nodes"])
        assert ep <= PERSIST_TOL, (b, ep)


def test_two_streams_back_to_back():
    """Two calls issued back to back on two streams (no synchronisation between
    them) give the results each gives alone."""
    _, da = small_inputs(61, 2, 16, 4, 12, 128, 128)
    _, db = small_inputs(62, 3, 16, 2, 6, 64, 64)
    ta, tb = dev_inputs(da), dev_inputs(db)
    ref_a = run_chain(ta, 16)
    ref_b = run_chain(tb, 16)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    oa, pa, fa = alloc_outputs(ta, 16)
    ob, pb, fb = alloc_outputs(tb, 16)
    torch.cuda.synchronize()
    for _ in range(3):
        gb.gdn_verify_chain(ta["q"], ta["k"], ta["v"], ta["alpha"], ta["beta"], ta["state0"], out=oa, persist=pa,
                            final_state=fa, stream=sa)
        gb.gdn_verify_chain(tb["q"], tb["k"], tb["v"], tb["alpha"], tb["beta"], tb["state0"], out=ob, persist=pb,
                            final_state=fb, stream=sb)
    sa.synchronize()
    sb.synchronize()
    assert torch.equal(oa, ref_a[0]) and torch.equal(pa, ref_a[1]) and torch.equal(fa, ref_a[2])
    assert torch.equal(ob, ref_b[0]) and torch.equal(pb, ref_b[1]) and torch.equal(fb, ref_b[2])
