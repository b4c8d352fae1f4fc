"""GPU parity of commit by replay (gdn_commit_replay, gdn_replay_verify_chain)
through the C ABI.  The replayed state must equal bit for bit the fp32 node
state a verify computes for the same node (same per-node arithmetic), and
match the fp64 oracle's node state within the state bar (2e-3)."""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_recurrence_gdn_amd import binding as gb
from gated_deltanet_recurrence_gdn_amd import workloads as wl
from helpers import (DEV, OUT_TOL, STATE_TOL, alloc_outputs, dev_inputs, max_rel, run_chain, run_tree, say,
                     small_inputs, to_host)

pytestmark = pytest.mark.gpu


def _replay(t, acc, state, parent=None, slot=None):
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    gb.gdn_commit_replay(torch.as_tensor(acc, dtype=torch.int32).to(DEV), t["q"], t["k"], t["v"], t["alpha"],
                         t["beta"], state, parent=parent, state_slot=slot, status=status)
    torch.cuda.synchronize()
    return int(status.item())


@pytest.mark.parametrize("B,N,Hqk,Hv,dk,dv,bf16", [
    (3, 16, 2, 6, 128, 128, True),
    (2, 1, 1, 2, 64, 64, True),      # one node: the replay is the root alone
    (2, 13, 1, 3, 32, 48, False),    # fp32 inputs, d_k != d_v
])
def test_replay_chain_equals_verify_node_state(B, N, Hqk, Hv, dk, dv, bf16):
    w, d = small_inputs(51, B, N, Hqk, Hv, dk, dv, bf16=bf16)
    t = dev_inputs(d, bf16=bf16)
    _, per, fin = run_chain(t, N, persist_dtype=torch.float32)
    ref = oracle.chain(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"])
    rng = np.random.default_rng(7)
    for acc in (rng.integers(0, N, size=B).astype(np.int32), np.full(B, N - 1, np.int32), np.zeros(B, np.int32)):
        st = t["state0"].clone()
        assert _replay(t, acc, st) == 0
        for b in range(B):
            assert torch.equal(st[b], per[b, int(acc[b])]), (b, int(acc[b]))
        assert torch.equal(st[acc == N - 1], fin[acc == N - 1])
        expect = ref["nodes"][np.arange(B), acc]
        e = max_rel(to_host(st), expect)
        say(f"replay chain B={B} N={N} acc={acc.tolist()} max-rel {e:.2e}")
        assert e <= STATE_TOL


def test_replay_tree_workload_equals_tree_verify():
    w = wl.WORKLOADS["tree"]
    d = wl.make_inputs(w)
    t = dev_inputs(d)
    par = d["parent"]
    say("tree replay parent", par.tolist())
    _, per = run_tree(t, par, w.n_nodes, persist_dtype=torch.float32)
    ref = oracle.tree(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], par)
    for a in [int(d["accepted"][0])] + list(range(w.n_nodes)):
        st = t["state0"].clone()
        assert _replay(t, [a], st, parent=par) == 0
        assert torch.equal(st[0], per[0, a]), a
        assert max_rel(to_host(st), ref["nodes"][:, a]) <= STATE_TOL


def test_replay_per_sequence_trees_across_launches():
    """20 sequences, each with its own tree: replay launches carry 16 trees each."""
    B, N = 20, 12
    w, d = small_inputs(61, B, N, 1, 2, 64, 64, tree=True)
    rng = np.random.default_rng(61)
    pars = np.stack([wl.random_tree(N, 16, rng) for _ in range(B)]).astype(np.int32)
    t = dev_inputs(d)
    _, per = run_tree(t, pars, N, persist_dtype=torch.float32)
    acc = rng.integers(0, N, size=B).astype(np.int32)
    st = t["state0"].clone()
    assert _replay(t, acc, st, parent=pars) == 0
    for b in range(B):
        assert torch.equal(st[b], per[b, int(acc[b])]), b
    ref = oracle.tree(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], pars)
    assert max_rel(to_host(st), ref["nodes"][np.arange(B), acc]) <= STATE_TOL


def test_replay_chain_workload_and_batched_full_size():
    w = wl.WORKLOADS["chain"]
    d = wl.make_inputs(w)
    t = dev_inputs(d)
    st = t["state0"].clone()
    assert _replay(t, d["accepted"], st) == 0
    ref = oracle.chain(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"])
    e = max_rel(to_host(st), ref["nodes"][:, int(d["accepted"][0])])
    say(f"chain workload replay acc={d['accepted'].tolist()} max-rel {e:.2e}")
    assert e <= STATE_TOL
    # 384 units in one launch (two row groups per wave): full acceptance replays to the
    # verify's exact final state; sampled units against the oracle at their drawn length
    w = wl.WORKLOADS["batched_chain"]
    d = wl.make_inputs(w)
    t = dev_inputs(d)
    _, _, fin = run_chain(t, w.n_nodes, persist_dtype=None)
    st = t["state0"].clone()
    assert _replay(t, np.full(w.batch, w.n_nodes - 1, np.int32), st) == 0
    assert torch.equal(st, fin)
    st = t["state0"].clone()
    assert _replay(t, d["accepted"], st) == 0
    for b in (0, 77, 383):
        sl = slice(b, b + 1)
        ref = oracle.chain(d["q"][sl], d["k"][sl], d["v"][sl], d["alpha"][sl], d["beta"][sl], d["state0"][sl])
        assert max_rel(to_host(st[sl]), ref["nodes"][:, int(d["accepted"][b])]) <= STATE_TOL


def test_replay_state_slots_and_bad_entries():
    B, N = 4, 8
    w, d = small_inputs(71, B, N, 1, 2, 64, 64)
    t = dev_inputs(d)
    _, per, _ = run_chain(t, N, persist_dtype=torch.float32)
    # cache of 6 slots; sequence b lives in slot 5 - b
    cache = torch.randn(6, 2, 64, 64, device=DEV)
    slot = torch.tensor([5, 4, 3, 2], dtype=torch.int32, device=DEV)
    for b in range(B):
        cache[5 - b] = t["state0"][b]
    keep = cache.clone()
    acc = np.array([2, 9, 7, 0], np.int32)  # sequence 1: node out of range
    assert _replay(t, acc, cache, slot=slot) == gb.CODES["GDN_ERR_NODE"]
    assert torch.equal(cache[4], keep[4])  # skipped
    assert torch.equal(cache[0], keep[0]) and torch.equal(cache[1], keep[1])  # not addressed
    for b in (0, 2, 3):
        assert torch.equal(cache[5 - b], per[b, int(acc[b])])
    bad = torch.tensor([5, 6, 3, 2], dtype=torch.int32, device=DEV)  # slot 6 out of range
    cache2 = keep.clone()
    assert _replay(t, np.array([1, 1, 1, 1], np.int32), cache2, slot=bad) == gb.CODES["GDN_ERR_SLOT"]
    assert torch.equal(cache2[4], keep[4]) and torch.equal(cache2[5], per[0, 1])


@pytest.mark.parametrize("persist_dtype", [None, torch.float16])
def test_replay_verify_equals_replay_then_verify(persist_dtype):
    B, N = 3, 16
    _, d1 = small_inputs(81, B, N, 2, 6, 128, 128)
    _, d2 = small_inputs(82, B, N, 2, 6, 128, 128)
    t1, t2 = dev_inputs(d1), dev_inputs(d2)
    acc = np.array([3, 15, 0], np.int32)
    st_ref = t1["state0"].clone()
    assert _replay(t1, acc, st_ref) == 0
    out_r, per_r, fin_r = run_chain(t2, N, persist_dtype=persist_dtype, state=st_ref)
    st = t1["state0"].clone()
    out, per, fin = alloc_outputs(t2, N, persist_dtype)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    gb.gdn_replay_verify_chain(torch.from_numpy(acc).to(DEV), t1["q"], t1["k"], t1["v"], t1["alpha"], t1["beta"],
                               t2["q"], t2["k"], t2["v"], t2["alpha"], t2["beta"], st, out=out, persist=per,
                               final_state=fin, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(st, st_ref)
    assert torch.equal(out, out_r) and torch.equal(fin, fin_r)
    if persist_dtype is not None:
        assert torch.equal(per, per_r)


def test_replay_verify_batched_full_size():
    """384 units in one launch (two row groups per wave, both blocks staged):
    the fused replay + verify equals the replay followed by a verify, bit for
    bit, for the committed state and every output; sampled units against the
    oracle."""
    w = wl.WORKLOADS["batched_chain"]
    d1 = wl.make_inputs(w)
    d2 = wl.make_inputs(w, seed=wl.WORKLOAD_SEEDS[w.name] + 1)
    t1, t2 = dev_inputs(d1), dev_inputs(d2)
    acc = torch.from_numpy(np.ascontiguousarray(d1["accepted"], dtype=np.int32)).to(DEV)
    st_ref = t1["state0"].clone()
    assert _replay(t1, d1["accepted"], st_ref) == 0
    out_r, _, _ = run_chain(t2, w.n_nodes, persist_dtype=None, final=False, state=st_ref)
    st = t1["state0"].clone()
    out = torch.full_like(out_r, float("nan"))
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    gb.gdn_replay_verify_chain(acc, t1["q"], t1["k"], t1["v"], t1["alpha"], t1["beta"], t2["q"], t2["k"], t2["v"],
                               t2["alpha"], t2["beta"], st, out=out, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(st, st_ref)
    assert torch.equal(out, out_r)
    for b in (0, 191, 383):
        sl = slice(b, b + 1)
        a = int(d1["accepted"][b])
        ref1 = oracle.chain(d1["q"][sl], d1["k"][sl], d1["v"][sl], d1["alpha"][sl], d1["beta"][sl], d1["state0"][sl])
        s1 = np.ascontiguousarray(ref1["nodes"][:, a])
        ref2 = oracle.chain(d2["q"][sl], d2["k"][sl], d2["v"][sl], d2["alpha"][sl], d2["beta"][sl], s1)
        e_s = max_rel(to_host(st[sl]), s1)
        e_o = max_rel(to_host(out[sl]), ref2["out"])
        say(f"batched replay+verify unit {b} acc={a}: state {e_s:.2e} out {e_o:.2e}")
        assert e_s <= STATE_TOL and e_o <= OUT_TOL


def test_replay_decode_loop_matches_oracle():
    """Four decode steps with one replay + verify launch each (accepted lengths
    vary per sequence) against the oracle applied step by step; the state
    stays exact fp32 throughout."""
    B, N = 2, 16
    steps = [small_inputs(91 + i, B, N, 2, 4, 128, 128)[1] for i in range(4)]
    accs = [np.array([4, 9], np.int32), np.array([15, 15], np.int32), np.array([0, 7], np.int32),
            np.array([11, 2], np.int32)]
    st = dev_inputs(steps[0])["state0"].clone()
    ref_state = steps[0]["state0"].astype(np.float64)
    prev = None
    for i, d in enumerate(steps):
        t = dev_inputs(d)
        out, _, _ = alloc_outputs(t, N, persist_dtype=None, final=False)
        if i == 0:
            gb.gdn_verify_chain(t["q"], t["k"], t["v"], t["alpha"], t["beta"], st, out=out)
        else:
            tp, acc = prev
            gb.gdn_replay_verify_chain(acc, tp["q"], tp["k"], tp["v"], tp["alpha"], tp["beta"], t["q"], t["k"],
                                       t["v"], t["alpha"], t["beta"], st, out=out)
        torch.cuda.synchronize()
        ref = oracle.chain(d["q"], d["k"], d["v"], d["alpha"], d["beta"], ref_state)
        e = max_rel(to_host(out), ref["out"])
        say(f"replay decode step {i}: out max-rel {e:.2e}")
        assert e <= OUT_TOL
        ref_state = ref["nodes"][np.arange(B), accs[i]]
        prev = (t, torch.from_numpy(accs[i]).to(DEV))
    assert _replay(prev[0], accs[-1], st) == 0
    e = max_rel(to_host(st), ref_state)
    say(f"replay decode final state max-rel {e:.2e}")
    assert e <= STATE_TOL
