"""GPU parity of chain / tree verify and commit against the fp64 oracle,
through the C ABI.  Bar: max relative error (max |x - ref| / max |ref|) <= 2e-3
for outputs and fp32 states, <= 1e-2 for persisted f16 states; index and copy
handling bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_recurrence_gdn_amd import binding as gb
from gated_deltanet_recurrence_gdn_amd import workloads as wl
from helpers import (DEV, OUT_TOL, PERSIST_TOL, STATE_TOL, alloc_outputs, dev_inputs, max_rel, run_chain,
                     run_tree, say, small_inputs, to_host)

pytestmark = pytest.mark.gpu


def _commit(t_acc, persist, state, final=None, slot=None):
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    gb.gdn_commit(t_acc, persist, state, final_state=final, state_slot=slot, status=status)
    torch.cuda.synchronize()
    return int(status.item())


# --------------------------------------------------------------------------
# the workloads at full size
# --------------------------------------------------------------------------
def test_tiny_chain_fp32_parity():
    w = wl.WORKLOADS["tiny_chain"]
    d = wl.make_inputs(w)
    say("tiny_chain", w)
    t = dev_inputs(d, bf16=False)
    out, persist, fin = run_chain(t, w.n_nodes, persist_dtype=torch.float32)
    ref = oracle.chain(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"])
    assert max_rel(to_host(out), ref["out"]) <= OUT_TOL
    assert max_rel(to_host(fin), ref["final"]) <= STATE_TOL
    assert max_rel(to_host(persist), ref["nodes"]) <= STATE_TOL
    # fp32 throughout: far inside the bar
    assert max_rel(to_host(out), ref["out"]) <= 1e-5


def test_chain_parity_and_commit():
    w = wl.WORKLOADS["chain"]
    d = wl.make_inputs(w)
    say("chain", w, "accepted", d["accepted"])
    t = dev_inputs(d)
    out, persist, fin = run_chain(t, w.n_nodes)
    ref = oracle.chain(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"])
    e_out, e_fin, e_p = (max_rel(to_host(out), ref["out"]), max_rel(to_host(fin), ref["final"]),
                         max_rel(to_host(persist), ref["nodes"]))
    say(f"chain max-rel out {e_out:.2e} final {e_fin:.2e} persist {e_p:.2e}")
    assert e_out <= OUT_TOL and e_fin <= STATE_TOL and e_p <= PERSIST_TOL
    # commit at the drawn accepted length, and at full acceptance
    for acc in (d["accepted"], np.array([w.n_nodes - 1], np.int32)):
        state = t["state0"].clone()
        assert _commit(torch.from_numpy(acc).to(DEV), persist, state, final=fin) == 0
        a = int(acc[0])
        expect = fin[0] if a == w.n_nodes - 1 else persist[0, a].float()
        assert torch.equal(state[0], expect)
        new, _ = oracle.commit(d["state0"].astype(np.float64), ref["nodes"], acc, final=ref["final"])
        assert max_rel(to_host(state), new) <= STATE_TOL


def test_tree_parity_and_commit():
    w = wl.WORKLOADS["tree"]
    d = wl.make_inputs(w)
    say("tree", w, "parent", d["parent"].tolist(), "accepted", d["accepted"])
    t = dev_inputs(d)
    out, persist = run_tree(t, d["parent"], w.n_nodes)
    ref = oracle.tree(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], d["parent"])
    e_out, e_p = max_rel(to_host(out), ref["out"]), max_rel(to_host(persist), ref["nodes"])
    say(f"tree max-rel out {e_out:.2e} persist {e_p:.2e}")
    assert e_out <= OUT_TOL and e_p <= PERSIST_TOL
    state = t["state0"].clone()
    acc = d["accepted"]
    assert _commit(torch.from_numpy(acc).to(DEV), persist, state) == 0
    assert torch.equal(state[0], persist[0, int(acc[0])].float())
    new, _ = oracle.commit(d["state0"].astype(np.float64), ref["nodes"], acc)
    assert max_rel(to_host(state), new) <= STATE_TOL


@pytest.mark.parametrize("tree", [False, True])
def test_slow_decay_gates(tree):
    """Gates in [0.99, 1] and beta in [0, 1]: no node's state is damped toward
    zero, so every node depends on the cached state and on all its ancestors
    (the workloads' gates decay by about half per node)."""
    w, d = small_inputs(33, 2, 22 if tree else 16, 2, 6, 128, 128, tree=tree)
    rng = np.random.default_rng(6)
    d["alpha"] = (0.99 + 0.01 * rng.random(d["alpha"].shape)).astype(np.float32)
    d["beta"] = rng.random(d["beta"].shape).astype(np.float32)
    t = dev_inputs(d)
    if tree:
        out, persist = run_tree(t, d["parent"], w.n_nodes, persist_dtype=torch.float32)
        ref = oracle.tree(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], d["parent"])
    else:
        out, persist, fin = run_chain(t, w.n_nodes, persist_dtype=torch.float32)
        ref = oracle.chain(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"])
        assert max_rel(to_host(fin), ref["final"]) <= STATE_TOL
    e_out, e_p = max_rel(to_host(out), ref["out"]), max_rel(to_host(persist), ref["nodes"])
    say(f"slow decay {'tree' if tree else 'chain'}: out {e_out:.2e} node states {e_p:.2e}")
    assert e_out <= OUT_TOL and e_p <= STATE_TOL


def test_batched_chain_full_size_sampled():
    """8 sequences x 48 layers in one launch (the benchmark's configuration);
    the oracle checks a sample of whole (sequence x layer) units."""
    w = wl.WORKLOADS["batched_chain"]
    d = wl.make_inputs(w)
    say("batched_chain", w)
    t = dev_inputs(d)
    out, persist, fin = run_chain(t, w.n_nodes)
    state = t["state0"].clone()
    acc_t = torch.from_numpy(d["accepted"]).to(DEV)
    assert _commit(acc_t, persist, state, final=fin) == 0
    for b in (0, 1, 191, 250, w.batch - 1):
        sl = slice(b, b + 1)
        ref = oracle.chain(d["q"][sl], d["k"][sl], d["v"][sl], d["alpha"][sl], d["beta"][sl], d["state0"][sl])
        e = (max_rel(to_host(out[sl]), ref["out"]), max_rel(to_host(fin[sl]), ref["final"]),
             max_rel(to_host(persist[sl]), ref["nodes"]))
        say(f"unit {b}: out {e[0]:.2e} final {e[1]:.2e} persist {e[2]:.2e}")
        assert e[0] <= OUT_TOL and e[1] <= STATE_TOL and e[2] <= PERSIST_TOL
        a = int(d["accepted"][b])
        expect = fin[b] if a == w.n_nodes - 1 else persist[b, a].float()
        assert torch.equal(state[b], expect)
    # units not sampled: every committed state equals its source (bit-exact index work)
    a = acc_t.long()
    src = persist[torch.arange(w.batch, device=DEV), a].float()
    full = a == w.n_nodes - 1
    src[full] = fin[full]
    assert torch.equal(state, src)


# --------------------------------------------------------------------------
# shapes, dtypes, options
# --------------------------------------------------------------------------
@pytest.mark.parametrize("B,N,Hqk,Hv,dk,dv", [
    (3, 1, 2, 4, 64, 64),      # one node, odd batch
    (2, 5, 1, 3, 32, 64),      # d_k != d_v, GQA 3
    (1, 32, 4, 8, 128, 128),   # maximum nodes
    (5, 16, 2, 2, 128, 32),    # d_v < d_k
    (2, 7, 2, 4, 128, 256),    # d_v > d_k
    (1, 16, 1, 1, 32, 16),     # smallest d_v
])
@pytest.mark.parametrize("bf16", [True, False])
def test_chain_shapes(B, N, Hqk, Hv, dk, dv, bf16):
    w, d = small_inputs(11 + B + N + dk, B, N, Hqk, Hv, dk, dv, bf16=bf16)
    say("chain shape", (B, N, Hqk, Hv, dk, dv), "bf16", bf16)
    t = dev_inputs(d, bf16=bf16)
    out, persist, fin = run_chain(t, N)
    ref = oracle.chain(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"])
    assert max_rel(to_host(out), ref["out"]) <= OUT_TOL
    assert max_rel(to_host(fin), ref["final"]) <= STATE_TOL
    assert max_rel(to_host(persist), ref["nodes"]) <= PERSIST_TOL


@pytest.mark.parametrize("out_dtype,persist_dtype", [(torch.float16, torch.float32), (torch.bfloat16, torch.float16)])
def test_output_and_persist_dtypes(out_dtype, persist_dtype):
    w, d = small_inputs(5, 2, 16, 2, 6, 128, 128)
    t = dev_inputs(d)
    out, persist, fin = run_chain(t, 16, persist_dtype=persist_dtype, out_dtype=out_dtype, scale=128 ** -0.5)
    ref = oracle.chain(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], scale=128 ** -0.5)
    # bf16 outputs carry their own rounding (2^-9 relative); f16 2^-12
    tol = 4e-3 if out_dtype == torch.bfloat16 else OUT_TOL
    assert max_rel(to_host(out), ref["out"]) <= tol
    assert max_rel(to_host(persist), ref["nodes"]) <= (STATE_TOL if persist_dtype == torch.float32 else PERSIST_TOL)
    if persist_dtype == torch.float32:
        assert torch.equal(persist[:, -1], fin)


def test_optional_outputs_and_in_place_advance():
    w, d = small_inputs(6, 3, 16, 2, 4, 128, 128)
    t = dev_inputs(d)
    ref = oracle.chain(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"])
    # only the final state, written over the input state (a plain advance)
    state = t["state0"].clone()
    gb.gdn_verify_chain(t["q"], t["k"], t["v"], t["alpha"], t["beta"], state, final_state=state)
    torch.cuda.synchronize()
    assert max_rel(to_host(state), ref["final"]) <= STATE_TOL
    # outputs only
    out = torch.zeros(3, 16, 4, 128, device=DEV)
    gb.gdn_verify_chain(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["state0"], out=out)
    torch.cuda.synchronize()
    assert max_rel(to_host(out), ref["out"]) <= OUT_TOL


def test_state_slots():
    w, d = small_inputs(7, 4, 8, 1, 2, 64, 64)
    t = dev_inputs(d)
    n_slots = 9
    slots = np.array([7, 2, 5, 0], np.int32)
    pool = torch.randn(n_slots, 2, 64, 64, device=DEV)
    pool[torch.from_numpy(slots).long()] = t["state0"]
    slot_t = torch.from_numpy(slots).to(DEV)
    out, persist, fin = run_chain(t, 8, state=pool, state_slot=slot_t)
    ref = oracle.chain(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"])
    assert max_rel(to_host(out), ref["out"]) <= OUT_TOL
    assert max_rel(to_host(fin), ref["final"]) <= STATE_TOL
    before = pool.clone()
    acc = torch.tensor([0, 7, 3, 5], dtype=torch.int32, device=DEV)
    assert _commit(acc, persist, pool, final=fin, slot=slot_t) == 0
    for b, s in enumerate(slots):
        a = int(acc[b])
        expect = fin[b] if a == 7 else persist[b, a].float()
        assert torch.equal(pool[s], expect)
    untouched = [s for s in range(n_slots) if s not in set(slots.tolist())]
    assert torch.equal(pool[untouched], before[untouched])


def test_per_sequence_trees_cross_launch_boundary():
    rng = np.random.default_rng(77)
    B, N = 21, 22  # more sequences than one launch carries
    w, d = small_inputs(8, B, N, 2, 4, 128, 128, tree=True)
    parents = np.stack([wl.random_tree(N, 16, rng) for _ in range(B)])
    t = dev_inputs(d)
    out, persist = run_tree(t, parents, N)
    ref = oracle.tree(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], parents)
    assert max_rel(to_host(out), ref["out"]) <= OUT_TOL
    assert max_rel(to_host(persist), ref["nodes"]) <= PERSIST_TOL


@pytest.mark.parametrize("dk,dv", [(32, 64), (64, 32), (128, 128)])
def test_tree_deep_forks(dk, dv):
    """A 16-node spine with a leaf on every spine node: 15 live fork slots."""
    par = [-1]
    spine = [0]
    for _ in range(15):
        par.append(spine[-1]); spine.append(len(par) - 1)
    for s in spine[:-1]:
        par.append(s)
    par = np.array(par, np.int32)
    N = len(par)
    w, d = small_inputs(9, 2, N, 1, 2, dk, dv, tree=True)
    t = dev_inputs(d)
    out, persist = run_tree(t, par, N, persist_dtype=torch.float32)
    ref = oracle.tree(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], par)
    assert max_rel(to_host(out), ref["out"]) <= OUT_TOL
    assert max_rel(to_host(persist), ref["nodes"]) <= STATE_TOL


# --------------------------------------------------------------------------
# bit-exact properties of the GPU path
# --------------------------------------------------------------------------
def test_tree_node_equals_gpu_chain_over_its_path():
    w = wl.WORKLOADS["tree"]
    d = wl.make_inputs(w)
    t = dev_inputs(d)
    out, persist = run_tree(t, d["parent"], w.n_nodes, persist_dtype=torch.float32)
    parent = d["parent"]
    for n in range(w.n_nodes):
        path = []
        m = n
        while m >= 0:
            path.append(m); m = int(parent[m])
        path = path[::-1]
        idx = torch.tensor(path, device=DEV)
        tp = {k_: (v_[:, idx].contiguous() if k_ != "state0" else v_) for k_, v_ in t.items()}
        cout, cpersist, _ = run_chain(tp, len(path), persist_dtype=torch.float32, final=False)
        assert torch.equal(persist[:, n], cpersist[:, -1]), n
        assert torch.equal(out[:, n], cout[:, -1]), n


def test_tree_without_forks_in_two_row_groups_equals_chain():
    """A tree whose parents form a chain has no fork slot to restore, yet the tree
    kernel reads a slot every step: the launch reserves one.  At a batch large
    enough for two row groups per wave, its outputs and node states equal the chain
    kernel's bit for bit."""
    B, N = 12, 8
    w, d = small_inputs(91, B, N, 16, 48, 128, 128)
    t = dev_inputs(d)
    parent = np.arange(-1, N - 1, dtype=np.int32)
    out, persist = run_tree(t, parent, N)
    cout, cpersist, _ = run_chain(t, N, final=False)
    assert torch.equal(out, cout)
    assert torch.equal(persist, cpersist)


def test_non_ancestor_inputs_do_not_reach_a_node():
    w = wl.WORKLOADS["tree"]
    d = wl.make_inputs(w)
    t = dev_inputs(d)
    out, persist = run_tree(t, d["parent"], w.n_nodes, persist_dtype=torch.float32)
    n = w.n_nodes - 1
    anc, m = set(), n
    while m >= 0:
        anc.add(m); m = int(d["parent"][m])
    others = torch.tensor([i for i in range(w.n_nodes) if i not in anc], device=DEV)
    t2 = {k_: v_.clone() for k_, v_ in t.items()}
    t2["v"][:, others] = -t2["v"][:, others]
    t2["alpha"][:, others] *= 0.5
    t2["k"][:, others] = t2["k"][:, others].roll(1, dims=-1)
    out2, persist2 = run_tree(t2, d["parent"], w.n_nodes, persist_dtype=torch.float32)
    assert torch.equal(persist2[:, n], persist[:, n]) and torch.equal(out2[:, n], out[:, n])


def test_identity_gates_keep_state_bitwise():
    w, d = small_inputs(12, 2, 16, 2, 4, 128, 128)
    t = dev_inputs(d)
    t["alpha"].fill_(1.0)
    t["beta"].fill_(0.0)
    out, persist, fin = run_chain(t, 16, persist_dtype=torch.float32)
    assert torch.equal(fin, t["state0"])
    assert torch.equal(persist, t["state0"][:, None].expand_as(persist))
    ref = oracle.chain(d["q"], d["k"], d["v"], np.ones_like(d["alpha"]), np.zeros_like(d["beta"]), d["state0"])
    assert max_rel(to_host(out), ref["out"]) <= 1e-5


def test_zero_decay_resets_bitwise():
    w, d = small_inputs(13, 2, 16, 2, 4, 128, 128)
    t = dev_inputs(d)
    t["alpha"][:, 3] = 0.0
    out1, p1, f1 = run_chain(t, 16, persist_dtype=torch.float32)
    out2, p2, f2 = run_chain(t, 16, persist_dtype=torch.float32, state=t["state0"] * -2.5 + 0.25)
    assert torch.equal(p1[:, 3:], p2[:, 3:]) and torch.equal(f1, f2) and torch.equal(out1[:, 3:], out2[:, 3:])
    assert not torch.equal(p1[:, :3], p2[:, :3])


def test_deterministic():
    w = wl.WORKLOADS["chain"]
    d = wl.make_inputs(w, seed=5)
    t = dev_inputs(d)
    a = run_chain(t, 16)
    b = run_chain(t, 16)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# --------------------------------------------------------------------------
# device-side error handling, guard bands, streams
# --------------------------------------------------------------------------
def test_bad_slot_and_bad_node_skip_and_report():
    w, d = small_inputs(14, 3, 8, 1, 2, 64, 64)
    t = dev_inputs(d)
    out, persist, fin = alloc_outputs(t, 8)
    out.zero_(); persist.zero_(); fin.zero_()
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    slots = torch.tensor([0, 5, 2], dtype=torch.int32, device=DEV)  # 5 is outside 3 slots
    gb.gdn_verify_chain(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["state0"], out=out, persist=persist,
                        final_state=fin, state_slot=slots, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == gb.CODES["GDN_ERR_SLOT"]
    assert torch.count_nonzero(out[1]) == 0 and torch.count_nonzero(persist[1]) == 0
    assert torch.count_nonzero(out[0]) > 0 and torch.count_nonzero(out[2]) > 0
    state = t["state0"].clone()
    acc = torch.tensor([3, 8, -1], dtype=torch.int32, device=DEV)
    assert _commit(acc, persist, state, final=fin) == gb.CODES["GDN_ERR_NODE"]
    assert torch.equal(state[1], t["state0"][1]) and torch.equal(state[2], t["state0"][2])
    assert torch.equal(state[0], persist[0, 3].float())


def test_guard_bands_untouched():
    B, N, Hqk, Hv, dk, dv = 3, 22, 2, 6, 128, 128
    w, d = small_inputs(15, B, N, Hqk, Hv, dk, dv, tree=True)
    t = dev_inputs(d)
    pad = 4096

    def guarded(shape, dtype):
        n = int(np.prod(shape))
        esz = torch.tensor([], dtype=dtype).element_size()
        pe = pad // esz
        buf = torch.full((n + 2 * pe,), 1234.5, dtype=dtype, device=DEV)
        return buf, buf[pe:pe + n].view(shape), pe

    ob, out, pe_o = guarded((B, N, Hv, dv), torch.float32)
    pb, persist, pe_p = guarded((B, N, Hv, dv, dk), torch.float16)
    fb, fin, pe_f = guarded((B, Hv, dv, dk), torch.float32)
    gb.gdn_verify_chain(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["state0"], out=out, persist=persist,
                        final_state=fin)
    gb.gdn_verify_tree(d["parent"], t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["state0"], out=out,
                       persist=persist)
    sb, st, pe_s = guarded((B, Hv, dv, dk), torch.float32)
    st.copy_(t["state0"])
    gb.gdn_commit(torch.from_numpy(d["accepted"]).to(DEV), persist, st)
    torch.cuda.synchronize()
    for buf, pe in ((ob, pe_o), (pb, pe_p), (fb, pe_f), (sb, pe_s)):
        assert bool((buf[:pe] == 1234.5).all()) and bool((buf[-pe:] == 1234.5).all())


def test_runs_on_a_side_stream():
    w, d = small_inputs(16, 2, 16, 2, 4, 128, 128)
    t = dev_inputs(d)
    ref_out, ref_p, ref_f = run_chain(t, 16)
    s = torch.cuda.Stream()
    out, persist, fin = alloc_outputs(t, 16)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        gb.gdn_verify_chain(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["state0"], out=out, persist=persist,
                            final_state=fin)
    s.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(persist, ref_p) and torch.equal(fin, ref_f)


# --------------------------------------------------------------------------
# fused commit + verify (one launch per decode step)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("persist_dtype", [torch.float16, torch.float32])
@pytest.mark.parametrize("same_buffers", [False, True])
def test_fused_commit_verify_equals_commit_then_verify(persist_dtype, same_buffers):
    w, d1 = small_inputs(21, 3, 16, 2, 6, 128, 128)
    _, d2 = small_inputs(22, 3, 16, 2, 6, 128, 128)
    t1, t2 = dev_inputs(d1), dev_inputs(d2)
    out1, per1, fin1 = run_chain(t1, 16, persist_dtype=persist_dtype)
    acc = torch.tensor([3, 15, 0], dtype=torch.int32, device=DEV)
    st_ref = t1["state0"].clone()
    assert _commit(acc, per1, st_ref, final=fin1) == 0
    out_r, per_r, fin_r = run_chain(t2, 16, persist_dtype=persist_dtype, state=st_ref)
    st = t1["state0"].clone()
    if same_buffers:  # the step writes over the very buffers it commits from
        out, per, fin = out1.clone(), per1.clone(), fin1.clone()
        per_prev, fin_prev = per, fin
    else:
        out, per, fin = alloc_outputs(t2, 16, persist_dtype)
        per_prev, fin_prev = per1, fin1
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    gb.gdn_commit_verify_chain(acc, per_prev, t2["q"], t2["k"], t2["v"], t2["alpha"], t2["beta"], st,
                               final_prev=fin_prev, out=out, persist=per, final_state=fin, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(st, st_ref)
    assert torch.equal(out, out_r) and torch.equal(per, per_r) and torch.equal(fin, fin_r)


@pytest.mark.parametrize("persist_dtype", [torch.float16, torch.float32])
def test_fused_commit_verify_through_state_slots(persist_dtype):
    """The fused step on a state pool addressed through slots equals commit then verify on the same pool;
    slots no sequence names keep their contents."""
    B, N, n_slots = 5, 16, 11
    w, d1 = small_inputs(41, B, N, 2, 6, 128, 128)
    _, d2 = small_inputs(42, B, N, 2, 6, 128, 128)
    t1, t2 = dev_inputs(d1), dev_inputs(d2)
    slots = torch.tensor([9, 0, 4, 10, 2], dtype=torch.int32, device=DEV)
    pool0 = torch.randn(n_slots, 6, 128, 128, device=DEV)
    pool0[slots.long()] = t1["state0"]
    out1, per1, fin1 = run_chain(t1, N, persist_dtype=persist_dtype, state=pool0, state_slot=slots)
    acc = torch.tensor([15, 0, 7, 3, 15], dtype=torch.int32, device=DEV)
    pool_ref = pool0.clone()
    assert _commit(acc, per1, pool_ref, final=fin1, slot=slots) == 0
    out_r, per_r, fin_r = run_chain(t2, N, persist_dtype=persist_dtype, state=pool_ref, state_slot=slots)
    pool = pool0.clone()
    out, per, fin = alloc_outputs(t2, N, persist_dtype)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    gb.gdn_commit_verify_chain(acc, per1, t2["q"], t2["k"], t2["v"], t2["alpha"], t2["beta"], pool,
                               final_prev=fin1, out=out, persist=per, final_state=fin, state_slot=slots,
                               status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(pool, pool_ref)
    untouched = [s for s in range(n_slots) if s not in set(slots.tolist())]
    assert torch.equal(pool[untouched], pool0[untouched])
    assert torch.equal(out, out_r) and torch.equal(per, per_r) and torch.equal(fin, fin_r)


def test_fused_decode_loop_matches_oracle():
    """Three fused steps (accepted lengths 5, 16, 1) against the oracle applied step by step."""
    B, N = 2, 16
    steps = [small_inputs(31 + i, B, N, 2, 4, 128, 128)[1] for i in range(3)]
    accs = [np.array([4, 9], np.int32), np.array([15, 15], np.int32), np.array([0, 7], np.int32)]
    st = dev_inputs(steps[0])["state0"].clone()
    ref_state = steps[0]["state0"].astype(np.float64)
    per_prev = fin_prev = acc_prev = None
    for i, d in enumerate(steps):
        t = dev_inputs(d)
        out, per, fin = alloc_outputs(t, N)
        if i == 0:
            gb.gdn_verify_chain(t["q"], t["k"], t["v"], t["alpha"], t["beta"], st, out=out, persist=per,
                                final_state=fin)
        else:
            gb.gdn_commit_verify_chain(acc_prev, per_prev, t["q"], t["k"], t["v"], t["alpha"], t["beta"], st,
                                       final_prev=fin_prev, out=out, persist=per, final_state=fin)
        torch.cuda.synchronize()
        ref = oracle.chain(d["q"], d["k"], d["v"], d["alpha"], d["beta"], ref_state)
        assert max_rel(to_host(out), ref["out"]) <= OUT_TOL
        assert max_rel(to_host(per), ref["nodes"]) <= PERSIST_TOL
        ref_state, _ = oracle.commit(ref_state, ref["nodes"], accs[i], final=ref["final"])
        # the committed state the next step reads comes from the f16 copy unless fully accepted
        acc_prev = torch.from_numpy(accs[i]).to(DEV)
        per_prev, fin_prev = per, fin
    assert _commit(acc_prev, per_prev, st, final=fin_prev) == 0
    assert max_rel(to_host(st), ref_state) <= STATE_TOL


# --------------------------------------------------------------------------
# fused commit + tree verify (one launch per tree decode step)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("persist_dtype", [torch.float16, torch.float32])
@pytest.mark.parametrize("same_buffers", [False, True])
def test_fused_commit_verify_tree_equals_commit_then_verify(persist_dtype, same_buffers):
    """The fused tree step equals gdn_commit followed by gdn_verify_tree, bit for bit, also when it
    writes over the node states it commits from."""
    rng = np.random.default_rng(61)
    B, N = 3, 22
    _, d1 = small_inputs(61, B, N, 2, 6, 128, 128, tree=True)
    _, d2 = small_inputs(62, B, N, 2, 6, 128, 128, tree=True)
    p1, p2 = wl.random_tree(N, 16, rng), wl.random_tree(N, 16, rng)
    t1, t2 = dev_inputs(d1), dev_inputs(d2)
    out1, per1 = run_tree(t1, p1, N, persist_dtype=persist_dtype)
    acc = torch.tensor([21, 0, 9], dtype=torch.int32, device=DEV)
    st_ref = t1["state0"].clone()
    assert _commit(acc, per1, st_ref) == 0
    out_r, per_r = run_tree({**t2, "state0": st_ref}, p2, N, persist_dtype=persist_dtype)
    st = t1["state0"].clone()
    if same_buffers:
        out, per = out1.clone(), per1.clone()
        per_prev = per
    else:
        out, per, _ = alloc_outputs(t2, N, persist_dtype, final=False)
        per_prev = per1
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    gb.gdn_commit_verify_tree(acc, per_prev, p2, t2["q"], t2["k"], t2["v"], t2["alpha"], t2["beta"], st,
                              out=out, persist=per, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(st, st_ref)
    assert torch.equal(out, out_r) and torch.equal(per, per_r)


def test_fused_commit_verify_per_sequence_trees_through_slots():
    """One tree per sequence, more sequences than one launch carries, states in a slot pool."""
    rng = np.random.default_rng(63)
    B, N, n_slots = 21, 12, 25
    _, d1 = small_inputs(63, B, N, 1, 2, 64, 64, tree=True)
    _, d2 = small_inputs(64, B, N, 1, 2, 64, 64, tree=True)
    t1, t2 = dev_inputs(d1), dev_inputs(d2)
    par1 = np.stack([wl.random_tree(N, 8, rng) for _ in range(B)])
    par2 = np.stack([wl.random_tree(N, 8, rng) for _ in range(B)])
    slots = torch.from_numpy(rng.permutation(n_slots)[:B].astype(np.int32)).to(DEV)
    pool0 = torch.randn(n_slots, 2, 64, 64, device=DEV)
    pool0[slots.long()] = t1["state0"]
    _, per1 = run_tree({**t1, "state0": pool0}, par1, N, state_slot=slots)
    acc = torch.from_numpy(rng.integers(0, N, B).astype(np.int32)).to(DEV)
    pool_ref = pool0.clone()
    assert _commit(acc, per1, pool_ref, slot=slots) == 0
    out_r, per_r = run_tree({**t2, "state0": pool_ref}, par2, N, state_slot=slots)
    pool = pool0.clone()
    out, per, _ = alloc_outputs(t2, N, final=False)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    gb.gdn_commit_verify_tree(acc, per1, par2, t2["q"], t2["k"], t2["v"], t2["alpha"], t2["beta"], pool,
                              out=out, persist=per, state_slot=slots, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(pool, pool_ref)
    assert torch.equal(out, out_r) and torch.equal(per, per_r)


@pytest.mark.parametrize("out_dtype,persist", [(torch.bfloat16, True), (torch.float16, True), (torch.float32, False)])
def test_fused_tree_output_dtypes_and_no_persist(out_dtype, persist):
    """The fused tree step with bf16 / f16 outputs, or persisting nothing, equals commit then tree verify
    with the same options bit for bit."""
    rng = np.random.default_rng(69)
    B, N = 2, 16
    _, d1 = small_inputs(69, B, N, 2, 4, 64, 64, tree=True)
    _, d2 = small_inputs(70, B, N, 2, 4, 64, 64, tree=True)
    t1, t2 = dev_inputs(d1), dev_inputs(d2)
    p1, p2 = wl.random_tree(N, 8, rng), wl.random_tree(N, 8, rng)
    _, per1 = run_tree(t1, p1, N)
    acc = torch.tensor([11, 4], dtype=torch.int32, device=DEV)
    st_ref = t1["state0"].clone()
    assert _commit(acc, per1, st_ref) == 0
    pdt = torch.float16 if persist else None
    out_r, per_r = run_tree({**t2, "state0": st_ref}, p2, N, persist_dtype=pdt, out_dtype=out_dtype)
    st = t1["state0"].clone()
    out, per, _ = alloc_outputs(t2, N, pdt, out_dtype, final=False)
    gb.gdn_commit_verify_tree(acc, per1, p2, t2["q"], t2["k"], t2["v"], t2["alpha"], t2["beta"], st, out=out,
                              persist=per)
    torch.cuda.synchronize()
    assert torch.equal(st, st_ref) and torch.equal(out, out_r)
    if persist:
        assert torch.equal(per, per_r)


def test_fused_fork_free_tree_in_two_row_groups_equals_fused_chain():
    """A tree with no forks at a batch large enough for two row groups per wave: the fused tree step equals
    the fused chain step bit for bit (node states, outputs and the committed state)."""
    B, N = 12, 8
    _, d1 = small_inputs(71, B, N, 16, 48, 128, 128)
    _, d2 = small_inputs(72, B, N, 16, 48, 128, 128)
    t1, t2 = dev_inputs(d1), dev_inputs(d2)
    chain_par = np.arange(-1, N - 1, dtype=np.int32)
    _, per1, fin1 = run_chain(t1, N)
    acc = torch.tensor([0, 3, 6, 2, 5, 1, 4, 6, 0, 2, 3, 5], dtype=torch.int32, device=DEV)  # never N - 1
    st_c, st_t = t1["state0"].clone(), t1["state0"].clone()
    out_c, per_c, fin_c = alloc_outputs(t2, N)
    out_t, per_t, _ = alloc_outputs(t2, N, final=False)
    gb.gdn_commit_verify_chain(acc, per1, t2["q"], t2["k"], t2["v"], t2["alpha"], t2["beta"], st_c,
                               final_prev=fin1, out=out_c, persist=per_c, final_state=fin_c)
    gb.gdn_commit_verify_tree(acc, per1, chain_par, t2["q"], t2["k"], t2["v"], t2["alpha"], t2["beta"], st_t,
                              out=out_t, persist=per_t)
    torch.cuda.synchronize()
    assert torch.equal(st_t, st_c)
    assert torch.equal(out_t, out_c) and torch.equal(per_t, per_c)


def test_fused_tree_plain_store_launches_equal_commit_then_verify():
    """Per-sequence trees writing more than 256 MB of node states (plain stores, several launches of
    sixteen trees): the fused step equals commit then tree verify bit for bit."""
    rng = np.random.default_rng(73)
    B, N = 40, 12
    _, d1 = small_inputs(73, B, N, 16, 48, 128, 128, tree=True)
    _, d2 = small_inputs(74, B, N, 16, 48, 128, 128, tree=True)
    t1, t2 = dev_inputs(d1), dev_inputs(d2)
    par1 = np.stack([wl.random_tree(N, 6, rng) for _ in range(B)])
    par2 = np.stack([wl.random_tree(N, 6, rng) for _ in range(B)])
    _, per1 = run_tree(t1, par1, N)
    assert per1.numel() * 2 >= 256 << 20
    acc = torch.from_numpy(rng.integers(0, N, B).astype(np.int32)).to(DEV)
    st_ref = t1["state0"].clone()
    assert _commit(acc, per1, st_ref) == 0
    out_r, per_r = run_tree({**t2, "state0": st_ref}, par2, N)
    st = t1["state0"].clone()
    out, per, _ = alloc_outputs(t2, N, final=False)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    gb.gdn_commit_verify_tree(acc, per1, par2, t2["q"], t2["k"], t2["v"], t2["alpha"], t2["beta"], st,
                              out=out, persist=per, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(st, st_ref)
    assert torch.equal(out, out_r) and torch.equal(per, per_r)


def test_fused_tree_decode_loop_matches_oracle():
    """Three tree steps, the second and third fused with the commit of the step before, against the
    oracle applied step by step (commit of the accepted node's exact state)."""
    rng = np.random.default_rng(65)
    B, N = 2, 22
    steps = [small_inputs(65 + i, B, N, 2, 4, 128, 128, tree=True)[1] for i in range(3)]
    pars = [wl.random_tree(N, 16, rng) for _ in range(3)]
    accs = [np.array([5, 21], np.int32), np.array([0, 13], np.int32), np.array([17, 2], np.int32)]
    st = dev_inputs(steps[0])["state0"].clone()
    ref_state = steps[0]["state0"].astype(np.float64)
    per_prev = acc_prev = None
    for i, d in enumerate(steps):
        t = dev_inputs(d)
        out, per, _ = alloc_outputs(t, N, final=False)
        if i == 0:
            gb.gdn_verify_tree(pars[0], t["q"], t["k"], t["v"], t["alpha"], t["beta"], st, out=out, persist=per)
        else:
            gb.gdn_commit_verify_tree(acc_prev, per_prev, pars[i], t["q"], t["k"], t["v"], t["alpha"],
                                      t["beta"], st, out=out, persist=per)
        torch.cuda.synchronize()
        ref = oracle.tree(d["q"], d["k"], d["v"], d["alpha"], d["beta"], ref_state, pars[i])
        e = (max_rel(to_host(out), ref["out"]), max_rel(to_host(per), ref["nodes"]))
        say(f"tree step {i}: out {e[0]:.2e} node states {e[1]:.2e}")
        assert e[0] <= OUT_TOL and e[1] <= PERSIST_TOL
        ref_state, _ = oracle.commit(ref_state, ref["nodes"], accs[i])
        acc_prev = torch.from_numpy(accs[i]).to(DEV)
        per_prev = per
    assert _commit(acc_prev, per_prev, st) == 0
    assert max_rel(to_host(st), ref_state) <= STATE_TOL


def test_fused_tree_bad_accepted_node_skips_sequence():
    rng = np.random.default_rng(67)
    w, d = small_inputs(67, 3, 8, 1, 2, 64, 64, tree=True)
    t = dev_inputs(d)
    par = wl.random_tree(8, 4, rng)
    _, per1 = run_tree(t, par, 8)
    st = t["state0"].clone()
    out, per, _ = alloc_outputs(t, 8, final=False)
    out.zero_(); per.zero_()
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    acc = torch.tensor([2, -1, 7], dtype=torch.int32, device=DEV)
    gb.gdn_commit_verify_tree(acc, per1, par, t["q"], t["k"], t["v"], t["alpha"], t["beta"], st, out=out,
                              persist=per, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == gb.CODES["GDN_ERR_NODE"]
    assert torch.equal(st[1], t["state0"][1]) and torch.count_nonzero(per[1]) == 0
    assert torch.count_nonzero(out[1]) == 0
    assert torch.equal(st[0], per1[0, 2].float()) and torch.equal(st[2], per1[2, 7].float())


def test_fused_bad_accepted_node_skips_sequence():
    w, d = small_inputs(41, 3, 8, 1, 2, 64, 64)
    t = dev_inputs(d)
    out1, per1, fin1 = run_chain(t, 8)
    st = t["state0"].clone()
    out, per, fin = alloc_outputs(t, 8)
    out.zero_(); per.zero_(); fin.zero_()
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    acc = torch.tensor([2, 8, 5], dtype=torch.int32, device=DEV)
    gb.gdn_commit_verify_chain(acc, per1, t["q"], t["k"], t["v"], t["alpha"], t["beta"], st, final_prev=fin1,
                               out=out, persist=per, final_state=fin, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == gb.CODES["GDN_ERR_NODE"]
    assert torch.equal(st[1], t["state0"][1]) and torch.count_nonzero(per[1]) == 0
    assert torch.equal(st[0], per1[0, 2].float()) and torch.equal(st[2], per1[2, 5].float())


def test_f16_persist_is_the_fp32_node_state_rounded():
    """Each persisted f16 node state is the kernel's fp32 node state rounded once
    to nearest even (bit for bit), for chains and trees."""
    w, d = small_inputs(151, 2, 16, 2, 6, 128, 128, tree=True)
    t = dev_inputs(d)
    _, p16, f16fin = run_chain(t, 16, persist_dtype=torch.float16)
    _, p32, _ = run_chain(t, 16, persist_dtype=torch.float32)
    assert torch.equal(p16, p32.to(torch.float16))
    _, q16 = run_tree(t, d["parent"], 16, persist_dtype=torch.float16)
    _, q32 = run_tree(t, d["parent"], 16, persist_dtype=torch.float32)
    assert torch.equal(q16, q32.to(torch.float16))
