"""GPU parity of the index-table commit (gdn_commit_index) and of the decode
loop it serves: verify persists fp32 node states into the pool's draft rows
through the index table, the commit points the table at the accepted row, and
the next verify reads the exact fp32 state from there."""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_recurrence_gdn_amd import binding as gb
from helpers import DEV, OUT_TOL, STATE_TOL, dev_inputs, max_rel, run_chain, say, small_inputs, to_host

pytestmark = pytest.mark.gpu


def test_commit_index_definition_and_rejections():
    B, N, row0, n_slots = 300, 7, 5, 5 + 300 * 7
    rng = np.random.default_rng(130)
    acc = rng.integers(0, N, size=B).astype(np.int32)
    acc[3], acc[299] = N, -1
    slot0 = rng.integers(0, 5, size=B).astype(np.int32)
    slot = torch.from_numpy(slot0).to(DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    gb.gdn_commit_index(torch.from_numpy(acc).to(DEV), slot, N, row0, n_slots, status=status)
    torch.cuda.synchronize()
    ref, bad = oracle.commit_index(slot0, acc, row0, N, n_slots)
    assert bad == 2 and int(status.item()) == gb.CODES["GDN_ERR_NODE"]
    assert np.array_equal(slot.cpu().numpy(), ref)


@pytest.mark.parametrize("tree", [False, True])
def test_index_commit_decode_loop(tree):
    """Three decode steps: verify through the index table with fp32 persist into
    the pool's draft rows, then an index commit; outputs and the state the
    table points at match the oracle applied step by step, and the state each
    step starts from is the previous accepted node's exact fp32 state."""
    B, N, Hqk, Hv, dk, dv = 3, 12, 2, 4, 128, 64
    canon = B  # rows 0 .. B-1 hold the initial states
    row0, n_slots = canon, canon + B * N
    steps = [small_inputs(140 + i, B, N, Hqk, Hv, dk, dv, tree=tree)[1] for i in range(3)]
    pool = torch.full((n_slots, Hv, dv, dk), float("nan"), device=DEV)
    pool[:B] = dev_inputs(steps[0])["state0"]
    slot = torch.arange(B, dtype=torch.int32, device=DEV)
    ref_state = steps[0]["state0"].astype(np.float64)
    persist = pool[row0:].view(B, N, Hv, dv, dk)
    for i, d in enumerate(steps):
        t = dev_inputs(d)
        start = pool[slot.long()].clone()
        out = torch.empty(B, N, Hv, dv, device=DEV)
        if tree:
            gb.gdn_verify_tree(d["parent"], t["q"], t["k"], t["v"], t["alpha"], t["beta"], pool, out=out,
                               persist=persist, state_slot=slot)
            ref = oracle.tree(d["q"], d["k"], d["v"], d["alpha"], d["beta"], ref_state, d["parent"])
        else:
            gb.gdn_verify_chain(t["q"], t["k"], t["v"], t["alpha"], t["beta"], pool, out=out, persist=persist,
                                state_slot=slot)
            ref = oracle.chain(d["q"], d["k"], d["v"], d["alpha"], d["beta"], ref_state)
        torch.cuda.synchronize()
        e = max_rel(to_host(out), ref["out"])
        say(f"index loop {'tree' if tree else 'chain'} step {i}: out max-rel {e:.2e}")
        assert e <= OUT_TOL
        assert max_rel(to_host(persist), ref["nodes"]) <= STATE_TOL
        # the persisted rows are the verify's exact node states (same run, fp32 persist, no index table)
        if not tree:
            _, per_ref, _ = run_chain(t, N, persist_dtype=torch.float32, state=start)
            assert torch.equal(persist, per_ref)
        acc = d["accepted"]
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        gb.gdn_commit_index(torch.from_numpy(acc).to(DEV), slot, N, row0, n_slots, status=status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert np.array_equal(slot.cpu().numpy(), row0 + np.arange(B) * N + acc)
        ref_state = ref["nodes"][np.arange(B), acc]
        assert max_rel(to_host(pool[slot.long()]), ref_state) <= STATE_TOL
