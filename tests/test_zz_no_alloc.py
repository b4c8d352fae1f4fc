"""The chunked prefill that allocates nothing (gdn_prefill_chunked_noalloc)
against gdn_prefill_chunked through the C ABI, on calls in a row, each smaller
than the one before: results bit for bit equal (and the smallest against the
fp64 oracle at the parity bar)."""
import pytest
import torch

import oracle
from gated_deltanet_recurrence_gdn_amd import binding as gb
from gated_deltanet_recurrence_gdn_amd import workloads as wl
from helpers import DEV, OUT_TOL, STATE_TOL, dev_inputs, max_rel, say, to_host

pytestmark = pytest.mark.gpu


def run(fn, t, **kw):
    B, T, _, _ = t["q"].shape
    Hv, dv = t["v"].shape[2], t["v"].shape[3]
    st = t["state0"].clone()
    out = torch.full((B, T, Hv, dv), float("nan"), device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    fn(t["q"], t["k"], t["v"], t["alpha"], t["beta"], st, out, status=status, **kw)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return out, st


def test_noalloc_equals_chunked_on_calls_in_a_row():
    cases = [
        # the 4096-token prompt at 16 / 48 heads: three segments of the 32 MiB array
        wl.WORKLOADS["prefill"],
        # three sequences: eight chunks of each per segment, a ragged last chunk
        wl.Workload("custom", 3, 1000, 16, 48, 128, 128),
        # small heads: one segment
        wl.Workload("custom", 2, 300, 2, 6, 64, 64),
    ]
    for i, w in enumerate(cases):
        d = wl.make_inputs(w, seed=900 + i)
        t = dev_inputs(d)
        say("no-alloc prefill call", i, w)
        ref_out, ref_st = run(gb.gdn_prefill_chunked, t)
        out, st = run(gb.gdn_prefill_chunked_noalloc, t)
        assert torch.equal(out, ref_out) and torch.equal(st, ref_st)
    ref = oracle.chain(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], nodes=False)
    assert max_rel(to_host(out), ref["out"]) <= OUT_TOL
    assert max_rel(to_host(st), ref["final"]) <= STATE_TOL


def test_noalloc_rejects_heads_beyond_the_array():
    """One 64-token chunk of 2048 value heads needs more than the array holds:
    refused on the host, nothing enqueued, the state untouched."""
    q = torch.zeros(1, 64, 16, 128, dtype=torch.bfloat16, device=DEV)
    v = torch.zeros(1, 64, 2048, 32, dtype=torch.bfloat16, device=DEV)
    g = torch.ones(1, 64, 2048, device=DEV)
    st = torch.full((1, 2048, 32, 128), 3.0, device=DEV)
    out = torch.zeros(1, 64, 2048, 32, device=DEV)
    with pytest.raises(gb.GdnError) as ei:
        gb.gdn_prefill_chunked_noalloc(q, q, v, g, g, st, out)
    assert ei.value.code == gb.CODES["GDN_ERR_WORKSPACE"]
    torch.cuda.synchronize()
    assert bool((st == 3.0).all())


@pytest.mark.parametrize("w", [wl.Workload("custom", 2, 300, 2, 6, 64, 64),       # one prepare + scan pair
                               wl.Workload("custom", 3, 1000, 16, 48, 128, 128)],  # segments of the array
                         ids=["one-launch-pair", "segments"])
def test_noalloc_prefill_replays_from_a_hip_graph(w):
    """What the entry point is for: a call that allocates nothing can be
    captured in a HIP graph.  Captured once (after an eager call), then
    replayed three times with eager work and synchronizations between the
    replays; every replay equals the eager call bit for bit (the state and the
    outputs are reset before each replay, outside the graph)."""
    d = wl.make_inputs(w, seed=950)
    t = dev_inputs(d)
    B, T, _, _ = t["q"].shape
    Hv, dv = t["v"].shape[2], t["v"].shape[3]
    st = t["state0"].clone()
    out = torch.zeros(B, T, Hv, dv, device=DEV)
    args = (t["q"], t["k"], t["v"], t["alpha"], t["beta"], st, out)
    gb.gdn_prefill_chunked_noalloc(*args)
    torch.cuda.synchronize()
    ref_out, ref_st = out.clone(), st.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        gb.gdn_prefill_chunked_noalloc(*args)
    torch.cuda.synchronize()
    for i in range(3):
        st.copy_(t["state0"])
        out.zero_()
        busy = torch.randn(1 << 20, device=DEV)
        busy.mul_(2.0).sum().item()  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say("graph replay", i)
        assert torch.equal(out, ref_out) and torch.equal(st, ref_st), i
