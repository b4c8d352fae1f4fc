"""GPU parity of the chunked prefill against the stepwise fp64 oracle,
through the C ABI.  Bar: max relative error <= 2e-3 on outputs and on the
final fp32 state."""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_recurrence_gdn_amd import binding as gb
from gated_deltanet_recurrence_gdn_amd import workloads as wl
from helpers import DEV, OUT_TOL, STATE_TOL, dev_inputs, max_rel, say, to_host

pytestmark = pytest.mark.gpu


def run_prefill(t, out_dtype=torch.float32, scale=1.0, state=None, **kw):
    B, T, _, _ = t["q"].shape
    Hv, dv = t["v"].shape[2], t["v"].shape[3]
    st = (t["state0"] if state is None else state).clone()
    out = torch.full((B, T, Hv, dv), float("nan"), dtype=out_dtype, device=DEV)
    gb.gdn_prefill_chunked(t["q"], t["k"], t["v"], t["alpha"], t["beta"], st, out, scale=scale, **kw)
    torch.cuda.synchronize()
    return out, st


def sub_inputs(d, heads, G):
    """Inputs restricted to value heads `heads` (consecutive group members kept with their q/k head)."""
    qk = sorted({h // G for h in heads})
    hv = [h for h in heads]
    e = {}
    for n in ("q", "k"):
        e[n] = d[n][:, :, qk]
    e["v"] = d["v"][:, :, hv]
    for n in ("alpha", "beta"):
        e[n] = d[n][:, :, hv]
    e["state0"] = d["state0"][:, hv]
    return e


def test_prefill_full_size_all_heads():
    """The 4096-token prompt at 16 q/k and 48 value heads, d = 128: every output
    and the final state of every head against the stepwise fp64 recurrence
    (one multi-threaded oracle call over the 48 heads)."""
    w = wl.WORKLOADS["prefill"]
    d = wl.make_inputs(w)
    say("prefill", w)
    t = dev_inputs(d)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, st = run_prefill(t, status=status)
    assert int(status.item()) == 0
    ref = oracle.chain(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], nodes=False)
    eo, ef = max_rel(to_host(out), ref["out"]), max_rel(to_host(st), ref["final"])
    per_head = [max_rel(to_host(out[:, :, h]), ref["out"][:, :, h]) for h in range(w.h_v)]
    say(f"all 48 heads: out {eo:.2e} final {ef:.2e}; worst head out {max(per_head):.2e}")
    assert eo <= OUT_TOL and ef <= STATE_TOL


@pytest.mark.parametrize("B,T,Hqk,Hv,dk,dv", [
    (1, 1, 1, 1, 128, 32),
    (1, 63, 1, 2, 128, 64),
    (2, 64, 2, 4, 128, 128),
    (1, 65, 1, 1, 64, 32),
    (3, 200, 1, 3, 32, 64),
    (1, 130, 2, 2, 64, 96),
    (1, 300, 1, 1, 128, 256),
    (2, 300, 16, 48, 128, 128),  # more scan workgroups than CUs: two per CU where they fit
    (3, 150, 16, 48, 64, 64),     # the same at d_k = 64 (288 scan workgroups)
])
@pytest.mark.parametrize("bf16", [True, False])
def test_prefill_shapes_and_ragged_tails(B, T, Hqk, Hv, dk, dv, bf16):
    w = wl.Workload("custom", B, T, Hqk, Hv, dk, dv, qkv_bf16=bf16)
    d = wl.make_inputs(w, seed=T + dk + dv)
    say("prefill shape", (B, T, Hqk, Hv, dk, dv), "bf16", bf16)
    t = dev_inputs(d, bf16=bf16)
    out, st = run_prefill(t)
    ref = oracle.chain(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], nodes=False)
    assert max_rel(to_host(out), ref["out"]) <= OUT_TOL
    assert max_rel(to_host(st), ref["final"]) <= STATE_TOL


@pytest.mark.parametrize("alpha_lo,T", [(0.99, 1024), (1.0, 1000)])
def test_prefill_slow_decay_carries_state_across_chunks(alpha_lo, T):
    """Gates near or at 1: the state entering a chunk is not damped away within
    it, so every chunk's output and the final state depend on all earlier
    chunks (the workload's gates decay by about half per token)."""
    w = wl.Workload("custom", 1, T, 2, 4, 128, 128)
    d = wl.make_inputs(w, seed=11)
    rng = np.random.default_rng(5)
    d["alpha"] = (alpha_lo + (1.0 - alpha_lo) * rng.random(d["alpha"].shape)).astype(np.float32)
    d["beta"] = rng.random(d["beta"].shape).astype(np.float32)
    t = dev_inputs(d)
    out, st = run_prefill(t)
    ref = oracle.chain(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], nodes=False)
    eo, es = max_rel(to_host(out), ref["out"]), max_rel(to_host(st), ref["final"])
    say(f"slow decay alpha >= {alpha_lo}, T={T}: out {eo:.2e} state {es:.2e}")
    assert eo <= OUT_TOL and es <= STATE_TOL


def test_prefill_resume_equals_one_pass():
    w = wl.Workload("custom", 1, 257, 2, 4, 128, 64)
    d = wl.make_inputs(w, seed=3)
    t = dev_inputs(d)
    whole_out, whole_st = run_prefill(t)
    t1 = 100  # not a chunk multiple
    a = {n: (x[:, :t1].contiguous() if n != "state0" else x) for n, x in t.items()}
    o1, s1 = run_prefill(a)
    b = {n: (x[:, t1:].contiguous() if n != "state0" else x) for n, x in t.items()}
    o2, s2 = run_prefill(b, state=s1)
    ref = oracle.chain(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], nodes=False)
    assert max_rel(to_host(torch.cat([o1, o2], dim=1)), ref["out"]) <= OUT_TOL
    assert max_rel(to_host(s2), ref["final"]) <= STATE_TOL
    assert max_rel(to_host(s2), to_host(whole_st)) <= STATE_TOL


def test_prefill_f16_output_scale_and_zero_gates():
    w = wl.Workload("custom", 1, 192, 2, 6, 128, 128)
    d = wl.make_inputs(w, seed=4)
    d["alpha"][:, 70] = 0.0   # a reset inside a chunk
    d["alpha"][:, 128] = 0.0  # a reset at a chunk start
    d["beta"][:, 5:9] = 0.0
    t = dev_inputs(d)
    sc = 128 ** -0.5
    out, st = run_prefill(t, out_dtype=torch.float16, scale=sc)
    ref = oracle.chain(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], scale=sc, nodes=False)
    assert max_rel(to_host(out), ref["out"]) <= OUT_TOL
    assert max_rel(to_host(st), ref["final"]) <= STATE_TOL


def test_prefill_state_slots_and_guard_bands():
    w = wl.Workload("custom", 3, 100, 1, 2, 64, 64)
    d = wl.make_inputs(w, seed=5)
    t = dev_inputs(d)
    slots = torch.tensor([4, 0, 2], dtype=torch.int32, device=DEV)
    pool = torch.randn(6, 2, 64, 64, device=DEV)
    pool[slots.long()] = t["state0"]
    before = pool.clone()
    pad = 1024
    buf = torch.full((3 * 100 * 2 * 64 + 2 * pad,), 7.25, device=DEV)
    out = buf[pad:pad + 3 * 100 * 2 * 64].view(3, 100, 2, 64)
    gb.gdn_prefill_chunked(t["q"], t["k"], t["v"], t["alpha"], t["beta"], pool, out, state_slot=slots)
    torch.cuda.synchronize()
    ref = oracle.chain(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], nodes=False)
    assert max_rel(to_host(out), ref["out"]) <= OUT_TOL
    assert max_rel(to_host(pool[slots.long()]), ref["final"]) <= STATE_TOL
    assert torch.equal(pool[[1, 3, 5]], before[[1, 3, 5]])
    assert bool((buf[:pad] == 7.25).all()) and bool((buf[-pad:] == 7.25).all())


def test_prefill_bad_slot_reports_and_skips():
    w = wl.Workload("custom", 2, 70, 1, 1, 32, 32)
    d = wl.make_inputs(w, seed=6)
    t = dev_inputs(d)
    st = t["state0"].clone()
    out = torch.zeros(2, 70, 1, 32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    gb.gdn_prefill_chunked(t["q"], t["k"], t["v"], t["alpha"], t["beta"], st, out,
                           state_slot=torch.tensor([1, 9], dtype=torch.int32, device=DEV), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == gb.CODES["GDN_ERR_SLOT"]
    assert torch.count_nonzero(out[1]) == 0 and torch.equal(st[0], t["state0"][0])


def test_prefill_deterministic_and_workspace():
    w = wl.Workload("custom", 1, 128, 1, 3, 128, 128)
    d = wl.make_inputs(w, seed=7)
    t = dev_inputs(d)
    a = run_prefill(t)
    b = run_prefill(t)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    need = gb.gdn_prefill_workspace_bytes(t["q"], t["v"], t["state0"], a[0])
    # 2 chunks x (3 heads x (T', P) f16 + 3 heads x gates + 1 q/k head x (K, Q) f16)
    assert need == 2 * (3 * 2 * 64 * 64 * 2 + 3 * 3 * 64 * 4 + 2 * 128 * 64 * 2)
    # a caller-provided workspace with stale contents gives the same result
    ws = torch.full((need,), 255, dtype=torch.uint8, device=DEV)
    c = run_prefill(t, workspace=ws)
    assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1])
    with pytest.raises(gb.GdnError) as ei:
        run_prefill(t, workspace=ws[:need - 16])
    assert ei.value.code == gb.CODES["GDN_ERR_WORKSPACE"]


@pytest.mark.parametrize("out_dtype", [torch.float16, torch.bfloat16])
def test_prefill_two_block_scan_with_narrow_outputs(out_dtype):
    """More scan workgroups than CUs (the two-LDS-block scan) with f16 and bf16
    outputs; bf16 outputs alone cost about 1.5e-3 of rounding, so their bar is
    the bf16 rounding of the reference plus the usual budget."""
    w = wl.Workload("custom", 2, 200, 16, 48, 128, 128)
    d = wl.make_inputs(w, seed=21)
    t = dev_inputs(d)
    out, st = run_prefill(t, out_dtype=out_dtype)
    ref = oracle.chain(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["state0"], nodes=False)
    tol = OUT_TOL if out_dtype == torch.float16 else OUT_TOL + 2.0 ** -8
    assert max_rel(to_host(out), ref["out"]) <= tol
    assert max_rel(to_host(st), ref["final"]) <= STATE_TOL


@pytest.mark.parametrize("where", ["q", "k", "v", "state0", "none"])
def test_prefill_reports_values_outside_the_f16_range(where):
    """A q or k element beyond the f16 range is reported by the prepare kernel;
    a v element or an initial state beyond it makes the state non-finite, which
    the scan reports.  In-range inputs report nothing."""
    w = wl.Workload("custom", 1, 150, 1, 2, 64, 32)
    d = wl.make_inputs(w, seed=31)
    if where in ("q", "k", "v"):
        big = wl.round_bf16(np.array([1.0e5], np.float32))[0]
        d[where][0, 77, 0, 5] = big
        d[where + "_bits"] = wl.bf16_bits(d[where])
    elif where == "state0":
        d["state0"][0, 1, 3, 7] = 1.0e6
    t = dev_inputs(d)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    run_prefill(t, status=status)
    want = 0 if where == "none" else gb.CODES["GDN_ERR_RANGE"]
    assert int(status.item()) == want
