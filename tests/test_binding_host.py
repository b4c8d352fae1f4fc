"""The Python binding checks tensor shapes against each other before anything
reaches the C ABI (host only: every call here is refused on the host, with
CPU tensors, so nothing is launched)."""
import numpy as np
import pytest
import torch

from gated_deltanet_recurrence_gdn_amd import binding as gb

B, N, HQK, HV, DK, DV = 2, 4, 2, 4, 32, 16


def verify_args(**over):
    a = dict(q=torch.zeros(B, N, HQK, DK, dtype=torch.bfloat16), k=torch.zeros(B, N, HQK, DK, dtype=torch.bfloat16),
             v=torch.zeros(B, N, HV, DV, dtype=torch.bfloat16), alpha=torch.zeros(B, N, HV),
             beta=torch.zeros(B, N, HV), state=torch.zeros(B, HV, DV, DK), out=torch.zeros(B, N, HV, DV),
             persist=torch.zeros(B, N, HV, DV, DK, dtype=torch.float16), final_state=torch.zeros(B, HV, DV, DK))
    a.update(over)
    return a


def call_chain(a):
    return gb.gdn_verify_chain(a.pop("q"), a.pop("k"), a.pop("v"), a.pop("alpha"), a.pop("beta"), a.pop("state"),
                               **a)


def test_well_formed_cpu_tensors_are_refused_as_host_memory():
    with pytest.raises(TypeError, match="device tensor"):
        call_chain(verify_args())


@pytest.mark.parametrize("name,bad", [
    ("k", torch.zeros(B, N, HQK, DK + 1, dtype=torch.bfloat16)),
    ("k", torch.zeros(B, N + 1, HQK, DK, dtype=torch.bfloat16)),
    ("v", torch.zeros(B, N - 1, HV, DV, dtype=torch.bfloat16)),
    ("alpha", torch.zeros(B, N, HV + 1)),
    ("beta", torch.zeros(B, N)),
    ("out", torch.zeros(B, N, HV, DV + 16)),
    ("persist", torch.zeros(B, N, HV, DV, DK // 2, dtype=torch.float16)),
    ("final_state", torch.zeros(B + 1, HV, DV, DK)),
    ("state", torch.zeros(B - 1, HV, DV, DK)),           # fewer rows than sequences, no state_slot
    ("state", torch.zeros(B, HV, DK, DV * 2)),
    ("state_slot", torch.zeros(B + 1, dtype=torch.int32)),
    ("status", torch.zeros(0, dtype=torch.int32)),
])
def test_verify_chain_rejects_mismatched_shapes(name, bad):
    with pytest.raises(ValueError):
        call_chain(verify_args(**{name: bad}))


@pytest.mark.parametrize("name,bad", [
    ("k", torch.zeros(B, N, HQK, DK)),                       # k fp32, q bf16
    ("alpha", torch.zeros(B, N, HV, dtype=torch.float64)),
    ("state", torch.zeros(B, HV, DV, DK, dtype=torch.float16)),
    ("state_slot", torch.zeros(B, dtype=torch.int64)),
    ("persist", torch.zeros(B, N, HV, DV, DK, dtype=torch.bfloat16)),
])
def test_verify_chain_rejects_wrong_dtypes(name, bad):
    with pytest.raises(TypeError):
        call_chain(verify_args(**{name: bad}))


def test_state_slot_lifts_the_row_count_rule():
    a = verify_args(state=torch.zeros(1, HV, DV, DK), state_slot=torch.zeros(B, dtype=torch.int32))
    with pytest.raises(TypeError, match="device tensor"):  # shapes accepted; refused only as host memory
        call_chain(a)


def test_tree_parent_must_match_the_node_count():
    a = verify_args()
    for parent in (np.array([-1, 0, 1], np.int32), np.array([[-1, 0, 1, 2]] * 3, np.int32)):
        with pytest.raises(ValueError, match="parent"):
            gb.gdn_verify_tree(parent, a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["state"], out=a["out"])


def test_fused_commit_verify_checks_the_previous_block():
    a = verify_args()
    acc = torch.zeros(B, dtype=torch.int32)
    with pytest.raises(ValueError):
        gb.gdn_commit_verify_chain(torch.zeros(B + 1, dtype=torch.int32), a["persist"], a["q"], a["k"], a["v"],
                                   a["alpha"], a["beta"], a["state"], out=a["out"], persist=a["persist"])
    with pytest.raises(ValueError):
        gb.gdn_commit_verify_chain(acc, torch.zeros(B, N + 1, HV, DV, DK, dtype=torch.float16), a["q"], a["k"], a["v"],
                                   a["alpha"], a["beta"], a["state"], out=a["out"], persist=a["persist"])
    with pytest.raises(TypeError):
        gb.gdn_commit_verify_chain(acc, a["persist"].float(), a["q"], a["k"], a["v"], a["alpha"], a["beta"],
                                   a["state"], out=a["out"], persist=a["persist"])
    with pytest.raises(ValueError):
        gb.gdn_commit_verify_chain(acc, a["persist"], a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["state"],
                                   final_prev=torch.zeros(B, HV, DV, DK + 32), persist=a["persist"])


def test_fused_commit_verify_tree_checks_the_previous_block_and_the_tree():
    a = verify_args()
    acc = torch.zeros(B, dtype=torch.int32)
    par = np.array([-1] + list(range(N - 1)), np.int32)
    args = (a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["state"])
    with pytest.raises(ValueError):
        gb.gdn_commit_verify_tree(torch.zeros(B + 1, dtype=torch.int32), a["persist"], par, *args, out=a["out"],
                                  persist=a["persist"])
    with pytest.raises(ValueError):
        gb.gdn_commit_verify_tree(acc, torch.zeros(B, N + 1, HV, DV, DK, dtype=torch.float16), par, *args,
                                  out=a["out"], persist=a["persist"])
    with pytest.raises(TypeError):
        gb.gdn_commit_verify_tree(acc, a["persist"].float(), par, *args, out=a["out"], persist=a["persist"])
    with pytest.raises(ValueError, match="parent"):
        gb.gdn_commit_verify_tree(acc, a["persist"], par[:-1], *args, out=a["out"], persist=a["persist"])


def test_commit_checks_index_state_and_final_shapes():
    per = torch.zeros(B, N, HV, DV, DK, dtype=torch.float16)
    st = torch.zeros(B, HV, DV, DK)
    with pytest.raises(ValueError):
        gb.gdn_commit(torch.zeros(B + 1, dtype=torch.int32), per, st)
    with pytest.raises(ValueError):
        gb.gdn_commit(torch.zeros(B, dtype=torch.int32), per, torch.zeros(B, HV, DV + 16, DK))
    with pytest.raises(ValueError):
        gb.gdn_commit(torch.zeros(B, dtype=torch.int32), per, st, final_state=torch.zeros(B, HV + 1, DV, DK))
    with pytest.raises(TypeError):
        gb.gdn_commit(torch.zeros(B, dtype=torch.int32), per.bfloat16(), st)


def test_replay_verify_checks_the_previous_block_shapes():
    a = verify_args()
    acc = torch.zeros(B, dtype=torch.int32)
    with pytest.raises(ValueError):
        gb.gdn_replay_verify_chain(acc, a["q"][:, :2], a["k"][:, :2], a["v"][:, :2], a["alpha"][:, :2],
                                   a["beta"][:, :2], a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["state"],
                                   out=a["out"])


def test_conv_commit_checks_history_shape():
    x = torch.zeros(B, N, 64, dtype=torch.bfloat16)
    acc = torch.zeros(B, dtype=torch.int32)
    with pytest.raises(ValueError):
        gb.gdn_conv_commit(acc, x, torch.zeros(B, 3, 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        gb.gdn_conv_commit(acc, x, torch.zeros(B - 1, 3, 64, dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        gb.gdn_conv_commit(acc, x, torch.zeros(B, 3, 64))
    with pytest.raises(ValueError):
        gb.gdn_conv_commit(acc, x, torch.zeros(B, 3, 64, dtype=torch.bfloat16), parent=np.array([-1, 0], np.int32))


def test_prefill_checks_shapes_and_requires_out():
    T = 100
    q = torch.zeros(1, T, HQK, DK, dtype=torch.bfloat16)
    v = torch.zeros(1, T, HV, DV * 2, dtype=torch.bfloat16)
    g = torch.zeros(1, T, HV)
    st = torch.zeros(1, HV, DV * 2, DK)
    with pytest.raises(ValueError):
        gb.gdn_prefill_chunked(q, q, v, g, g, st, None)
    with pytest.raises(ValueError):
        gb.gdn_prefill_chunked(q, q, v, g, g, st, torch.zeros(1, T - 1, HV, DV * 2))
    with pytest.raises(ValueError):
        gb.gdn_prefill_chunked(q, q[:, :, :1], v, g, g, st, torch.zeros(1, T, HV, DV * 2))


def test_prefill_varlen_checks_cu_seqlens_and_chunk_states():
    total = 300
    q = torch.zeros(total, HQK, DK, dtype=torch.bfloat16)
    v = torch.zeros(total, HV, DV * 2, dtype=torch.bfloat16)
    g = torch.zeros(total, HV)
    st = torch.zeros(2, HV, DV * 2, DK)
    out = torch.zeros(total, HV, DV * 2)
    cu = np.array([0, 130, 300], np.int32)
    with pytest.raises(ValueError, match="cu_seqlens"):
        gb.gdn_prefill_varlen(np.array([0, 130, 299], np.int32), q, q, v, g, g, st, out)
    need = gb.gdn_prefill_boundary_states(cu, 1)
    assert need == 2 + 2  # full 64-token chunks: 130 -> 2, 170 -> 2
    with pytest.raises(ValueError, match="chunk_states"):
        gb.gdn_prefill_varlen(cu, q, q, v, g, g, st, out, chunk_states=torch.zeros(need - 1, HV, DV * 2, DK),
                              state_interval=1)
    with pytest.raises(TypeError, match="device tensor"):  # a large enough array is accepted
        gb.gdn_prefill_varlen(cu, q, q, v, g, g, st, out, chunk_states=torch.zeros(need, HV, DV * 2, DK),
                              state_interval=1, workspace=torch.zeros(16, dtype=torch.uint8))


def test_commit_index_checks_table_shapes():
    with pytest.raises(ValueError):
        gb.gdn_commit_index(torch.zeros(3, dtype=torch.int32), torch.zeros(2, dtype=torch.int32), N, 1, 1 + 2 * N)
    with pytest.raises(TypeError):
        gb.gdn_commit_index(torch.zeros(2, dtype=torch.int32), torch.zeros(2, dtype=torch.int64), N, 1, 1 + 2 * N)
