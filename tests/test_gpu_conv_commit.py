"""GPU parity of the convolution-history commit (gdn_conv_commit) through the
C ABI: the committed history must equal the oracle's, bit for bit (it is
index work: rows are copied, never computed)."""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_recurrence_gdn_amd import binding as gb
from gated_deltanet_recurrence_gdn_amd import workloads as wl
from helpers import DEV, say

pytestmark = pytest.mark.gpu

DT = {"bf16": (torch.bfloat16, np.uint16), "f16": (torch.float16, np.uint16), "f32": (torch.float32, np.uint32)}


def _draw(seed, B, N, C, W, slots, dtype):
    """Random bit patterns: the commit copies bits, so any pattern is a valid input."""
    rng = np.random.default_rng(seed)
    tdt, ndt = DT[dtype]
    x = rng.integers(0, np.iinfo(ndt).max, size=(B, N, C), dtype=ndt)
    h = rng.integers(0, np.iinfo(ndt).max, size=(slots, W - 1, C), dtype=ndt)
    sdt = np.int16 if ndt == np.uint16 else np.int32
    tx = torch.from_numpy(x.view(sdt)).to(DEV).view(tdt)
    th = torch.from_numpy(h.view(sdt)).to(DEV).view(tdt)
    return x, h, tx, th


def _bits(t):
    sdt = torch.int16 if t.element_size() == 2 else torch.int32
    return t.view(sdt).cpu().numpy().view(np.uint16 if t.element_size() == 2 else np.uint32)


def _run(acc, tx, th, parent=None, slot=None):
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    gb.gdn_conv_commit(torch.as_tensor(acc, dtype=torch.int32).to(DEV), tx, th, parent=parent, state_slot=slot,
                       status=status)
    torch.cuda.synchronize()
    return int(status.item())


@pytest.mark.parametrize("W", [2, 4, 8])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_conv_commit_chain_bit_exact(W, dtype):
    B, N, C = 5, 16, 10240 if dtype == "bf16" else 1000  # 10240: q, k, v channels of a 16/48-head d=128 layer
    x, h, tx, th = _draw(100 + W, B, N, C, W, B, dtype)
    acc = np.array([0, 1, W - 2, 9, N - 1], np.int32)
    assert _run(acc, tx, th) == 0
    ref, bad = oracle.conv_commit(h, x, acc)
    assert bad == 0
    got = _bits(th)
    say(f"conv chain W={W} {dtype}: rows equal {np.array_equal(got, ref)}")
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("per_seq", [False, True])
def test_conv_commit_tree_paths_bit_exact(per_seq):
    B, N, C, W = 20, 22, 256, 4
    rng = np.random.default_rng(110)
    pars = np.stack([wl.random_tree(N, 16, rng) for _ in range(B if per_seq else 1)]).astype(np.int32)
    par = pars if per_seq else pars[0]
    x, h, tx, th = _draw(111, B, N, C, W, B, "f16")
    acc = rng.integers(0, N, size=B).astype(np.int32)
    acc[0] = 0
    assert _run(acc, tx, th, parent=par) == 0
    ref, _ = oracle.conv_commit(h, x, acc, parent=par)
    assert np.array_equal(_bits(th), ref)


def test_conv_commit_slots_and_bad_entries():
    B, N, C, W = 4, 8, 64, 4
    x, h, tx, th = _draw(120, B, N, C, W, 6, "bf16")
    slot = np.array([5, 0, 3, 2], np.int32)
    acc = np.array([3, 8, 0, 7], np.int32)  # sequence 1: node out of range
    assert _run(acc, tx, th, slot=torch.from_numpy(slot).to(DEV)) == gb.CODES["GDN_ERR_NODE"]
    ref, bad = oracle.conv_commit(h, x, acc, state_slot=slot)
    assert bad == 1
    assert np.array_equal(_bits(th), ref)
    x, h, tx, th = _draw(121, B, N, C, W, 6, "bf16")
    bad_slot = np.array([5, 6, 3, 2], np.int32)
    assert _run(np.array([1, 1, 1, 1], np.int32), tx, th,
                slot=torch.from_numpy(bad_slot).to(DEV)) == gb.CODES["GDN_ERR_SLOT"]
    ref, _ = oracle.conv_commit(h, x, np.array([1, 1, 1, 1], np.int32), state_slot=bad_slot)
    assert np.array_equal(_bits(th), ref)
