"""The seeded input recipes: number formats, shapes, tree and accept draws."""
import numpy as np
import torch

from gated_deltanet_recurrence_gdn_amd import workloads as wl


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.0078125, 3.3895314e38, 1e-40], np.float32)])
    x = x.astype(np.float32)
    ours = wl.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = wl.bf16_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_inputs_shapes_and_distributions():
    w = wl.WORKLOADS["chain"]
    d = wl.make_inputs(w)
    assert d["q"].shape == (1, 16, 16, 128) and d["v"].shape == (1, 16, 48, 128)
    assert d["state0"].shape == (1, 48, 128, 128)
    assert np.array_equal(wl.bf16_to_f32(d["q_bits"]), d["q"])
    n = np.linalg.norm(d["k"].astype(np.float64), axis=-1)
    assert np.all(np.abs(n - 1) < 1e-2)
    assert np.all((d["beta"] > 0) & (d["beta"] < 1)) and np.all((d["alpha"] > 0) & (d["alpha"] < 1))
    assert 0.09 < d["state0"].std() < 0.11
    d2 = wl.make_inputs(w)
    assert np.array_equal(d["v_bits"], d2["v_bits"])  # seeded


def test_random_tree_constraints():
    rng = np.random.default_rng(1)
    for _ in range(200):
        p = wl.random_tree(22, 16, rng)
        assert p[0] == -1 and all(0 <= p[i] < i for i in range(1, 22))
        assert wl.tree_depths(p).max() <= 16


def test_accepted_draws_in_range():
    rng = np.random.default_rng(2)
    a = wl.accepted_chain(1000, 16, rng)
    assert a.min() == 0 and a.max() == 15
    p = wl.random_tree(22, 16, rng)
    t = wl.accepted_tree(p, 1000, rng)
    assert t.min() >= 0 and t.max() < 22
    assert 0 in t  # prefix length 1 is the root


def test_ledger_matches_hand_count():
    led = wl.algorithmic_bytes_verify(wl.WORKLOADS["chain"])
    assert led["verify_total"] == 32_184_320
    assert led["commit"] == 4_718_592
    assert led["total"] == 36_902_912


def test_bench_refuses_more_than_one_gpu():
    """The benchmark measures one GPU; asking for more exits with a message before touching a device."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr
