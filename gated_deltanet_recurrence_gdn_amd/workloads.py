"""Seeded synthetic inputs for the verify / commit / prefill path.

Holds input recipes only (shapes, value distributions, tree shapes, accepted
lengths) and none of the recurrence's arithmetic, so the GPU tests, the
benchmark and the CPU oracle can all draw the same inputs.  Pure numpy.

Recipe (every workload):
  q, k   rows ~ N(0, 1) in fp32, L2-normalised per (token, q/k head), then
         rounded to bf16 (round-to-nearest-even) unless the workload is fp32
  v      ~ N(0, 1), rounded to bf16 unless fp32
  beta   = sigmoid(N(0, 1))            fp32, one per (token, value head)
  alpha  = exp(-softplus(N(0, 1)))     fp32, one per (token, value head)
  state  ~ N(0, 1) * 0.1               fp32, S laid out [Hv][dv][dk]
A tree draws node i's parent uniformly from the earlier nodes whose depth is
at most max_depth - 1 (node 0 is the root, depth 1).  The accepted node of a
chain is L - 1 for an accepted length L uniform in [1, N]; in a tree a leaf is
drawn uniformly and then a prefix length uniform in [1, depth(leaf)].
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 1000


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the exact fp32 values they encode."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    return bf16_to_f32(bf16_bits(x))


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_nodes: int
    h_qk: int
    h_v: int
    d_k: int
    d_v: int
    qkv_bf16: bool = True
    persist_f16: bool = True
    tree: bool = False
    max_depth: int = 16
    prefill: bool = False
    chunk: int = 64
    notes: str = field(default="", compare=False)


WORKLOADS = {
    "tiny_chain": Workload("tiny_chain", 1, 16, 1, 2, 32, 32, qkv_bf16=False, persist_f16=False,
                           notes="1 sequence, 2 value heads on 1 q/k head, d=32, fp32 throughout"),
    "chain": Workload("chain", 1, 16, 16, 48, 128, 128,
                      notes="one layer, batch 1, 16/48 heads, d=128, 16-token chain"),
    "tree": Workload("tree", 1, 22, 16, 48, 128, 128, tree=True,
                     notes="one layer, batch 1, 22-node tree, depth <= 16"),
    "batched_chain": Workload("batched_chain", 8 * 48, 16, 16, 48, 128, 128,
                              notes="8 sequences x 48 layers folded into the batch"),
    "prefill": Workload("prefill", 1, 4096, 16, 48, 128, 128, prefill=True, chunk=64,
                        notes="4096-token prompt, chunk 64"),
}
WORKLOAD_SEEDS = {"tiny_chain": SEED_BASE + 0, "chain": SEED_BASE + 1, "tree": SEED_BASE + 2,
                  "batched_chain": SEED_BASE + 3, "prefill": SEED_BASE + 4}


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32), dtype=np.float32)
    n = np.where(n > 0, n, np.float32(1.0))
    return (x / n).astype(np.float32)


def random_tree(n_nodes: int, max_depth: int, rng: np.random.Generator) -> np.ndarray:
    """parent[0] = -1; parent[i] uniform over {j < i : depth(j) <= max_depth - 1}."""
    parent = np.full(n_nodes, -1, dtype=np.int32)
    depth = np.zeros(n_nodes, dtype=np.int32)
    if n_nodes == 0:
        return parent
    depth[0] = 1
    for i in range(1, n_nodes):
        ok = np.nonzero(depth[:i] <= max_depth - 1)[0]
        p = int(ok[rng.integers(0, ok.size)])
        parent[i] = p
        depth[i] = depth[p] + 1
    return parent


def tree_depths(parent: np.ndarray) -> np.ndarray:
    d = np.zeros(len(parent), dtype=np.int32)
    for i, p in enumerate(parent):
        d[i] = 1 if p < 0 else d[p] + 1
    return d


def chain_parent(n_nodes: int) -> np.ndarray:
    return np.arange(-1, n_nodes - 1, dtype=np.int32)


def accepted_chain(batch: int, n_nodes: int, rng) -> np.ndarray:
    """Accepted length L ~ U[1, N] per sequence -> node index L - 1."""
    return (rng.integers(1, n_nodes + 1, size=batch) - 1).astype(np.int32)


def accepted_tree(parent: np.ndarray, batch: int, rng) -> np.ndarray:
    """A leaf uniformly, then a prefix of its root path of uniform length."""
    n = len(parent)
    has_child = np.zeros(n, dtype=bool)
    for p in parent[1:]:
        has_child[p] = True
    leaves = np.nonzero(~has_child)[0]
    depth = tree_depths(parent)
    out = np.empty(batch, dtype=np.int32)
    for b in range(batch):
        leaf = int(leaves[rng.integers(0, leaves.size)])
        length = int(rng.integers(1, depth[leaf] + 1))
        node = leaf
        for _ in range(depth[leaf] - length):
            node = int(parent[node])
        out[b] = node
    return out


def make_inputs(w: Workload, seed: int | None = None, batch: int | None = None,
                n_nodes: int | None = None) -> dict:
    """Draw one set of inputs for workload ``w``.

    Returns numpy arrays: q, k, v as the exact fp32 values (already rounded to
    bf16 when the workload is bf16) plus q_bits/k_bits/v_bits (uint16) for
    bf16 workloads; alpha, beta, state0 (fp32); parent and accepted.
    """
    rng = np.random.default_rng(WORKLOAD_SEEDS.get(w.name, SEED_BASE) if seed is None else seed)
    B = w.batch if batch is None else batch
    N = w.n_nodes if n_nodes is None else n_nodes
    q = _unit_rows(_normal(rng, (B, N, w.h_qk, w.d_k)))
    k = _unit_rows(_normal(rng, (B, N, w.h_qk, w.d_k)))
    v = _normal(rng, (B, N, w.h_v, w.d_v))
    beta = (1.0 / (1.0 + np.exp(-_normal(rng, (B, N, w.h_v))))).astype(np.float32)
    alpha = np.exp(-np.logaddexp(np.float32(0.0), _normal(rng, (B, N, w.h_v)))).astype(np.float32)
    state0 = (_normal(rng, (B, w.h_v, w.d_v, w.d_k)) * np.float32(0.1)).astype(np.float32)
    d = {"alpha": alpha, "beta": beta, "state0": state0}
    if w.qkv_bf16:
        for name, x in (("q", q), ("k", k), ("v", v)):
            bits = bf16_bits(x)
            d[name + "_bits"] = bits
            d[name] = bf16_to_f32(bits)
    else:
        d.update(q=q, k=k, v=v)
    if w.tree:
        parent = random_tree(N, w.max_depth, rng)
        d["parent"] = parent
        d["accepted"] = accepted_tree(parent, B, rng)
    else:
        d["parent"] = chain_parent(N)
        d["accepted"] = accepted_chain(B, N, rng) if N > 0 else np.zeros(B, np.int32)
    return d


def algorithmic_bytes_verify(w: Workload, out_bytes: int = 4) -> dict:
    """Bytes the verify + commit step must move (inputs once, outputs once)."""
    B, N = w.batch, w.n_nodes
    qk_b = 2 if w.qkv_bf16 else 4
    p_b = 2 if w.persist_f16 else 4
    hs = w.d_v * w.d_k
    items = {
        "state_read": B * w.h_v * hs * 4,
        "qk": 2 * B * N * w.h_qk * w.d_k * qk_b,
        "v": B * N * w.h_v * w.d_v * qk_b,
        "gates": 2 * B * N * w.h_v * 4,
        "out": B * N * w.h_v * w.d_v * out_bytes,
        "persist": B * N * w.h_v * hs * p_b,
        "final_state": 0 if w.tree else B * w.h_v * hs * 4,
        "commit": B * w.h_v * hs * (p_b + 4),
    }
    items["verify_total"] = sum(v for k, v in items.items() if k != "commit")
    items["total"] = items["verify_total"] + items["commit"]
    # one launch per step: the previous step's accepted node is read (its f16/fp32
    # copy) instead of the cached state, and written back as the committed state
    items["fused_total"] = (items["verify_total"] - items["state_read"] + B * w.h_v * hs * p_b
                            + B * w.h_v * hs * 4 + B * 4)
    return items


def algorithmic_bytes_replay(w: Workload, out_bytes: int = 4) -> dict:
    """Bytes of one decode step with commit by replay, in one launch: the cached
    state read and the committed state written (fp32), the replayed block's
    inputs (counted whole: the accepted prefix is drawn per step) and the
    accepted index, the next block's inputs and its outputs.  No node states
    are persisted and no final state is written."""
    B, N = w.batch, w.n_nodes
    qk_b = 2 if w.qkv_bf16 else 4
    hs = w.d_v * w.d_k
    block_in = 2 * B * N * w.h_qk * w.d_k * qk_b + B * N * w.h_v * w.d_v * qk_b + 2 * B * N * w.h_v * 4
    items = {
        "state_read": B * w.h_v * hs * 4,
        "replayed_inputs": block_in,
        "accepted": B * 4,
        "inputs": block_in,
        "out": B * N * w.h_v * w.d_v * out_bytes,
        "state_write": B * w.h_v * hs * 4,
    }
    items["total"] = sum(items.values())
    return items


def algorithmic_bytes_index(w: Workload, out_bytes: int = 4) -> dict:
    """Bytes of one decode step with the index-table commit: the verify reads
    the state through the index table and persists every node's state in fp32
    into the pool's draft rows; the commit writes one index per sequence."""
    B, N = w.batch, w.n_nodes
    qk_b = 2 if w.qkv_bf16 else 4
    hs = w.d_v * w.d_k
    items = {
        "index_read": B * 4,
        "state_read": B * w.h_v * hs * 4,
        "qk": 2 * B * N * w.h_qk * w.d_k * qk_b,
        "v": B * N * w.h_v * w.d_v * qk_b,
        "gates": 2 * B * N * w.h_v * 4,
        "out": B * N * w.h_v * w.d_v * out_bytes,
        "persist_f32": B * N * w.h_v * hs * 4,
        "commit": B * 4 + B * 4,
    }
    items["total"] = sum(items.values())
    return items
