"""Shared helpers for the GPU tests: device copies of seeded inputs, the
error metric, tolerances and small launch wrappers."""
from __future__ import annotations

import sys

import numpy as np
import torch

from gated_deltanet_recurrence_gdn_amd import binding as gb
from gated_deltanet_recurrence_gdn_amd import workloads as wl

DEV = "cuda:0"

# Parity bar: max relative error (max |x - ref| / max |ref| over the whole
# tensor) of outputs and fp32 states against the fp64 oracle; persisted f16
# states get a wider bar.
OUT_TOL = 2e-3
STATE_TOL = 2e-3
PERSIST_TOL = 1e-2


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def max_rel(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    if den == 0.0:
        return float(np.max(np.abs(x))) if x.size else 0.0
    return float(np.max(np.abs(x - ref))) / den


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy() if t.dtype != torch.float32 else t.detach().cpu().numpy()


def dev_inputs(d: dict, bf16: bool = True) -> dict:
    t = {}
    for n in ("q", "k", "v"):
        if bf16:
            t[n] = torch.from_numpy(np.ascontiguousarray(d[n + "_bits"]).view(np.int16)).to(DEV).view(torch.bfloat16)
        else:
            t[n] = torch.from_numpy(np.ascontiguousarray(d[n])).to(DEV)
    for n in ("alpha", "beta", "state0"):
        t[n] = torch.from_numpy(np.ascontiguousarray(d[n])).to(DEV)
    return t


def alloc_outputs(t, n_nodes, persist_dtype=torch.float16, out_dtype=torch.float32, final=True):
    B = t["q"].shape[0]
    Hv, dv = t["v"].shape[2], t["v"].shape[3]
    dk = t["q"].shape[3]
    out = torch.full((B, n_nodes, Hv, dv), float("nan"), dtype=out_dtype, device=DEV)
    persist = (torch.full((B, n_nodes, Hv, dv, dk), float("nan"), dtype=persist_dtype, device=DEV)
               if persist_dtype is not None else None)
    fin = torch.full((B, Hv, dv, dk), float("nan"), dtype=torch.float32, device=DEV) if final else None
    return out, persist, fin


def run_chain(t, n_nodes, persist_dtype=torch.float16, out_dtype=torch.float32, final=True, scale=1.0,
              state=None, **kw):
    out, persist, fin = alloc_outputs(t, n_nodes, persist_dtype, out_dtype, final)
    gb.gdn_verify_chain(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["state0"] if state is None else state,
                        out=out, persist=persist, final_state=fin, scale=scale, **kw)
    torch.cuda.synchronize()
    return out, persist, fin


def run_tree(t, parent, n_nodes, persist_dtype=torch.float16, out_dtype=torch.float32, scale=1.0, **kw):
    out, persist, _ = alloc_outputs(t, n_nodes, persist_dtype, out_dtype, final=False)
    gb.gdn_verify_tree(parent, t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["state0"], out=out,
                       persist=persist, scale=scale, **kw)
    torch.cuda.synchronize()
    return out, persist


def small_inputs(seed, B, N, Hqk, Hv, dk, dv, bf16=True, tree=False):
    w = wl.Workload("custom", B, N, Hqk, Hv, dk, dv, qkv_bf16=bf16, tree=tree)
    return w, wl.make_inputs(w, seed=seed)
