"""fp64 CPU oracle for the Gated DeltaNet recurrent-state path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the benchmark's CPU-baseline leg, never by the product path.  It shares
no code with the HIP library and imports nothing from the package.

Arrays follow one layout (C order, float64 unless stated):
  q, k        [B][N][Hqk][dk]
  v           [B][N][Hv][dv]
  alpha, beta [B][N][Hv]
  state       [slots][Hv][dv][dk]   S = H^T, row j = value channel j
  out         [B][N][Hv][dv]
  nodes       [B][N][Hv][dv][dk]    state after each node
Value head h reads q/k head h // (Hv // Hqk).

Parity status per function (the tests that pin each one are in
``tests/test_oracle_pins.py``):
  step     pinned: exact-rational brute force of the printed matrix rule,
           closed forms (beta=0, alpha=0, delta write, orthonormal keys)
  chain    pinned: composition of exact-rational steps, linearity, decay
  tree     pinned: equals the chain along every root path; non-ancestor
           inputs do not reach a node
  chunked  pinned: equals the stepwise chain for every chunk length
  commit   pinned: by its definition (index semantics), exercised in tests
  conv_commit  pinned: a causal convolution over the committed history and
           the next inputs equals the convolution over the whole accepted
           stream (chains and tree paths); index and slot handling
  commit_index  pinned by its definition (index semantics) and by the
           property that the pool row it selects holds the accepted node's
           state, checked against the chain in tests
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build  # noqa: WPS433 (test infrastructure)
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    i, d = ctypes.c_int, ctypes.c_double
    lib.oracle_gdn_step.argtypes = [i, i, d, _dp, _dp, _dp, _dp, d, d, _dp, _dp]
    lib.oracle_gdn_step.restype = None
    lib.oracle_gdn_chain.argtypes = [i, i, i, i, i, i, d, _dp, _dp, _dp, _dp, _dp, _dp,
                                     _dp, _dp, _dp, i]
    lib.oracle_gdn_chain.restype = i
    lib.oracle_gdn_tree.argtypes = [i, i, i, i, i, i, d, _dp, _dp, _dp, _dp, _dp, _dp,
                                    _ip, _dp, _dp, i]
    lib.oracle_gdn_tree.restype = i
    lib.oracle_gdn_chunked.argtypes = [i, i, i, i, i, i, d, i, _dp, _dp, _dp, _dp, _dp, _dp,
                                       _dp, _dp, i]
    lib.oracle_gdn_chunked.restype = i
    _lib = lib
    return lib


def default_threads() -> int:
    """Worker threads for the oracle: the CPUs this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _threads(n: int) -> int:
    return int(n) if n and n > 0 else default_threads()


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def _dims(q, v):
    B, N, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    return B, N, Hqk, Hv, dk, dv


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def step(S, q, k, v, alpha, beta, scale: float = 1.0):
    """One application of the gated delta rule to one head.

    S [dv][dk], q,k [dk], v [dv], scalars alpha, beta.  Returns (S', o) with
    S' = alpha S (I - beta k k^T) + beta v k^T and o = scale S' q.
    """
    lib = _load()
    S = _f64(S); q = _f64(q); k = _f64(k); v = _f64(v)
    dv, dk = S.shape
    Sout = np.empty_like(S)
    o = np.empty(dv, dtype=np.float64)
    lib.oracle_gdn_step(dk, dv, float(scale), _ptr(S), _ptr(q), _ptr(k), _ptr(v),
                        float(alpha), float(beta), _ptr(Sout), _ptr(o))
    return Sout, o


def chain(q, k, v, alpha, beta, state0, scale: float = 1.0, nodes: bool = True,
          nthreads: int = 0):
    """Stepwise recurrence over a chain of N nodes per sequence.

    Returns dict(out [B][N][Hv][dv], nodes [B][N][Hv][dv][dk] or None,
    final [B][Hv][dv][dk]).  ``state0`` is [B][Hv][dv][dk].
    """
    lib = _load()
    q, k, v, alpha, beta, state0 = map(_f64, (q, k, v, alpha, beta, state0))
    B, N, Hqk, Hv, dk, dv = _dims(q, v)
    out = np.zeros((B, N, Hv, dv))
    nd = np.zeros((B, N, Hv, dv, dk)) if nodes else None
    fin = np.zeros((B, Hv, dv, dk))
    rc = lib.oracle_gdn_chain(B, N, Hqk, Hv, dk, dv, float(scale), _ptr(q), _ptr(k), _ptr(v),
                              _ptr(alpha), _ptr(beta), _ptr(state0), _ptr(out), _ptr(nd),
                              _ptr(fin), _threads(nthreads))
    _check(rc, "chain")
    return {"out": out, "nodes": nd, "final": fin}


def tree(q, k, v, alpha, beta, state0, parent, scale: float = 1.0, nodes: bool = True,
         nthreads: int = 0):
    """Each node n starts from node parent[n]'s state (-1: the cached state).

    ``parent`` is [N] (one tree for every sequence) or [B][N].  Returns
    dict(out, nodes) as for :func:`chain`.
    """
    lib = _load()
    q, k, v, alpha, beta, state0 = map(_f64, (q, k, v, alpha, beta, state0))
    B, N, Hqk, Hv, dk, dv = _dims(q, v)
    par = np.asarray(parent, dtype=np.int32)
    if par.ndim == 1:
        par = np.broadcast_to(par, (B, N))
    par = np.ascontiguousarray(par, dtype=np.int32)
    out = np.zeros((B, N, Hv, dv))
    nd = np.zeros((B, N, Hv, dv, dk)) if nodes else None
    rc = lib.oracle_gdn_tree(B, N, Hqk, Hv, dk, dv, float(scale), _ptr(q), _ptr(k), _ptr(v),
                             _ptr(alpha), _ptr(beta), _ptr(state0),
                             par.ctypes.data_as(_ip), _ptr(out), _ptr(nd), _threads(nthreads))
    _check(rc, "tree")
    return {"out": out, "nodes": nd}


def chunked(q, k, v, alpha, beta, state0, chunk: int, scale: float = 1.0, nthreads: int = 0):
    """Chunked WY/UT form of the chain; returns dict(out, final)."""
    lib = _load()
    q, k, v, alpha, beta, state0 = map(_f64, (q, k, v, alpha, beta, state0))
    B, T, Hqk, Hv, dk, dv = _dims(q, v)
    out = np.zeros((B, T, Hv, dv))
    fin = np.zeros((B, Hv, dv, dk))
    rc = lib.oracle_gdn_chunked(B, T, Hqk, Hv, dk, dv, float(scale), int(chunk), _ptr(q),
                                _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state0),
                                _ptr(out), _ptr(fin), _threads(nthreads))
    _check(rc, "chunked")
    return {"out": out, "final": fin}


def commit(state, nodes, accepted, final=None, state_slot=None):
    """Commit of the accepted node, by definition.

    For every sequence b with a = accepted[b] in [0, N): the cache entry
    s = state_slot[b] (or b) becomes the state after node a; when ``final``
    is given and a == N-1 that state is ``final[b]``.  Out-of-range nodes or
    slots leave the cache entry as it was.  Page "400 tok/s with Qwen3.5",
    section "Handling recurrent state": the state is reconstructed at the
    accepted boundary, and a fully accepted block uses the verified state.
    Returns (new_state, n_rejected).
    """
    new = np.array(state, copy=True)
    B, N = nodes.shape[0], nodes.shape[1]
    bad = 0
    for b in range(B):
        a = int(accepted[b])
        s = int(state_slot[b]) if state_slot is not None else b
        if not (0 <= a < N) or not (0 <= s < new.shape[0]):
            bad += 1
            continue
        src = final[b] if (final is not None and a == N - 1) else nodes[b, a]
        new[s] = src
    return new, bad


def conv_commit(history, x, accepted, parent=None, state_slot=None):
    """Commit of the causal-convolution input history, by definition.

    Page "400 tok/s with Qwen3.5", section "Handling recurrent state": the
    convolution history is committed to the same boundary as the recurrent
    state.  A causal convolution of width W reads the current input row and the
    W - 1 rows before it, so the history a sequence keeps is its last W - 1
    input rows, oldest first.

    history [slots][W-1][C]; x [B][N][C] (the draft block's inputs);
    accepted [B]; parent None (a chain: node n follows node n - 1) or [N] /
    [B][N] (node 0 follows the history).  For sequence b with a = accepted[b],
    the accepted input stream is the history rows followed by the inputs of
    the nodes on a's root path, root first; the new history is the last W - 1
    rows of that stream.  Out-of-range nodes or slots leave the entry as it
    was.  Returns (new_history, n_rejected).
    """
    hist = np.asarray(history)
    new = np.array(hist, copy=True)
    B, N = x.shape[0], x.shape[1]
    keep = hist.shape[1]
    bad = 0
    for b in range(B):
        a = int(accepted[b])
        s = int(state_slot[b]) if state_slot is not None else b
        if not (0 <= a < N) or not (0 <= s < hist.shape[0]):
            bad += 1
            continue
        if parent is None:
            path = list(range(a + 1))
        else:
            par = np.asarray(parent)
            par = par[b] if par.ndim == 2 else par
            path, n = [], a
            while n >= 0:
                path.append(n)
                n = int(par[n])
            path.reverse()
        stream = [hist[s, i] for i in range(keep)] + [x[b, n] for n in path]
        for i in range(keep):
            new[s, i] = stream[len(stream) - keep + i]
    return new, bad


def causal_conv(history, x_rows, weight):
    """The causal depthwise convolution the history serves (for pins only):
    y_t[c] = sum_j weight[c][j] * u_{t - (W-1) + j}[c] over the stream u =
    history rows followed by x_rows; one output per x row.  history [W-1][C],
    x_rows [T][C], weight [C][W]."""
    hist = np.asarray(history, dtype=np.float64)
    xs = np.asarray(x_rows, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    W = w.shape[1]
    u = np.concatenate([hist, xs], axis=0)
    y = np.zeros_like(xs)
    for t in range(xs.shape[0]):
        for j in range(W):
            y[t] += w[:, j] * u[t + j]
    return y


def commit_index(state_slot, accepted, draft_row0, n_nodes, n_slots):
    """Index-table commit, by definition.

    Page "LightSeek's TokenSpeed Hits 580 Tokens per Second on Qwen3.5's 400B
    Model", section "How they actually got there" (move pointers, not data):
    the state buffer is extended with a draft region that holds every node's
    state, and an index table records which row holds a sequence's state;
    the commit writes one index instead of copying a state.  With node n of
    sequence b persisted in row draft_row0 + b * n_nodes + n, the commit sets
    state_slot[b] to the accepted node's row.  An accepted node outside
    [0, n_nodes), or a row outside [0, n_slots), leaves the entry as it was.
    Returns (new_state_slot, n_rejected).
    """
    new = np.array(state_slot, dtype=np.int64, copy=True)
    bad = 0
    for b in range(len(new)):
        a = int(accepted[b])
        row = draft_row0 + b * n_nodes + a
        if not (0 <= a < n_nodes) or not (0 <= row < n_slots):
            bad += 1
            continue
        new[b] = row
    return new.astype(np.int32), bad
