"""Thin ctypes binding of libgdn.so (include/gdn.h), same entry-point names.

Argument marshalling only: shapes are read off the tensors and checked
against each other, dtypes mapped to gdn_dtype codes, device pointers and the
current HIP stream handed to the C ABI.  Every step of the computation runs
in the library's kernels; there is no fallback of any kind, and a missing
library raises.

Every entry point also takes ``prepare=True``: the tensors are checked and
marshalled once and a :class:`PreparedCall` is returned, whose call only
launches (the C function is called with the stored argument tuple; no tensor
is inspected again).  The prepared call keeps its tensors alive; they must
keep their storage, shapes and the stream must stay valid while it is used.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

# GDN_LIBRARY selects another build of the library (the debug build, libgdn_debug.so)
_LIB_PATH = os.environ.get("GDN_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")
_lib = None
_raw_fns: dict = {}

GDN_F32, GDN_BF16, GDN_F16 = 0, 1, 2
GDN_MAX_NODES = 32
GDN_MAX_TREE_DEPTH = 16
GDN_PREFILL_CHUNK = 64
GDN_MAX_CONV_WIDTH = 8
GDN_F16_MAX = 65504.0
GDN_PREFILL_SCRATCH_BYTES = 32 << 20

STATUS = {
    0: "GDN_OK", -1: "GDN_ERR_NULL", -2: "GDN_ERR_SHAPE", -3: "GDN_ERR_DTYPE", -4: "GDN_ERR_ALIGN",
    -5: "GDN_ERR_PARENT", -6: "GDN_ERR_NODE", -7: "GDN_ERR_WORKSPACE", -8: "GDN_ERR_UNSUPPORTED",
    -9: "GDN_ERR_HIP", -10: "GDN_ERR_SLOT", -11: "GDN_ERR_RANGE", -12: "GDN_ERR_INTERNAL",
}
CODES = {v: k for k, v in STATUS.items()}


class GdnError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {STATUS.get(code, code)} ({gdn_status_string(code)})")


class GdnConvShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_nodes", ctypes.c_int32), ("channels", ctypes.c_int32),
                ("width", ctypes.c_int32), ("n_slots", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class GdnShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_nodes", ctypes.c_int32), ("h_qk", ctypes.c_int32),
                ("h_v", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("n_slots", ctypes.c_int32), ("qkv_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("persist_dtype", ctypes.c_int32),
                ("scale", ctypes.c_float)]


_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_SIGS = {
    "gdn_verify_chain": [ctypes.POINTER(GdnShape)] + [_vp] * 12,
    "gdn_verify_tree": [ctypes.POINTER(GdnShape), _vp, _i32] + [_vp] * 11,
    "gdn_commit_verify_chain": [ctypes.POINTER(GdnShape)] + [_vp] * 15,
    "gdn_commit_verify_tree": [ctypes.POINTER(GdnShape), _vp, _vp, _vp, _i32] + [_vp] * 11,
    "gdn_commit": [ctypes.POINTER(GdnShape)] + [_vp] * 7,
    "gdn_commit_replay": [ctypes.POINTER(GdnShape), _vp, _i32] + [_vp] * 10,
    "gdn_replay_verify_chain": [ctypes.POINTER(GdnShape)] + [_vp] * 18,
    "gdn_conv_commit": [ctypes.POINTER(GdnConvShape), _vp, _i32] + [_vp] * 6,
    "gdn_commit_index": [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp],
    "gdn_status_string": [ctypes.c_int],
    "gdn_tree_walk": [_vp, _i32, _vp, _vp],
    "gdn_prefill_workspace_bytes": [ctypes.POINTER(GdnShape)],
    "gdn_prefill_chunked": [ctypes.POINTER(GdnShape)] + [_vp] * 9 + [ctypes.c_size_t, _vp, _vp],
    "gdn_prefill_varlen_workspace_bytes": [ctypes.POINTER(GdnShape), _vp],
    "gdn_prefill_boundary_states": [_vp, _i32, _i32],
    "gdn_prefill_varlen": [ctypes.POINTER(GdnShape)] + [_vp] * 10 + [_i32, _vp, ctypes.c_size_t, _vp, _vp],
    "gdn_prefill_chunked_noalloc": [ctypes.POINTER(GdnShape)] + [_vp] * 10,
}
_RESTYPES = {"gdn_status_string": ctypes.c_char_p, "gdn_prefill_workspace_bytes": ctypes.c_size_t,
             "gdn_prefill_varlen_workspace_bytes": ctypes.c_size_t, "gdn_prefill_boundary_states": ctypes.c_int64}


def lib() -> ctypes.CDLL:
    """The loaded HIP library (argument types declared); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(_LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = _RESTYPES.get(name, ctypes.c_int)
        _lib = L
    return _lib


def _raw(name: str):
    """The entry point without declared argument types: called with ctypes
    instances only, so ctypes converts nothing per call."""
    fn = _raw_fns.get(name)
    if fn is None:
        fn = lib()[name]  # a fresh function object, independent of the declared one
        fn.restype = ctypes.c_int
        _raw_fns[name] = fn
    return fn


def library_path() -> str:
    return _LIB_PATH


def gdn_status_string(code: int) -> str:
    return lib().gdn_status_string(int(code)).decode()


class PreparedCall:
    """One marshalled call of an entry point: calling it launches, nothing else."""

    __slots__ = ("name", "_fn", "_args", "_keep")

    def __init__(self, name, args, keep):
        self.name = name
        self._fn = _raw(name)
        self._args = tuple(args)
        self._keep = keep

    def __call__(self) -> None:
        rc = self._fn(*self._args)
        if rc != 0:
            raise GdnError(rc, self.name)


def _invoke(name, args, keep, prepare):
    call = PreparedCall(name, args, keep)
    if prepare:
        return call
    call()
    return None


# ---------------------------------------------------------------------------
# argument checks (host side, before anything reaches the C ABI)
# ---------------------------------------------------------------------------
def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return GDN_F32
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float16:
        return GDN_F16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _shape_of(t, name, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    return tuple(t.shape)


def _expect(t, name, shape, dtype=None):
    """t must be a tensor of exactly `shape` (None = any size) and `dtype`."""
    if t is None:
        return
    got = _shape_of(t, name, len(shape))
    for i, (g, e) in enumerate(zip(got, shape)):
        if e is not None and g != e:
            raise ValueError(f"{name} has shape {got}; dimension {i} must be {e}")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _dev_ptr(t, name: str):
    if t is None:
        return _vp(None)
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return _vp(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        return _vp(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return _vp(stream)
    return _vp(stream.cuda_stream)


_QKV = (torch.float32, torch.bfloat16)
_OUT = (torch.float32, torch.bfloat16, torch.float16)


def _check_qkv(q, k, v, alpha, beta, name=""):
    """q, k [B][N][h_qk][d_k] and v [B][N][h_v][d_v] of one dtype; alpha, beta [B][N][h_v] fp32."""
    B, N, Hqk, dk = _shape_of(q, "q" + name, 4)
    _expect(k, "k" + name, (B, N, Hqk, dk), q.dtype)
    _expect(v, "v" + name, (B, N, None, None), q.dtype)
    if q.dtype not in _QKV:
        raise TypeError(f"q{name} must be float32 or bfloat16, got {q.dtype}")
    Hv, dv = v.shape[2], v.shape[3]
    _expect(alpha, "alpha" + name, (B, N, Hv), torch.float32)
    _expect(beta, "beta" + name, (B, N, Hv), torch.float32)
    return B, N, Hqk, Hv, dk, dv


def _check_state(state, state_slot, B, Hv, dv, dk):
    _expect(state, "state", (None, Hv, dv, dk), torch.float32)
    if state_slot is None:
        if state.shape[0] < B:
            raise ValueError(f"state holds {state.shape[0]} rows; without state_slot it needs one per sequence ({B})")
    else:
        _expect(state_slot, "state_slot", (B,), torch.int32)


def _check_status(status):
    _expect(status, "status", (None,), torch.int32)
    if status is not None and status.numel() < 1:
        raise ValueError("status needs one element")


def _verify_shape(q, k, v, alpha, beta, state, state_slot, out, persist, final_state, status, scale):
    B, N, Hqk, Hv, dk, dv = _check_qkv(q, k, v, alpha, beta)
    _check_state(state, state_slot, B, Hv, dv, dk)
    _expect(out, "out", (B, N, Hv, dv), _OUT)
    _expect(persist, "persist", (B, N, Hv, dv, dk), (torch.float16, torch.float32))
    _expect(final_state, "final_state", (B, Hv, dv, dk), torch.float32)
    _check_status(status)
    return GdnShape(B, N, Hqk, Hv, dk, dv, state.shape[0], _dtype_code(q),
                    _dtype_code(out) if out is not None else GDN_F32,
                    _dtype_code(persist) if persist is not None else GDN_F16, float(scale))


def _host_parent(parent, n_nodes: int, batch: int) -> np.ndarray:
    if isinstance(parent, torch.Tensor):
        parent = parent.detach().cpu().numpy()
    par = np.ascontiguousarray(parent, dtype=np.int32)
    if par.ndim not in (1, 2) or par.shape[-1] != n_nodes or (par.ndim == 2 and par.shape[0] not in (1, batch)):
        raise ValueError(f"parent must be [N] or [B][N] with N = {n_nodes}, B = {batch}; got {par.shape}")
    return par


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def gdn_verify_chain(q, k, v, alpha, beta, state, *, out=None, persist=None, final_state=None,
                     state_slot=None, status=None, scale: float = 1.0, stream=None, prepare: bool = False):
    """Chain verify; see include/gdn.h.  Outputs are caller-allocated tensors."""
    sh = _verify_shape(q, k, v, alpha, beta, state, state_slot, out, persist, final_state, status, scale)
    args = (ctypes.byref(sh), _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dev_ptr(alpha, "alpha"),
            _dev_ptr(beta, "beta"), _dev_ptr(state, "state"), _dev_ptr(state_slot, "state_slot"),
            _dev_ptr(out, "out"), _dev_ptr(persist, "persist"), _dev_ptr(final_state, "final_state"),
            _dev_ptr(status, "status"), _stream(stream))
    return _invoke("gdn_verify_chain", args, (sh, q, k, v, alpha, beta, state, state_slot, out, persist,
                                              final_state, status), prepare)


def gdn_commit_verify_chain(accepted_prev, persist_prev, q, k, v, alpha, beta, state, *, final_prev=None,
                            out=None, persist=None, final_state=None, state_slot=None, status=None,
                            scale: float = 1.0, stream=None, prepare: bool = False):
    """Commit the previous step's accepted node and verify the next chain, in one launch."""
    sh = _verify_shape(q, k, v, alpha, beta, state, state_slot, out,
                       persist if persist is not None else persist_prev, final_state, status, scale)
    B, N, Hv, dv, dk = sh.batch, sh.n_nodes, sh.h_v, sh.d_v, sh.d_k
    _expect(accepted_prev, "accepted_prev", (B,), torch.int32)
    _expect(persist_prev, "persist_prev", (B, N, Hv, dv, dk), (torch.float16, torch.float32))
    if persist is not None and persist_prev is not None and persist.dtype != persist_prev.dtype:
        raise TypeError("persist and persist_prev must have one dtype")
    _expect(final_prev, "final_prev", (B, Hv, dv, dk), torch.float32)
    args = (ctypes.byref(sh), _dev_ptr(accepted_prev, "accepted_prev"), _dev_ptr(persist_prev, "persist_prev"),
            _dev_ptr(final_prev, "final_prev"), _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
            _dev_ptr(alpha, "alpha"), _dev_ptr(beta, "beta"), _dev_ptr(state, "state"),
            _dev_ptr(state_slot, "state_slot"), _dev_ptr(out, "out"), _dev_ptr(persist, "persist"),
            _dev_ptr(final_state, "final_state"), _dev_ptr(status, "status"), _stream(stream))
    return _invoke("gdn_commit_verify_chain", args, (sh, accepted_prev, persist_prev, final_prev, q, k, v, alpha,
                                                     beta, state, state_slot, out, persist, final_state, status),
                   prepare)


def gdn_verify_tree(parent, q, k, v, alpha, beta, state, *, out=None, persist=None, state_slot=None,
                    status=None, scale: float = 1.0, stream=None, prepare: bool = False):
    """Tree verify; ``parent`` is a host array [N] (shared) or [B][N]."""
    sh = _verify_shape(q, k, v, alpha, beta, state, state_slot, out, persist, None, status, scale)
    par = _host_parent(parent, sh.n_nodes, sh.batch)
    n_trees = 1 if par.ndim == 1 else par.shape[0]
    args = (ctypes.byref(sh), _vp(par.ctypes.data), _i32(n_trees), _dev_ptr(q, "q"), _dev_ptr(k, "k"),
            _dev_ptr(v, "v"), _dev_ptr(alpha, "alpha"), _dev_ptr(beta, "beta"), _dev_ptr(state, "state"),
            _dev_ptr(state_slot, "state_slot"), _dev_ptr(out, "out"), _dev_ptr(persist, "persist"),
            _dev_ptr(status, "status"), _stream(stream))
    return _invoke("gdn_verify_tree", args, (sh, par, q, k, v, alpha, beta, state, state_slot, out, persist, status),
                   prepare)


def gdn_commit_verify_tree(accepted_prev, persist_prev, parent, q, k, v, alpha, beta, state, *, out=None,
                           persist=None, state_slot=None, status=None, scale: float = 1.0, stream=None,
                           prepare: bool = False):
    """Commit the previous step's accepted node and verify the next tree, in one launch."""
    sh = _verify_shape(q, k, v, alpha, beta, state, state_slot, out,
                       persist if persist is not None else persist_prev, None, status, scale)
    B, N, Hv, dv, dk = sh.batch, sh.n_nodes, sh.h_v, sh.d_v, sh.d_k
    _expect(accepted_prev, "accepted_prev", (B,), torch.int32)
    _expect(persist_prev, "persist_prev", (B, N, Hv, dv, dk), (torch.float16, torch.float32))
    if persist is not None and persist_prev is not None and persist.dtype != persist_prev.dtype:
        raise TypeError("persist and persist_prev must have one dtype")
    par = _host_parent(parent, N, B)
    n_trees = 1 if par.ndim == 1 else par.shape[0]
    args = (ctypes.byref(sh), _dev_ptr(accepted_prev, "accepted_prev"), _dev_ptr(persist_prev, "persist_prev"),
            _vp(par.ctypes.data), _i32(n_trees), _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
            _dev_ptr(alpha, "alpha"), _dev_ptr(beta, "beta"), _dev_ptr(state, "state"),
            _dev_ptr(state_slot, "state_slot"), _dev_ptr(out, "out"), _dev_ptr(persist, "persist"),
            _dev_ptr(status, "status"), _stream(stream))
    return _invoke("gdn_commit_verify_tree", args, (sh, accepted_prev, persist_prev, par, q, k, v, alpha, beta,
                                                    state, state_slot, out, persist, status), prepare)


def gdn_tree_walk(parent):
    """(walk uint16[N], fork_slots) for one host parent array."""
    par = np.ascontiguousarray(parent.detach().cpu().numpy() if isinstance(parent, torch.Tensor) else parent,
                               dtype=np.int32)
    if par.ndim != 1:
        raise ValueError("parent must be one tree [N]")
    walk = np.zeros(max(par.size, 1), dtype=np.uint16)
    slots = ctypes.c_int32(0)
    rc = lib().gdn_tree_walk(par.ctypes.data, par.size, walk.ctypes.data, ctypes.byref(slots))
    if rc != 0:
        raise GdnError(rc, "gdn_tree_walk")
    return walk[:par.size], slots.value


def gdn_commit(accepted_node, persist, state, *, final_state=None, state_slot=None, status=None,
               stream=None, prepare: bool = False):
    """Commit; persist is [B][N][Hv][dv][dk] (f16 or fp32), state [slots][Hv][dv][dk]."""
    B, N, Hv, dv, dk = _shape_of(persist, "persist", 5)
    if persist.dtype not in (torch.float16, torch.float32):
        raise TypeError("persist must be float16 or float32")
    _expect(accepted_node, "accepted_node", (B,), torch.int32)
    _check_state(state, state_slot, B, Hv, dv, dk)
    _expect(final_state, "final_state", (B, Hv, dv, dk), torch.float32)
    _check_status(status)
    sh = GdnShape(B, N, 1, Hv, dk, dv, state.shape[0], GDN_BF16, GDN_F32, _dtype_code(persist), 1.0)
    args = (ctypes.byref(sh), _dev_ptr(accepted_node, "accepted_node"), _dev_ptr(persist, "persist"),
            _dev_ptr(final_state, "final_state"), _dev_ptr(state, "state"), _dev_ptr(state_slot, "state_slot"),
            _dev_ptr(status, "status"), _stream(stream))
    return _invoke("gdn_commit", args, (sh, accepted_node, persist, final_state, state, state_slot, status), prepare)


def gdn_commit_replay(accepted_node, q, k, v, alpha, beta, state, *, parent=None, state_slot=None, status=None,
                      stream=None, prepare: bool = False):
    """Commit by replay: state[slot(b)] <- the state after node accepted_node[b],
    re-run from state[slot(b)] over the node's root path (chain when ``parent``
    is None; else a host parent array [N] or [B][N])."""
    sh = _verify_shape(q, k, v, alpha, beta, state, state_slot, None, None, None, status, 1.0)
    _expect(accepted_node, "accepted_node", (sh.batch,), torch.int32)
    par, n_trees = None, 0
    if parent is not None:
        par = _host_parent(parent, sh.n_nodes, sh.batch)
        n_trees = 1 if par.ndim == 1 else par.shape[0]
    args = (ctypes.byref(sh), _vp(par.ctypes.data if par is not None else None), _i32(n_trees),
            _dev_ptr(accepted_node, "accepted_node"), _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
            _dev_ptr(alpha, "alpha"), _dev_ptr(beta, "beta"), _dev_ptr(state, "state"),
            _dev_ptr(state_slot, "state_slot"), _dev_ptr(status, "status"), _stream(stream))
    return _invoke("gdn_commit_replay", args, (sh, par, accepted_node, q, k, v, alpha, beta, state, state_slot,
                                               status), prepare)


def gdn_replay_verify_chain(accepted_prev, q_prev, k_prev, v_prev, alpha_prev, beta_prev, q, k, v, alpha, beta,
                            state, *, out=None, persist=None, final_state=None, state_slot=None, status=None,
                            scale: float = 1.0, stream=None, prepare: bool = False):
    """Commit the previous chain block by replay and verify the next one, in one launch."""
    sh = _verify_shape(q, k, v, alpha, beta, state, state_slot, out, persist, final_state, status, scale)
    if _check_qkv(q_prev, k_prev, v_prev, alpha_prev, beta_prev, "_prev") != (sh.batch, sh.n_nodes, sh.h_qk, sh.h_v,
                                                                            sh.d_k, sh.d_v):
        raise ValueError("the previous block's inputs must have this block's shapes")
    if q_prev.dtype != q.dtype:
        raise TypeError("the previous block's inputs must have this block's dtype")
    _expect(accepted_prev, "accepted_prev", (sh.batch,), torch.int32)
    args = (ctypes.byref(sh), _dev_ptr(accepted_prev, "accepted_prev"), _dev_ptr(q_prev, "q_prev"),
            _dev_ptr(k_prev, "k_prev"), _dev_ptr(v_prev, "v_prev"), _dev_ptr(alpha_prev, "alpha_prev"),
            _dev_ptr(beta_prev, "beta_prev"), _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
            _dev_ptr(alpha, "alpha"), _dev_ptr(beta, "beta"), _dev_ptr(state, "state"),
            _dev_ptr(state_slot, "state_slot"), _dev_ptr(out, "out"), _dev_ptr(persist, "persist"),
            _dev_ptr(final_state, "final_state"), _dev_ptr(status, "status"), _stream(stream))
    return _invoke("gdn_replay_verify_chain", args,
                   (sh, accepted_prev, q_prev, k_prev, v_prev, alpha_prev, beta_prev, q, k, v, alpha, beta, state,
                    state_slot, out, persist, final_state, status), prepare)


def gdn_commit_index(accepted_node, state_slot, n_nodes: int, draft_row0: int, n_slots: int, *, status=None,
                     stream=None, prepare: bool = False):
    """Index-table commit: state_slot[b] <- draft_row0 + b * n_nodes + accepted_node[b] (device arrays)."""
    (B,) = _shape_of(state_slot, "state_slot", 1)
    _expect(state_slot, "state_slot", (B,), torch.int32)
    _expect(accepted_node, "accepted_node", (B,), torch.int32)
    _check_status(status)
    args = (_dev_ptr(accepted_node, "accepted_node"), _dev_ptr(state_slot, "state_slot"), _i32(B), _i32(n_nodes),
            _i32(draft_row0), _i32(n_slots), _dev_ptr(status, "status"), _stream(stream))
    return _invoke("gdn_commit_index", args, (accepted_node, state_slot, status), prepare)


def gdn_conv_commit(accepted_node, x, conv_state, *, parent=None, state_slot=None, status=None,
                    stream=None, prepare: bool = False):
    """Commit the convolution history: conv_state [slots][W-1][C] <- the last
    W-1 rows of (history, inputs x [B][N][C] along the accepted node's root
    path); chain when ``parent`` is None, else a host array [N] or [B][N]."""
    B, N, C = _shape_of(x, "x", 3)
    _expect(conv_state, "conv_state", (None, None, C), x.dtype)
    _expect(accepted_node, "accepted_node", (B,), torch.int32)
    if state_slot is None:
        if conv_state.shape[0] < B:
            raise ValueError(f"conv_state holds {conv_state.shape[0]} rows; without state_slot it needs {B}")
    else:
        _expect(state_slot, "state_slot", (B,), torch.int32)
    _check_status(status)
    sh = GdnConvShape(B, N, C, conv_state.shape[1] + 1, conv_state.shape[0], _dtype_code(x))
    par, n_trees = None, 0
    if parent is not None:
        par = _host_parent(parent, N, B)
        n_trees = 1 if par.ndim == 1 else par.shape[0]
    args = (ctypes.byref(sh), _vp(par.ctypes.data if par is not None else None), _i32(n_trees),
            _dev_ptr(accepted_node, "accepted_node"), _dev_ptr(x, "x"), _dev_ptr(conv_state, "conv_state"),
            _dev_ptr(state_slot, "state_slot"), _dev_ptr(status, "status"), _stream(stream))
    return _invoke("gdn_conv_commit", args, (sh, par, accepted_node, x, conv_state, state_slot, status), prepare)


def _prefill_shape(q, k, v, alpha, beta, state, state_slot, out, status, scale) -> GdnShape:
    B, T, Hqk, Hv, dk, dv = _check_qkv(q, k, v, alpha, beta)
    _check_state(state, state_slot, B, Hv, dv, dk)
    _expect(out, "out", (B, T, Hv, dv), _OUT)
    if out is None:
        raise ValueError("out is required")
    _check_status(status)
    return GdnShape(B, T, Hqk, Hv, dk, dv, state.shape[0], _dtype_code(q), _dtype_code(out), GDN_F16,
                    float(scale))


def gdn_prefill_workspace_bytes(q, v, state, out, scale: float = 1.0) -> int:
    B, T, Hqk, dk = _shape_of(q, "q", 4)
    Hv, dv = v.shape[2], v.shape[3]
    sh = GdnShape(B, T, Hqk, Hv, dk, dv, state.shape[0], _dtype_code(q), _dtype_code(out), GDN_F16, float(scale))
    return int(lib().gdn_prefill_workspace_bytes(ctypes.byref(sh)))


def _bytes_of(t) -> int:
    return t.numel() * t.element_size()


def gdn_prefill_chunked(q, k, v, alpha, beta, state, out, *, state_slot=None, status=None, workspace=None,
                        scale: float = 1.0, stream=None, prepare: bool = False):
    """Chunked prefill; ``state`` is updated in place (see include/gdn.h).

    ``workspace`` is a device tensor of at least gdn_prefill_workspace_bytes
    bytes; when omitted one is allocated here with torch (plumbing only).
    """
    sh = _prefill_shape(q, k, v, alpha, beta, state, state_slot, out, status, scale)
    if workspace is None:
        need = int(lib().gdn_prefill_workspace_bytes(ctypes.byref(sh)))
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    args = (ctypes.byref(sh), _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dev_ptr(alpha, "alpha"),
            _dev_ptr(beta, "beta"), _dev_ptr(state, "state"), _dev_ptr(state_slot, "state_slot"),
            _dev_ptr(out, "out"), _dev_ptr(workspace, "workspace"), ctypes.c_size_t(_bytes_of(workspace)),
            _dev_ptr(status, "status"), _stream(stream))
    return _invoke("gdn_prefill_chunked", args, (sh, q, k, v, alpha, beta, state, state_slot, out, workspace,
                                                 status), prepare)


def gdn_prefill_chunked_noalloc(q, k, v, alpha, beta, state, out, *, state_slot=None, status=None,
                                scale: float = 1.0, stream=None, prepare: bool = False):
    """Chunked prefill that allocates nothing: the per-chunk operands go to the
    library's static per-GPU scratch array (see include/gdn.h).  Calls that may
    overlap on one GPU race."""
    sh = _prefill_shape(q, k, v, alpha, beta, state, state_slot, out, status, scale)
    args = (ctypes.byref(sh), _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dev_ptr(alpha, "alpha"),
            _dev_ptr(beta, "beta"), _dev_ptr(state, "state"), _dev_ptr(state_slot, "state_slot"),
            _dev_ptr(out, "out"), _dev_ptr(status, "status"), _stream(stream))
    return _invoke("gdn_prefill_chunked_noalloc", args, (sh, q, k, v, alpha, beta, state, state_slot, out, status),
                   prepare)


def _host_cu(cu_seqlens) -> np.ndarray:
    if isinstance(cu_seqlens, torch.Tensor):
        cu_seqlens = cu_seqlens.detach().cpu().numpy()
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    if cu.ndim != 1 or cu.size < 1:
        raise ValueError("cu_seqlens must be a 1-D host array [B + 1]")
    return cu


def gdn_prefill_boundary_states(cu_seqlens, state_interval: int) -> int:
    cu = _host_cu(cu_seqlens)
    return int(lib().gdn_prefill_boundary_states(cu.ctypes.data, cu.size - 1, int(state_interval)))


def _varlen_shape(cu, q, k, v, alpha, beta, state, state_slot, out, status, scale) -> GdnShape:
    total, Hqk, dk = _shape_of(q, "q", 3)
    _expect(k, "k", (total, Hqk, dk), q.dtype)
    _expect(v, "v", (total, None, None), q.dtype)
    if q.dtype not in _QKV:
        raise TypeError(f"q must be float32 or bfloat16, got {q.dtype}")
    Hv, dv = v.shape[1], v.shape[2]
    _expect(alpha, "alpha", (total, Hv), torch.float32)
    _expect(beta, "beta", (total, Hv), torch.float32)
    _expect(out, "out", (total, Hv, dv), _OUT)
    if out is None:
        raise ValueError("out is required")
    B = cu.size - 1
    if int(cu[-1]) != total:
        raise ValueError(f"cu_seqlens ends at {int(cu[-1])}, the inputs hold {total} tokens")
    _check_state(state, state_slot, B, Hv, dv, dk)
    _check_status(status)
    return GdnShape(B, total, Hqk, Hv, dk, dv, state.shape[0], _dtype_code(q), _dtype_code(out), GDN_F16,
                    float(scale))


def gdn_prefill_varlen_workspace_bytes(cu_seqlens, q, v, state, out, scale: float = 1.0) -> int:
    cu = _host_cu(cu_seqlens)
    total, Hqk, dk = _shape_of(q, "q", 3)
    Hv, dv = v.shape[1], v.shape[2]
    sh = GdnShape(cu.size - 1, total, Hqk, Hv, dk, dv, state.shape[0], _dtype_code(q), _dtype_code(out), GDN_F16,
                  float(scale))
    return int(lib().gdn_prefill_varlen_workspace_bytes(ctypes.byref(sh), cu.ctypes.data))


def gdn_prefill_varlen(cu_seqlens, q, k, v, alpha, beta, state, out, *, chunk_states=None, state_interval: int = 1,
                       state_slot=None, status=None, workspace=None, scale: float = 1.0, stream=None,
                       prepare: bool = False):
    """Varlen prefill of sequences packed along the token dimension (q [total][h_qk][d_k], ...);
    ``cu_seqlens`` is a host array [B + 1]; see include/gdn.h."""
    cu = _host_cu(cu_seqlens)
    sh = _varlen_shape(cu, q, k, v, alpha, beta, state, state_slot, out, status, scale)
    if chunk_states is not None:
        need = gdn_prefill_boundary_states(cu, state_interval)
        if need < 0:
            raise ValueError("invalid cu_seqlens or state_interval")
        _expect(chunk_states, "chunk_states", (None, sh.h_v, sh.d_v, sh.d_k), torch.float32)
        if chunk_states.shape[0] < need:
            raise ValueError(f"chunk_states holds {chunk_states.shape[0]} states; the call emits {need}")
    if workspace is None:
        need = int(lib().gdn_prefill_varlen_workspace_bytes(ctypes.byref(sh), cu.ctypes.data))
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    args = (ctypes.byref(sh), _vp(cu.ctypes.data), _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
            _dev_ptr(alpha, "alpha"), _dev_ptr(beta, "beta"), _dev_ptr(state, "state"),
            _dev_ptr(state_slot, "state_slot"), _dev_ptr(out, "out"), _dev_ptr(chunk_states, "chunk_states"),
            _i32(int(state_interval)), _dev_ptr(workspace, "workspace"), ctypes.c_size_t(_bytes_of(workspace)),
            _dev_ptr(status, "status"), _stream(stream))
    return _invoke("gdn_prefill_varlen", args, (sh, cu, q, k, v, alpha, beta, state, state_slot, out, chunk_states,
                                                workspace, status), prepare)
