"""Thin ctypes binding of libgdn.so (include/gdn.h), same entry-point names.

Argument marshalling only: shapes are read off the tensors, dtypes mapped to
gdn_dtype codes, device pointers and the current HIP stream handed to the C
ABI.  Every step of the computation runs in the library's kernels; there is
no fallback of any kind, and a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")
_lib = None

GDN_F32, GDN_BF16, GDN_F16 = 0, 1, 2
GDN_MAX_NODES = 32
GDN_MAX_TREE_DEPTH = 16
GDN_PREFILL_CHUNK = 64
GDN_MAX_CONV_WIDTH = 8

STATUS = {
    0: "GDN_OK", -1: "GDN_ERR_NULL", -2: "GDN_ERR_SHAPE", -3: "GDN_ERR_DTYPE", -4: "GDN_ERR_ALIGN",
    -5: "GDN_ERR_PARENT", -6: "GDN_ERR_NODE", -7: "GDN_ERR_WORKSPACE", -8: "GDN_ERR_UNSUPPORTED",
    -9: "GDN_ERR_HIP", -10: "GDN_ERR_SLOT",
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
_SIGS = {
    "gdn_verify_chain": [ctypes.POINTER(GdnShape)] + [_vp] * 12,
    "gdn_verify_tree": [ctypes.POINTER(GdnShape), _vp, ctypes.c_int32] + [_vp] * 11,
    "gdn_commit_verify_chain": [ctypes.POINTER(GdnShape)] + [_vp] * 15,
    "gdn_commit": [ctypes.POINTER(GdnShape)] + [_vp] * 7,
    "gdn_commit_replay": [ctypes.POINTER(GdnShape), _vp, ctypes.c_int32] + [_vp] * 10,
    "gdn_replay_verify_chain": [ctypes.POINTER(GdnShape)] + [_vp] * 18,
    "gdn_conv_commit": [ctypes.POINTER(GdnConvShape), _vp, ctypes.c_int32] + [_vp] * 6,
    "gdn_commit_index": [_vp, _vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp, _vp],
    "gdn_status_string": [ctypes.c_int],
    "gdn_tree_walk": [_vp, ctypes.c_int32, _vp, _vp],
    "gdn_prefill_workspace_bytes": [ctypes.POINTER(GdnShape)],
    "gdn_prefill_chunked": [ctypes.POINTER(GdnShape)] + [_vp] * 9 + [ctypes.c_size_t, _vp, _vp],
    "gdn_prefill_varlen_workspace_bytes": [ctypes.POINTER(GdnShape), _vp],
    "gdn_prefill_boundary_states": [_vp, ctypes.c_int32, ctypes.c_int32],
    "gdn_prefill_varlen": [ctypes.POINTER(GdnShape)] + [_vp] * 10 + [ctypes.c_int32, _vp, ctypes.c_size_t, _vp, _vp],
}


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(_LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = {"gdn_status_string": ctypes.c_char_p,
                          "gdn_prefill_workspace_bytes": ctypes.c_size_t,
                          "gdn_prefill_varlen_workspace_bytes": ctypes.c_size_t,
                          "gdn_prefill_boundary_states": ctypes.c_int64}.get(name, ctypes.c_int)
        _lib = L
    return _lib


def library_path() -> str:
    return _LIB_PATH


def gdn_status_string(code: int) -> str:
    return lib().gdn_status_string(int(code)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return GDN_F32
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float16:
        return GDN_F16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev_ptr(t, name: str):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise GdnError(rc, what)


def _verify_shape(q, v, state, out, persist, scale) -> GdnShape:
    B, N, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    return GdnShape(B, N, Hqk, Hv, dk, dv, state.shape[0], _dtype_code(q),
                    _dtype_code(out) if out is not None else GDN_F32,
                    _dtype_code(persist) if persist is not None else GDN_F16, float(scale))


def gdn_verify_chain(q, k, v, alpha, beta, state, *, out=None, persist=None, final_state=None,
                     state_slot=None, status=None, scale: float = 1.0, stream=None) -> None:
    """Chain verify; see include/gdn.h.  Outputs are caller-allocated tensors."""
    sh = _verify_shape(q, v, state, out, persist, scale)
    rc = lib().gdn_verify_chain(ctypes.byref(sh), _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                _dev_ptr(alpha, "alpha"), _dev_ptr(beta, "beta"), _dev_ptr(state, "state"),
                                _dev_ptr(state_slot, "state_slot"), _dev_ptr(out, "out"),
                                _dev_ptr(persist, "persist"), _dev_ptr(final_state, "final_state"),
                                _dev_ptr(status, "status"), _stream(stream))
    _check(rc, "gdn_verify_chain")


def gdn_commit_verify_chain(accepted_prev, persist_prev, q, k, v, alpha, beta, state, *, final_prev=None,
                            out=None, persist=None, final_state=None, state_slot=None, status=None,
                            scale: float = 1.0, stream=None) -> None:
    """Commit the previous step's accepted node and verify the next chain, in one launch."""
    sh = _verify_shape(q, v, state, out, persist if persist is not None else persist_prev, scale)
    rc = lib().gdn_commit_verify_chain(ctypes.byref(sh), _dev_ptr(accepted_prev, "accepted_prev"),
                                       _dev_ptr(persist_prev, "persist_prev"), _dev_ptr(final_prev, "final_prev"),
                                       _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                       _dev_ptr(alpha, "alpha"), _dev_ptr(beta, "beta"), _dev_ptr(state, "state"),
                                       _dev_ptr(state_slot, "state_slot"), _dev_ptr(out, "out"),
                                       _dev_ptr(persist, "persist"), _dev_ptr(final_state, "final_state"),
                                       _dev_ptr(status, "status"), _stream(stream))
    _check(rc, "gdn_commit_verify_chain")


def _host_parent(parent) -> np.ndarray:
    if isinstance(parent, torch.Tensor):
        parent = parent.detach().cpu().numpy()
    return np.ascontiguousarray(parent, dtype=np.int32)


def gdn_verify_tree(parent, q, k, v, alpha, beta, state, *, out=None, persist=None, state_slot=None,
                    status=None, scale: float = 1.0, stream=None) -> None:
    """Tree verify; ``parent`` is a host array [N] (shared) or [B][N]."""
    sh = _verify_shape(q, v, state, out, persist, scale)
    par = _host_parent(parent)
    n_trees = 1 if par.ndim == 1 else par.shape[0]
    rc = lib().gdn_verify_tree(ctypes.byref(sh), par.ctypes.data, n_trees, _dev_ptr(q, "q"),
                               _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dev_ptr(alpha, "alpha"),
                               _dev_ptr(beta, "beta"), _dev_ptr(state, "state"),
                               _dev_ptr(state_slot, "state_slot"), _dev_ptr(out, "out"),
                               _dev_ptr(persist, "persist"), _dev_ptr(status, "status"), _stream(stream))
    _check(rc, "gdn_verify_tree")


def gdn_tree_walk(parent):
    """(walk uint16[N], fork_slots) for one host parent array."""
    par = _host_parent(parent)
    walk = np.zeros(max(par.size, 1), dtype=np.uint16)
    slots = ctypes.c_int32(0)
    rc = lib().gdn_tree_walk(par.ctypes.data, par.size, walk.ctypes.data, ctypes.byref(slots))
    _check(rc, "gdn_tree_walk")
    return walk[:par.size], slots.value


def gdn_commit(accepted_node, persist, state, *, final_state=None, state_slot=None, status=None,
               stream=None) -> None:
    """Commit; persist is [B][N][Hv][dv][dk] (f16 or fp32), state [slots][Hv][dv][dk]."""
    B, N, Hv, dv, dk = persist.shape
    sh = GdnShape(B, N, 1, Hv, dk, dv, state.shape[0], GDN_BF16, GDN_F32, _dtype_code(persist), 1.0)
    rc = lib().gdn_commit(ctypes.byref(sh), _dev_ptr(accepted_node, "accepted_node"),
                          _dev_ptr(persist, "persist"), _dev_ptr(final_state, "final_state"),
                          _dev_ptr(state, "state"), _dev_ptr(state_slot, "state_slot"),
                          _dev_ptr(status, "status"), _stream(stream))
    _check(rc, "gdn_commit")


def gdn_commit_replay(accepted_node, q, k, v, alpha, beta, state, *, parent=None, state_slot=None, status=None,
                      stream=None) -> None:
    """Commit by replay: state[slot(b)] <- the state after node accepted_node[b],
    re-run from state[slot(b)] over the node's root path (chain when ``parent``
    is None; else a host parent array [N] or [B][N])."""
    sh = _verify_shape(q, v, state, None, None, 1.0)
    par, n_trees = None, 0
    if parent is not None:
        par = _host_parent(parent)
        n_trees = 1 if par.ndim == 1 else par.shape[0]
    rc = lib().gdn_commit_replay(ctypes.byref(sh), par.ctypes.data if par is not None else None, n_trees,
                                 _dev_ptr(accepted_node, "accepted_node"), _dev_ptr(q, "q"), _dev_ptr(k, "k"),
                                 _dev_ptr(v, "v"), _dev_ptr(alpha, "alpha"), _dev_ptr(beta, "beta"),
                                 _dev_ptr(state, "state"), _dev_ptr(state_slot, "state_slot"),
                                 _dev_ptr(status, "status"), _stream(stream))
    _check(rc, "gdn_commit_replay")


def gdn_replay_verify_chain(accepted_prev, q_prev, k_prev, v_prev, alpha_prev, beta_prev, q, k, v, alpha, beta,
                            state, *, out=None, persist=None, final_state=None, state_slot=None, status=None,
                            scale: float = 1.0, stream=None) -> None:
    """Commit the previous chain block by replay and verify the next one, in one launch."""
    sh = _verify_shape(q, v, state, out, persist, scale)
    rc = lib().gdn_replay_verify_chain(ctypes.byref(sh), _dev_ptr(accepted_prev, "accepted_prev"),
                                       _dev_ptr(q_prev, "q_prev"), _dev_ptr(k_prev, "k_prev"),
                                       _dev_ptr(v_prev, "v_prev"), _dev_ptr(alpha_prev, "alpha_prev"),
                                       _dev_ptr(beta_prev, "beta_prev"), _dev_ptr(q, "q"), _dev_ptr(k, "k"),
                                       _dev_ptr(v, "v"), _dev_ptr(alpha, "alpha"), _dev_ptr(beta, "beta"),
                                       _dev_ptr(state, "state"), _dev_ptr(state_slot, "state_slot"),
                                       _dev_ptr(out, "out"), _dev_ptr(persist, "persist"),
                                       _dev_ptr(final_state, "final_state"), _dev_ptr(status, "status"),
                                       _stream(stream))
    _check(rc, "gdn_replay_verify_chain")


def gdn_commit_index(accepted_node, state_slot, n_nodes: int, draft_row0: int, n_slots: int, *, status=None,
                     stream=None) -> None:
    """Index-table commit: state_slot[b] <- draft_row0 + b * n_nodes + accepted_node[b] (device arrays)."""
    B = state_slot.shape[0]
    rc = lib().gdn_commit_index(_dev_ptr(accepted_node, "accepted_node"), _dev_ptr(state_slot, "state_slot"), B,
                                int(n_nodes), int(draft_row0), int(n_slots), _dev_ptr(status, "status"),
                                _stream(stream))
    _check(rc, "gdn_commit_index")


def gdn_conv_commit(accepted_node, x, conv_state, *, parent=None, state_slot=None, status=None,
                    stream=None) -> None:
    """Commit the convolution history: conv_state [slots][W-1][C] <- the last
    W-1 rows of (history, inputs x [B][N][C] along the accepted node's root
    path); chain when ``parent`` is None, else a host array [N] or [B][N]."""
    B, N, C = x.shape
    if conv_state.dtype != x.dtype:
        raise TypeError("conv_state and x must have one dtype")
    sh = GdnConvShape(B, N, C, conv_state.shape[1] + 1, conv_state.shape[0], _dtype_code(x))
    par, n_trees = None, 0
    if parent is not None:
        par = _host_parent(parent)
        n_trees = 1 if par.ndim == 1 else par.shape[0]
    rc = lib().gdn_conv_commit(ctypes.byref(sh), par.ctypes.data if par is not None else None, n_trees,
                               _dev_ptr(accepted_node, "accepted_node"), _dev_ptr(x, "x"),
                               _dev_ptr(conv_state, "conv_state"), _dev_ptr(state_slot, "state_slot"),
                               _dev_ptr(status, "status"), _stream(stream))
    _check(rc, "gdn_conv_commit")


def _prefill_shape(q, v, state, out, scale) -> GdnShape:
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    return GdnShape(B, T, Hqk, Hv, dk, dv, state.shape[0], _dtype_code(q), _dtype_code(out), GDN_F16,
                    float(scale))


def gdn_prefill_workspace_bytes(q, v, state, out, scale: float = 1.0) -> int:
    sh = _prefill_shape(q, v, state, out, scale)
    return int(lib().gdn_prefill_workspace_bytes(ctypes.byref(sh)))


def gdn_prefill_chunked(q, k, v, alpha, beta, state, out, *, state_slot=None, status=None, workspace=None,
                        scale: float = 1.0, stream=None) -> None:
    """Chunked prefill; ``state`` is updated in place (see include/gdn.h).

    ``workspace`` is a device tensor of at least gdn_prefill_workspace_bytes
    bytes; when omitted one is allocated here with torch (plumbing only).
    """
    sh = _prefill_shape(q, v, state, out, scale)
    if workspace is None:
        need = int(lib().gdn_prefill_workspace_bytes(ctypes.byref(sh)))
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().gdn_prefill_chunked(ctypes.byref(sh), _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                   _dev_ptr(alpha, "alpha"), _dev_ptr(beta, "beta"), _dev_ptr(state, "state"),
                                   _dev_ptr(state_slot, "state_slot"), _dev_ptr(out, "out"),
                                   _dev_ptr(workspace, "workspace"), ws_bytes, _dev_ptr(status, "status"),
                                   _stream(stream))
    _check(rc, "gdn_prefill_chunked")


def _host_cu(cu_seqlens) -> np.ndarray:
    if isinstance(cu_seqlens, torch.Tensor):
        cu_seqlens = cu_seqlens.detach().cpu().numpy()
    return np.ascontiguousarray(cu_seqlens, dtype=np.int32)


def gdn_prefill_boundary_states(cu_seqlens, state_interval: int) -> int:
    cu = _host_cu(cu_seqlens)
    return int(lib().gdn_prefill_boundary_states(cu.ctypes.data, cu.size - 1, int(state_interval)))


def gdn_prefill_varlen_workspace_bytes(cu_seqlens, q, v, state, out, scale: float = 1.0) -> int:
    cu = _host_cu(cu_seqlens)
    total, Hqk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    sh = GdnShape(cu.size - 1, total, Hqk, Hv, dk, dv, state.shape[0], _dtype_code(q), _dtype_code(out), GDN_F16,
                  float(scale))
    return int(lib().gdn_prefill_varlen_workspace_bytes(ctypes.byref(sh), cu.ctypes.data))


def gdn_prefill_varlen(cu_seqlens, q, k, v, alpha, beta, state, out, *, chunk_states=None, state_interval: int = 1,
                       state_slot=None, status=None, workspace=None, scale: float = 1.0, stream=None) -> None:
    """Varlen prefill of sequences packed along the token dimension (q [total][h_qk][d_k], ...);
    ``cu_seqlens`` is a host array [B + 1]; see include/gdn.h."""
    cu = _host_cu(cu_seqlens)
    total, Hqk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    sh = GdnShape(cu.size - 1, total, Hqk, Hv, dk, dv, state.shape[0], _dtype_code(q), _dtype_code(out), GDN_F16,
                  float(scale))
    if workspace is None:
        need = int(lib().gdn_prefill_varlen_workspace_bytes(ctypes.byref(sh), cu.ctypes.data))
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    rc = lib().gdn_prefill_varlen(ctypes.byref(sh), cu.ctypes.data, _dev_ptr(q, "q"), _dev_ptr(k, "k"),
                                  _dev_ptr(v, "v"), _dev_ptr(alpha, "alpha"), _dev_ptr(beta, "beta"),
                                  _dev_ptr(state, "state"), _dev_ptr(state_slot, "state_slot"), _dev_ptr(out, "out"),
                                  _dev_ptr(chunk_states, "chunk_states"), int(state_interval),
                                  _dev_ptr(workspace, "workspace"), ws_bytes, _dev_ptr(status, "status"),
                                  _stream(stream))
    _check(rc, "gdn_prefill_varlen")
