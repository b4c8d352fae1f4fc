"""The C ABI on the host: the library loads, exports what include/gdn.h
declares, and rejects bad requests before any HIP call (no GPU needed: every
call here fails host validation or has batch 0, so nothing is launched)."""
import ctypes
import os
import re

import numpy as np
import pytest

from gated_deltanet_recurrence_gdn_amd import binding as gb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h")]

FAKE = 0x10000  # a 16-byte aligned non-null address; never dereferenced here


def declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(gdn_\w+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    L = gb.lib()
    names = declared_functions()
    assert "gdn_verify_chain" in names and "gdn_commit" in names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for code, name in gb.STATUS.items():
        s = gb.gdn_status_string(code)
        assert isinstance(s, str) and s
    assert gb.gdn_status_string(0) == "ok"
    assert gb.gdn_status_string(12345) == "unknown status"


def shape(**kw):
    d = dict(batch=1, n_nodes=16, h_qk=16, h_v=48, d_k=128, d_v=128, n_slots=1, qkv_dtype=gb.GDN_BF16,
             out_dtype=gb.GDN_F32, persist_dtype=gb.GDN_F16, scale=1.0)
    d.update(kw)
    return gb.GdnShape(*[d[f] for f, _ in gb.GdnShape._fields_])


def chain(sh, q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE, st=FAKE, slot=None, out=FAKE, per=FAKE, fin=None):
    return gb.lib().gdn_verify_chain(ctypes.byref(sh) if sh is not None else None, q, k, v, a, b, st, slot,
                                     out, per, fin, None, None)


def tree(sh, parent, n_trees=1, q=FAKE):
    par = np.ascontiguousarray(parent, dtype=np.int32)
    return gb.lib().gdn_verify_tree(ctypes.byref(sh), par.ctypes.data if par.size else None, n_trees, q, FAKE,
                                    FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None)


E = gb.CODES


@pytest.mark.parametrize("kw,code", [
    (dict(n_nodes=0), "GDN_ERR_SHAPE"),
    (dict(n_nodes=33), "GDN_ERR_SHAPE"),
    (dict(batch=-1), "GDN_ERR_SHAPE"),
    (dict(h_v=47), "GDN_ERR_SHAPE"),
    (dict(h_qk=0), "GDN_ERR_SHAPE"),
    (dict(d_k=96), "GDN_ERR_SHAPE"),
    (dict(d_v=24), "GDN_ERR_SHAPE"),
    (dict(d_v=512), "GDN_ERR_SHAPE"),
    (dict(qkv_dtype=gb.GDN_F16), "GDN_ERR_DTYPE"),
    (dict(qkv_dtype=7), "GDN_ERR_DTYPE"),
    (dict(persist_dtype=gb.GDN_BF16), "GDN_ERR_DTYPE"),
    (dict(scale=float("nan")), "GDN_ERR_SHAPE"),
    (dict(h_v=8192, h_qk=16), "GDN_ERR_SHAPE"),  # per-node persist offsets would pass 2^32
])
def test_verify_chain_rejects_bad_shapes(kw, code):
    assert chain(shape(**kw)) == E[code]


def test_verify_chain_rejects_null_and_misaligned():
    assert chain(None) == E["GDN_ERR_NULL"]
    assert chain(shape(), q=None) == E["GDN_ERR_NULL"]
    assert chain(shape(), st=None) == E["GDN_ERR_NULL"]
    assert chain(shape(), q=FAKE + 2) == E["GDN_ERR_ALIGN"]
    assert chain(shape(), per=FAKE + 8) == E["GDN_ERR_ALIGN"]
    assert chain(shape(), a=FAKE + 2) == E["GDN_ERR_ALIGN"]
    assert chain(shape(n_slots=0), slot=FAKE) == E["GDN_ERR_SHAPE"]
    # in-place final state needs the identity slot map
    assert chain(shape(), slot=FAKE, fin=FAKE) == E["GDN_ERR_SHAPE"]


def test_batch_zero_is_a_no_op():
    assert chain(shape(batch=0), q=None, k=None, v=None, a=None, b=None, st=None) == 0
    assert tree(shape(batch=0, n_nodes=3), [-1, 0, 0]) == 0


@pytest.mark.parametrize("parent", [
    [0, 0, 1],            # root must be -1
    [-1, 1, 0],           # parent[1] must be < 1
    [-1, 0, 3, 1],        # parent after child
    [-1, -1, 0],          # second root
    [-1, 0, -2],          # negative
    [-1] + list(range(16)),  # 17 nodes deep
])
def test_verify_tree_rejects_bad_parents(parent):
    assert tree(shape(n_nodes=len(parent)), parent) == E["GDN_ERR_PARENT"]


def test_verify_tree_rejects_bad_tree_count():
    p = np.array([[-1, 0, 0], [-1, 0, 1]], np.int32)
    assert tree(shape(batch=3, n_nodes=3), p, n_trees=2) == E["GDN_ERR_SHAPE"]
    bad = np.array([[-1, 0, 0], [-1, 0, 2], [-1, 0, 1]], np.int32)
    assert tree(shape(batch=3, n_nodes=3), bad, n_trees=3) == E["GDN_ERR_PARENT"]
    assert gb.lib().gdn_verify_tree(ctypes.byref(shape(n_nodes=3)), None, 1, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    FAKE, None, FAKE, FAKE, None, None) == E["GDN_ERR_NULL"]


def test_commit_rejects_bad_requests():
    L = gb.lib()
    c = lambda sh, acc=FAKE, per=FAKE, fin=None, st=FAKE, slot=None: L.gdn_commit(  # noqa: E731
        ctypes.byref(sh) if sh is not None else None, acc, per, fin, st, slot, None, None)
    assert c(None) == E["GDN_ERR_NULL"]
    assert c(shape(), acc=None) == E["GDN_ERR_NULL"]
    assert c(shape(), per=None) == E["GDN_ERR_NULL"]
    assert c(shape(persist_dtype=gb.GDN_BF16)) == E["GDN_ERR_DTYPE"]
    assert c(shape(n_nodes=40)) == E["GDN_ERR_SHAPE"]
    assert c(shape(), st=FAKE + 4) == E["GDN_ERR_ALIGN"]
    assert c(shape(), acc=FAKE + 1) == E["GDN_ERR_ALIGN"]
    assert c(shape(batch=0), acc=None, per=None, st=None) == 0


def simulate_walk(walk, parent):
    """Replay a walk on symbolic states: each state is the node it came from."""
    cur, slots, seen = -1, {}, []
    for code in walk:
        node = int(code) & 31
        if code & (1 << 5):
            cur = slots[(int(code) >> 6) & 15]
        assert cur == parent[node], (node, cur, parent[node])
        cur = node
        if code & (1 << 10):
            slots[(int(code) >> 11) & 15] = node
        seen.append(node)
    return seen


@pytest.mark.parametrize("seed", range(5))
def test_tree_walk_reaches_every_node_from_its_parent(seed):
    from gated_deltanet_recurrence_gdn_amd import workloads as wl
    rng = np.random.default_rng(seed)
    for n in (1, 2, 5, 22, 32):
        for _ in range(100):
            parent = wl.random_tree(n, 16, rng)
            walk, slots = gb.gdn_tree_walk(parent)
            seen = simulate_walk(walk, parent)
            assert sorted(seen) == list(range(n))
            assert slots <= max(0, wl.tree_depths(parent).max() - 1)


def test_tree_walk_of_a_chain_has_no_forks():
    walk, slots = gb.gdn_tree_walk(np.arange(-1, 15, dtype=np.int32))
    assert slots == 0 and list(walk) == list(range(16))


def test_tree_walk_star_and_deep_fork():
    star = np.array([-1] + [0] * 21, np.int32)
    walk, slots = gb.gdn_tree_walk(star)
    assert slots == 1 and simulate_walk(walk, star) == list(range(22))
    # a 16-deep spine where every spine node also has a leaf: 15 live forks
    par = [-1]
    spine = [0]
    for d in range(1, 16):
        par.append(spine[-1]); spine.append(len(par) - 1)
    for s in spine[:-1]:
        par.append(s)
    par = np.array(par, np.int32)
    walk, slots = gb.gdn_tree_walk(par)
    assert simulate_walk(walk, par) and slots <= 15


def prefill(sh, q=FAKE, out=FAKE, ws=FAKE, ws_bytes=1 << 40, st=FAKE):
    return gb.lib().gdn_prefill_chunked(ctypes.byref(sh) if sh is not None else None, q, FAKE, FAKE, FAKE, FAKE,
                                        st, None, out, ws, ws_bytes, None, None)


def test_prefill_rejects_bad_requests():
    P = dict(n_nodes=4096, d_k=128, d_v=128)
    assert prefill(None) == E["GDN_ERR_NULL"]
    assert prefill(shape(**{**P, "d_v": 48})) == E["GDN_ERR_SHAPE"]
    assert prefill(shape(**{**P, "d_k": 96})) == E["GDN_ERR_SHAPE"]
    assert prefill(shape(**{**P, "h_v": 47})) == E["GDN_ERR_SHAPE"]
    assert prefill(shape(**{**P, "qkv_dtype": gb.GDN_F16})) == E["GDN_ERR_DTYPE"]
    assert prefill(shape(**P), q=None) == E["GDN_ERR_NULL"]
    assert prefill(shape(**P), out=None) == E["GDN_ERR_NULL"]
    assert prefill(shape(**P), q=FAKE + 4) == E["GDN_ERR_ALIGN"]
    assert prefill(shape(**P), out=FAKE + 4) == E["GDN_ERR_ALIGN"]
    assert prefill(shape(**P), ws=None) == E["GDN_ERR_WORKSPACE"]
    sh = shape(**P)
    need = gb.lib().gdn_prefill_workspace_bytes(ctypes.byref(sh))
    # 64 chunks x (48 heads x (T', P) f16 + 48 x 3 x 64 fp32 gates + 16 q/k heads x (K, Q) f16)
    assert need == 64 * (48 * 2 * 64 * 64 * 2 + 48 * 3 * 64 * 4 + 16 * 2 * 128 * 64 * 2)
    assert prefill(sh, ws_bytes=need - 1) == E["GDN_ERR_WORKSPACE"]
    assert prefill(shape(**{**P, "n_nodes": 0}), q=None, ws=None) == 0
    assert prefill(shape(**{**P, "batch": 0}), q=None, ws=None) == 0


def test_fused_commit_verify_rejects_bad_requests():
    L = gb.lib()
    f = lambda sh, acc=FAKE, per_prev=FAKE, fin_prev=None, st=FAKE, fin=None: L.gdn_commit_verify_chain(  # noqa: E731
        ctypes.byref(sh), acc, per_prev, fin_prev, FAKE, FAKE, FAKE, FAKE, FAKE, st, None, FAKE, FAKE, fin, None, None)
    assert f(shape(), acc=None) == E["GDN_ERR_NULL"]
    assert f(shape(), per_prev=None) == E["GDN_ERR_NULL"]
    assert f(shape(), per_prev=FAKE + 8) == E["GDN_ERR_ALIGN"]
    assert f(shape(), acc=FAKE + 2) == E["GDN_ERR_ALIGN"]
    assert f(shape(), fin=FAKE) == E["GDN_ERR_SHAPE"]  # final_state == state
    assert f(shape(d_k=96)) == E["GDN_ERR_SHAPE"]


def test_fused_commit_verify_tree_rejects_bad_requests():
    L = gb.lib()

    def f(sh, parent=(-1, 0, 0), n_trees=1, acc=FAKE, per_prev=FAKE, st=FAKE):
        par = np.ascontiguousarray(parent, dtype=np.int32) if parent is not None else None
        return L.gdn_commit_verify_tree(ctypes.byref(sh), acc, per_prev,
                                        par.ctypes.data if par is not None else None, n_trees, FAKE, FAKE, FAKE,
                                        FAKE, FAKE, st, None, FAKE, FAKE, None, None)
    sh3 = dict(n_nodes=3)
    assert f(shape(**sh3), acc=None) == E["GDN_ERR_NULL"]
    assert f(shape(**sh3), per_prev=None) == E["GDN_ERR_NULL"]
    assert f(shape(**sh3), per_prev=FAKE + 8) == E["GDN_ERR_ALIGN"]
    assert f(shape(**sh3), acc=FAKE + 2) == E["GDN_ERR_ALIGN"]
    assert f(shape(**sh3), st=FAKE + 4) == E["GDN_ERR_ALIGN"]
    assert f(shape(n_nodes=3, d_k=96)) == E["GDN_ERR_SHAPE"]
    assert f(shape(**sh3, persist_dtype=gb.GDN_BF16)) == E["GDN_ERR_DTYPE"]
    # the parent rules of gdn_verify_tree, checked before anything is launched
    assert f(shape(**sh3), parent=None) == E["GDN_ERR_NULL"]
    assert f(shape(**sh3), parent=[0, 0, 1]) == E["GDN_ERR_PARENT"]
    assert f(shape(**sh3), parent=[-1, 0, 2]) == E["GDN_ERR_PARENT"]
    assert f(shape(n_nodes=3, batch=2), parent=[-1, 0, 1] * 3, n_trees=3) == E["GDN_ERR_SHAPE"]
    deep = [-1] + list(range(16))  # 17 nodes on one path
    assert f(shape(n_nodes=17), parent=deep) == E["GDN_ERR_PARENT"]
    # an empty batch validates the tree and launches nothing
    assert f(shape(n_nodes=3, batch=0), acc=None, per_prev=None) == 0
    assert f(shape(n_nodes=3, batch=0), parent=[-1, 0, 2]) == E["GDN_ERR_PARENT"]


def test_commit_replay_rejects_bad_requests():
    L = gb.lib()

    def f(sh, parent=None, n_trees=0, acc=FAKE, q=FAKE, st=FAKE):
        par = np.ascontiguousarray(parent, dtype=np.int32) if parent is not None else None
        return L.gdn_commit_replay(ctypes.byref(sh), par.ctypes.data if par is not None else None, n_trees, acc,
                                   q, FAKE, FAKE, FAKE, FAKE, st, None, None, None)
    assert f(shape(), acc=None) == E["GDN_ERR_NULL"]
    assert f(shape(), acc=FAKE + 2) == E["GDN_ERR_ALIGN"]
    assert f(shape(), q=None) == E["GDN_ERR_NULL"]
    assert f(shape(), st=FAKE + 4) == E["GDN_ERR_ALIGN"]
    assert f(shape(d_k=96)) == E["GDN_ERR_SHAPE"]
    assert f(shape(n_nodes=33)) == E["GDN_ERR_SHAPE"]
    # tree paths: the parent rules of gdn_verify_tree, checked before anything else
    assert f(shape(n_nodes=3), parent=[0, 0, 1], n_trees=1) == E["GDN_ERR_PARENT"]
    assert f(shape(n_nodes=3), parent=[-1, 0, 2], n_trees=1) == E["GDN_ERR_PARENT"]
    assert f(shape(n_nodes=3, batch=2), parent=[-1, 0, 1] * 3, n_trees=3) == E["GDN_ERR_SHAPE"]
    deep = [-1] + list(range(16))  # 17 nodes on one path
    assert f(shape(n_nodes=17), parent=deep, n_trees=1) == E["GDN_ERR_PARENT"]
    assert f(shape(batch=0), acc=None, q=None) == 0


def test_replay_verify_rejects_bad_requests():
    L = gb.lib()

    def f(sh, acc=FAKE, qp=FAKE, ap=FAKE, st=FAKE, fin=None, out=FAKE):
        return L.gdn_replay_verify_chain(ctypes.byref(sh), acc, qp, FAKE, FAKE, ap, FAKE, FAKE, FAKE, FAKE, FAKE,
                                         FAKE, st, None, out, None, fin, None, None)
    assert f(shape(), acc=None) == E["GDN_ERR_NULL"]
    assert f(shape(), qp=None) == E["GDN_ERR_NULL"]
    assert f(shape(), qp=FAKE + 8) == E["GDN_ERR_ALIGN"]
    assert f(shape(), ap=FAKE + 2) == E["GDN_ERR_ALIGN"]
    assert f(shape(), fin=FAKE) == E["GDN_ERR_SHAPE"]  # final_state == state
    assert f(shape(h_v=47)) == E["GDN_ERR_SHAPE"]
    assert f(shape(batch=0), acc=None, qp=None) == 0


def test_conv_commit_rejects_bad_requests():
    L = gb.lib()

    def f(batch=2, n_nodes=16, channels=64, width=4, n_slots=2, dtype=gb.GDN_BF16, parent=None, n_trees=0,
          acc=FAKE, x=FAKE, hist=FAKE, slot=None):
        sh = gb.GdnConvShape(batch, n_nodes, channels, width, n_slots, dtype)
        par = np.ascontiguousarray(parent, dtype=np.int32) if parent is not None else None
        return L.gdn_conv_commit(ctypes.byref(sh), par.ctypes.data if par is not None else None, n_trees, acc, x,
                                 hist, slot, None, None)
    assert L.gdn_conv_commit(None, None, 0, FAKE, FAKE, FAKE, None, None, None) == E["GDN_ERR_NULL"]
    assert f(width=1) == E["GDN_ERR_SHAPE"]
    assert f(width=9) == E["GDN_ERR_SHAPE"]
    assert f(channels=0) == E["GDN_ERR_SHAPE"]
    assert f(channels=12) == E["GDN_ERR_SHAPE"]          # 24 bytes a row: not whole 16-byte pieces
    assert f(n_nodes=0) == E["GDN_ERR_SHAPE"]
    assert f(n_nodes=33) == E["GDN_ERR_SHAPE"]
    assert f(dtype=5) == E["GDN_ERR_DTYPE"]
    assert f(acc=None) == E["GDN_ERR_NULL"]
    assert f(x=FAKE + 8) == E["GDN_ERR_ALIGN"]
    assert f(hist=FAKE + 4) == E["GDN_ERR_ALIGN"]
    assert f(acc=FAKE + 2) == E["GDN_ERR_ALIGN"]
    assert f(slot=FAKE, n_slots=0) == E["GDN_ERR_SHAPE"]
    assert f(n_nodes=3, parent=[-1, 0, 0], n_trees=3) == E["GDN_ERR_SHAPE"]
    assert f(n_nodes=3, parent=[-1, 1, 0], n_trees=1) == E["GDN_ERR_PARENT"]
    assert f(batch=0, acc=None, x=None, hist=None) == 0


def test_commit_index_rejects_bad_requests():
    L = gb.lib()
    f = lambda acc=FAKE, slot=FAKE, B=2, N=16, row0=4, n_slots=36, status=None: L.gdn_commit_index(  # noqa: E731
        acc, slot, B, N, row0, n_slots, status, None)
    assert f(acc=None) == E["GDN_ERR_NULL"]
    assert f(slot=None) == E["GDN_ERR_NULL"]
    assert f(acc=FAKE + 2) == E["GDN_ERR_ALIGN"]
    assert f(status=FAKE + 1) == E["GDN_ERR_ALIGN"]
    assert f(N=0) == E["GDN_ERR_SHAPE"]
    assert f(N=33) == E["GDN_ERR_SHAPE"]
    assert f(row0=-1) == E["GDN_ERR_SHAPE"]
    assert f(n_slots=35) == E["GDN_ERR_SHAPE"]  # the draft region passes the pool
    assert f(B=0, acc=None, slot=None) == 0


def test_prefill_varlen_rejects_bad_requests():
    L = gb.lib()
    P = dict(batch=3, n_nodes=300, h_qk=16, h_v=48, d_k=128, d_v=128, out_dtype=gb.GDN_F16)

    def f(cu, sh=None, cs=None, interval=1, ws=FAKE, ws_bytes=1 << 30, q=FAKE):
        c = np.ascontiguousarray(cu, dtype=np.int32) if cu is not None else None
        return L.gdn_prefill_varlen(ctypes.byref(sh or shape(**P)), c.ctypes.data if c is not None else None, q,
                                    FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, cs, interval, ws, ws_bytes, None, None)
    assert f([0, 100, 200, 300], q=None) == E["GDN_ERR_NULL"]
    assert f(None) == E["GDN_ERR_NULL"]
    assert f([1, 100, 200, 300]) == E["GDN_ERR_SHAPE"]     # does not start at 0
    assert f([0, 100, 90, 300]) == E["GDN_ERR_SHAPE"]      # decreasing
    assert f([0, 100, 200, 299]) == E["GDN_ERR_SHAPE"]     # does not end at the token count
    assert f([0, 100, 200, 300], cs=FAKE, interval=0) == E["GDN_ERR_SHAPE"]
    assert f([0, 100, 200, 300], ws=None) == E["GDN_ERR_WORKSPACE"]
    sh = shape(**P)
    cu = np.array([0, 100, 200, 300], np.int32)
    need = L.gdn_prefill_varlen_workspace_bytes(ctypes.byref(sh), cu.ctypes.data)
    per_unit = 48 * 2 * 64 * 64 * 2 + 48 * 3 * 64 * 4 + 16 * 2 * 128 * 64 * 2
    assert need == 6 * per_unit                            # 2 + 2 + 2 chunk units
    assert f(cu, ws_bytes=need - 1) == E["GDN_ERR_WORKSPACE"]
    assert f([0, 0, 0, 0], sh=shape(**{**P, "n_nodes": 0}), q=None, ws=None) == 0  # no tokens: no-op
    assert f(None, sh=shape(**{**P, "batch": 0}), q=None, ws=None) == 0


def test_prefill_boundary_state_count():
    L = gb.lib()
    cu = np.array([0, 64, 64, 200, 1864, 1865], np.int32)
    assert L.gdn_prefill_boundary_states(cu.ctypes.data, 5, 1) == 1 + 0 + 2 + 26 + 0
    assert L.gdn_prefill_boundary_states(cu.ctypes.data, 5, 2) == 0 + 0 + 1 + 13 + 0
    assert L.gdn_prefill_boundary_states(cu.ctypes.data, 5, 0) == -1
    bad = np.array([0, 10, 5], np.int32)
    assert L.gdn_prefill_boundary_states(bad.ctypes.data, 2, 1) == -1


def test_prefill_noalloc_rejects_heads_beyond_its_array_on_the_host():
    """The no-allocation prefill refuses a request whose single 64-token chunk
    needs more than its static array, before any HIP call; other checks are
    those of gdn_prefill_chunked."""
    L = gb.lib()

    def call(sh, q=FAKE):
        return L.gdn_prefill_chunked_noalloc(ctypes.byref(sh), q, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None)

    P = dict(batch=1, n_nodes=64, h_qk=16, d_k=128, d_v=32)
    assert call(shape(**P, h_v=2048)) == E["GDN_ERR_WORKSPACE"]
    per_unit = L.gdn_prefill_workspace_bytes(ctypes.byref(shape(**{**P, "h_v": 2048})))
    assert per_unit > gb.GDN_PREFILL_SCRATCH_BYTES
    assert call(shape(**P, h_v=48), q=None) == E["GDN_ERR_NULL"]
    assert call(shape(**P, h_v=47)) == E["GDN_ERR_SHAPE"]
    assert call(shape(**{**P, "n_nodes": 0}, h_v=48)) == E["GDN_OK"]
