"""ctypes wrapper of the CPU oracle (oracle/vrt_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library. See vrt_oracle.h for what
each routine follows on the RheoSampling and SMART pages.
"""
import contextlib
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

ROOT, DET, PROBE, FILL = 0, 1, 2, 3
TOPR, SMART = 0, 1
MAXSUP = 1024


class Cfg(ctypes.Structure):
    _fields_ = [
        ("V", ctypes.c_int32), ("trunc", ctypes.c_int32), ("K", ctypes.c_int32),
        ("m", ctypes.c_int32), ("probe", ctypes.c_int32), ("D", ctypes.c_int32),
        ("W", ctypes.c_int32), ("R", ctypes.c_int32), ("mode", ctypes.c_int32),
        ("budget", ctypes.c_int32), ("T", ctypes.c_float), ("eps_m0", ctypes.c_float),
        ("alpha", ctypes.c_double), ("lambda_", ctypes.c_double), ("gamma_", ctypes.c_double),
        ("delta_", ctypes.c_double), ("rho_", ctypes.c_double), ("order", ctypes.c_int32),
    ]


class Cand(ctypes.Structure):
    _fields_ = [("token", ctypes.c_int32), ("parent", ctypes.c_int32), ("depth", ctypes.c_int32),
                ("kind", ctypes.c_int32), ("slot", ctypes.c_int32), ("row", ctypes.c_int32),
                ("live", ctypes.c_int32), ("score", ctypes.c_float)]


class Exp(ctypes.Structure):
    _fields_ = [("node", ctypes.c_int32), ("n_sup", ctypes.c_int32),
                ("probe_rank", ctypes.c_int32), ("n_child", ctypes.c_int32),
                ("exempt", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("sup_id", ctypes.c_int32 * MAXSUP), ("sup_logit", ctypes.c_float * MAXSUP),
                ("q_raw", ctypes.c_float * MAXSUP), ("q_T", ctypes.c_double * MAXSUP),
                ("z_raw", ctypes.c_float), ("proxy", ctypes.c_float),
                ("z_T", ctypes.c_double), ("u", ctypes.c_double),
                ("probe_token", ctypes.c_int32), ("dense_q", ctypes.c_void_p)]


class NodeOut(ctypes.Structure):
    _fields_ = [("accept", ctypes.c_int32), ("token", ctypes.c_int32),
                ("exempt", ctypes.c_int32), ("n_tests", ctypes.c_int32), ("W", ctypes.c_double)]


_lib = None


def load(path):
    L = ctypes.CDLL(path)
    _declare(L)
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build()
        _lib = load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def using(path):
    """Temporarily route every call to another build of the oracle (mutation tests)."""
    global _lib
    old = lib()
    _lib = load(path)
    try:
        yield
    finally:
        _lib = old


def _declare(L):
    P = ctypes.POINTER
    i32, u32, u64, f32, f64 = ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_float, ctypes.c_double
    vp = ctypes.c_void_p
    L.orc_philox.argtypes = [P(u32), P(u32), P(u32)]
    L.orc_uniform.argtypes = [u64, u32, u32, u32, u32]
    L.orc_uniform.restype = f64
    L.orc_exp_rank.argtypes = [f32]
    L.orc_exp_rank.restype = f32
    L.orc_exp_rank_array.argtypes = [vp, vp, ctypes.c_int64]
    L.orc_pairwise128.argtypes = [vp]
    L.orc_pairwise128.restype = f32
    L.orc_support.argtypes = [vp, i32, i32, vp, vp]
    L.orc_support.restype = i32
    L.orc_support_mass.argtypes = [vp, i32, i32]
    L.orc_support_mass.restype = ctypes.c_double
    L.orc_tree_create.argtypes = [P(Cfg), u64, i32, u32]
    L.orc_tree_create.restype = vp
    L.orc_tree_free.argtypes = [vp]
    L.orc_expand_layer.argtypes = [vp, i32, vp, ctypes.c_int64]
    L.orc_expand_layer.restype = i32
    L.orc_frontier.argtypes = [vp, vp]
    L.orc_frontier.restype = i32
    L.orc_finish.argtypes = [vp]
    L.orc_finish.restype = i32
    L.orc_n_cand.argtypes = [vp]
    L.orc_n_cand.restype = i32
    L.orc_cands.argtypes = [vp]
    L.orc_cands.restype = P(Cand)
    L.orc_n_rows.argtypes = [vp]
    L.orc_n_rows.restype = i32
    L.orc_row.argtypes = [vp, i32]
    L.orc_row.restype = P(Exp)
    L.orc_layer_base.argtypes = [vp, i32]
    L.orc_layer_base.restype = i32
    L.orc_row_base.argtypes = [vp, i32]
    L.orc_row_base.restype = i32
    L.orc_n_exempt.argtypes = [vp]
    L.orc_n_exempt.restype = i32
    L.orc_flags.argtypes = [vp]
    L.orc_flags.restype = i32
    L.orc_tree_view.argtypes = [vp, i32, i32] + [vp] * 11
    L.orc_tree_view.restype = i32
    L.orc_verify.argtypes = [P(Cfg), i32] + [vp] * 9 + [i32, vp, ctypes.c_int64, u64, i32, u32,
                                                      vp, vp, vp, vp]
    L.orc_verify.restype = i32
    L.orc_table_trials.argtypes = [P(Cfg), i32, vp, vp, u64, i32, u32, i32, i32, vp, vp, vp]
    L.orc_table_trials.restype = i32
    L.orc_exact_law.argtypes = [P(Cfg), i32, vp, vp, vp, i32, i32, vp, vp, P(f64)]
    L.orc_exact_law.restype = i32
    L.orc_tree_mask.argtypes = [i32, vp, vp, vp]
    L.orc_tree_mask.restype = i32
    L.orc_accepted_kv.argtypes = [i32, vp, vp]
    L.orc_accepted_kv.restype = i32


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


PROBE_FIRST, PROBE_LAST = 0, 1
DENSE = 0  # trunc value: no truncation (the support is the whole vocabulary)


def make_cfg(V, trunc=128, K=8, m=1, probe=1, D=8, W=0, R=60, mode=TOPR, budget=128, T=1.0,
             eps_m0=1e-6, alpha=1.0, lam=0.0, gamma=0.0, delta=0.0, rho=1.0, order=PROBE_FIRST):
    return Cfg(V, trunc, K, m, probe, D, W, R, mode, budget, T, eps_m0, alpha, lam, gamma, delta, rho,
               order)


def philox(ctr, key):
    c = (ctypes.c_uint32 * 4)(*ctr)
    k = (ctypes.c_uint32 * 2)(*key)
    o = (ctypes.c_uint32 * 4)()
    lib().orc_philox(c, k, o)
    return tuple(o)


def uniform(seed, idx, b, step, purpose):
    return lib().orc_uniform(seed, idx, b, step, purpose)


def exp_rank(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty_like(x)
    lib().orc_exp_rank_array(_p(x), _p(y), x.size)
    return y


def pairwise128(v):
    v = np.ascontiguousarray(v, dtype=np.float32)
    assert v.size == 128
    return lib().orc_pairwise128(_p(v))


def support(row, trunc=128):
    row = np.ascontiguousarray(row, dtype=np.float32)
    ids = np.empty(trunc, np.int32)
    vals = np.empty(trunc, np.float32)
    n = lib().orc_support(_p(row), row.size, trunc, _p(ids), _p(vals))
    return ids[:n].copy(), vals[:n].copy()


def support_mass(row, trunc=128):
    """Share of the untempered softmax of `row` held by its min(trunc, V) largest logits."""
    row = np.ascontiguousarray(row, dtype=np.float32)
    return lib().orc_support_mass(_p(row), row.size, trunc)


class Tree:
    """One draft tree of the oracle, built layer by layer."""

    def __init__(self, cfg, seed, b, step):
        self.cfg = cfg
        self.L = lib()
        self.h = self.L.orc_tree_create(ctypes.byref(cfg), seed, b, step)

    def __del__(self):
        if getattr(self, "h", None):
            self.L.orc_tree_free(self.h)
            self.h = None

    def expand_layer(self, layer, rows):
        rows = np.ascontiguousarray(rows, dtype=np.float32)
        return self.L.orc_expand_layer(self.h, layer, _p(rows), rows.shape[-1])

    def frontier(self):
        out = np.empty(max(self.cfg.budget, self.cfg.W, self.cfg.K) + 1, np.int32)
        n = self.L.orc_frontier(self.h, _p(out))
        return out[:n].copy()

    def finish(self):
        return self.L.orc_finish(self.h)

    def cands(self):
        n = self.L.orc_n_cand(self.h)
        ptr = self.L.orc_cands(self.h)
        arr = np.ctypeslib.as_array((Cand * n).from_address(ctypes.addressof(ptr.contents)))
        return np.array(arr.tolist(), dtype=[("token", "i4"), ("parent", "i4"), ("depth", "i4"),
                                             ("kind", "i4"), ("slot", "i4"), ("row", "i4"),
                                             ("live", "i4"), ("score", "f4")])

    def n_rows(self):
        return self.L.orc_n_rows(self.h)

    def row(self, r):
        return self.L.orc_row(self.h, r).contents

    def layer_base(self, layer):
        return self.L.orc_layer_base(self.h, layer)

    def row_base(self, layer):
        return self.L.orc_row_base(self.h, layer)

    def n_exempt(self):
        return self.L.orc_n_exempt(self.h)

    def flags(self):
        return self.L.orc_flags(self.h)

    def view(self):
        """Verification view: dict of arrays (node 0 = root)."""
        cap = self.L.orc_n_cand(self.h) + 1
        tc = self.cfg.trunc if self.cfg.trunc != DENSE else self.cfg.V
        d = {k: np.zeros(cap, np.int32) for k in ("token", "parent", "depth", "kind", "cand", "tail_n")}
        d["child_off"] = np.zeros(cap + 1, np.int32)
        d["child"] = np.zeros(cap, np.int32)
        d["tail_id"] = np.zeros(cap * tc, np.int32)
        d["tail_q"] = np.zeros(cap * tc, np.float64)
        nn = ctypes.c_int32()
        r = self.L.orc_tree_view(self.h, cap, tc, ctypes.byref(nn), _p(d["token"]), _p(d["parent"]),
                                _p(d["depth"]), _p(d["kind"]), _p(d["cand"]), _p(d["child_off"]),
                                _p(d["child"]), _p(d["tail_n"]), _p(d["tail_id"]), _p(d["tail_q"]))
        assert r >= 0, r
        n = nn.value
        out = {k: d[k][:n].copy() for k in ("token", "parent", "depth", "kind", "cand", "tail_n")}
        out["child_off"] = d["child_off"][:n + 1].copy()
        out["child"] = d["child"][:out["child_off"][-1]].copy()
        out["tail_id"] = d["tail_id"][:n * tc].reshape(n, tc).copy()
        out["tail_q"] = d["tail_q"][:n * tc].reshape(n, tc).copy()
        out["n_nodes"] = n
        return out


def verify(cfg, view, target, seed, b, step):
    """Verify one tree against its target rows [n_nodes, V] (float32).

    Returns (tokens, nodes, per_node, exempt) where per_node is a structured
    array of the per-node outcomes."""
    n = view["n_nodes"]
    target = np.ascontiguousarray(target, dtype=np.float32)
    assert target.shape[0] >= n
    tc = view["tail_id"].shape[1]
    tail_id = np.ascontiguousarray(view["tail_id"], dtype=np.int32)
    tail_q = np.ascontiguousarray(view["tail_q"], dtype=np.float64)
    out_tok = np.full(64, -1, np.int32)
    out_nodes = np.full(64, -1, np.int32)
    out_len = ctypes.c_int32()
    per = (NodeOut * n)()
    iv = {k: np.ascontiguousarray(view[k], dtype=np.int32)
          for k in ("token", "parent", "depth", "kind", "child_off", "child", "tail_n")}
    if iv["child"].size == 0:
        iv["child"] = np.zeros(1, np.int32)
    ex = lib().orc_verify(ctypes.byref(cfg), n, _p(iv["token"]), _p(iv["parent"]), _p(iv["depth"]),
                          _p(iv["kind"]), _p(iv["child_off"]), _p(iv["child"]), _p(iv["tail_n"]),
                          _p(tail_id), _p(tail_q), tc, _p(target), target.shape[-1], seed, b, step,
                          _p(out_tok), _p(out_nodes), ctypes.byref(out_len), per)
    L = out_len.value
    pn = np.array([(p.accept, p.token, p.exempt, p.n_tests, p.W) for p in per],
                  dtype=[("accept", "i4"), ("token", "i4"), ("exempt", "i4"), ("n_tests", "i4"),
                         ("W", "f8")])
    return out_tok[:L].copy(), out_nodes[:L - 1].copy(), pn, ex


def table_trials(cfg, max_len, draft_tab, target_tab, seed, b, step0, n_trials, two=False):
    """Run repeated steps on a context-table model (see vrt_oracle.c)."""
    dt = np.ascontiguousarray(draft_tab, dtype=np.float32)
    tt = np.ascontiguousarray(target_tab, dtype=np.float32)
    out = np.full(2 * n_trials, -1, np.int32)
    nf = np.zeros(n_trials, np.int32)
    ne = ctypes.c_int32()
    r = lib().orc_table_trials(ctypes.byref(cfg), max_len, _p(dt), _p(tt), seed, b, step0, n_trials,
                               1 if two else 0, _p(out), _p(nf), ctypes.byref(ne))
    assert r == 0, "context table too short for the tree depth"
    return out.reshape(n_trials, 2), nf, ne.value


def exact_law(cfg, max_len, draft_tab, target_tab, prefix=(), two=True):
    """Exact laws of one step on a context-table model by enumeration (orc_exact_law):
    (law1 [V], law2 [V, V] or None, P(first token from the tree))."""
    V = cfg.V
    dt = np.ascontiguousarray(draft_tab, dtype=np.float32)
    tt = np.ascontiguousarray(target_tab, dtype=np.float32)
    pre = np.ascontiguousarray(list(prefix) or [0], dtype=np.int32)
    law1 = np.zeros(V, np.float64)
    law2 = np.zeros(V * V, np.float64)
    acc = ctypes.c_double()
    r = lib().orc_exact_law(ctypes.byref(cfg), max_len, _p(dt), _p(tt), _p(pre), len(prefix),
                            1 if two else 0, _p(law1), _p(law2), ctypes.byref(acc))
    assert r == 0, f"orc_exact_law returned {r}"
    return law1, (law2.reshape(V, V) if two else None), acc.value


def ctx_index(V, path):
    """Row of context path (t_1..t_k) in a context table."""
    k = len(path)
    off = sum(V ** i for i in range(k))
    pos = 0
    for t in path:
        pos = pos * V + int(t)
    return off + pos


def tree_mask(parent):
    """(mask bool [n, n], pos i32 [n]) of an emitted tree given its parent array, or None
    if a parent is out of range (orc_tree_mask)."""
    parent = np.ascontiguousarray(parent, np.int32)
    n = parent.size
    mask = np.zeros((n, n), np.uint8)
    pos = np.zeros(n, np.int32)
    if lib().orc_tree_mask(n, _p(parent), _p(mask), _p(pos)) != 0:
        return None
    return mask.astype(bool), pos


def accepted_kv(out_len, out_nodes):
    """KV entries kept after verification (orc_accepted_kv): root, then accepted nodes."""
    nodes = np.ascontiguousarray(out_nodes, np.int32)
    keep = np.zeros(max(int(out_len), 1), np.int32)
    n = lib().orc_accepted_kv(int(out_len), _p(nodes), _p(keep))
    return keep[:n]
