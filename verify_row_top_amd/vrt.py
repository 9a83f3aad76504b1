"""ctypes binding of libvrt (include/vrt.h): argument marshalling only.

Every entry point keeps the C name without its `vrt_` prefix. Tensors are passed
as raw device pointers; PyTorch only owns the memory and supplies the stream.
Loading fails loudly when libvrt.so is missing or does not load: there is no
fallback path.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libvrt.so")

OK, EINVAL, EDTYPE, ENOMEM, EHIP = 0, -1, -2, -3, -4
F32, BF16 = 0, 1
MODE_TOPR, MODE_SMART = 0, 1
ROOT, DET, PROBE, FILL = 0, 1, 2, 3
FINISH = -1
DENSE = 0  # trunc value: no truncation, the support is the whole vocabulary
ST_DRAFT_NONFINITE, ST_DRAFT_EMPTY, ST_TARGET_BAD = 0x1, 0x2, 0x4
EXPORTS = ("vrt_check_config", "vrt_tree_layout_of", "vrt_tree_bytes", "vrt_workspace_bytes",
           "vrt_build_tree", "vrt_verify_tree", "vrt_verify_tree_static", "vrt_verify_dense", "vrt_verify_lazy", "vrt_verify_nodes", "vrt_verify_walk", "vrt_tree_mask",
           "vrt_accepted_kv", "vrt_support_coverage", "vrt_read_probe", "vrt_last_error")


class VrtError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"vrt error {code}: {msg}")
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "V", "dtype", "trunc", "K", "m", "probe", "D", "W", "R", "mode", "budget")] + \
               [("T", ctypes.c_float), ("eps_m0", ctypes.c_float)] + \
               [(n, ctypes.c_double) for n in ("alpha", "lambda_", "gamma_", "delta_", "rho_")] + \
               [("order", ctypes.c_int32), ("tree_base", ctypes.c_int32)]


class TreeLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "NC", "NR", "N", "TC", "FP", "cand_token", "cand_parent", "cand_score", "cand_kind",
        "row_tail_n", "row_tail_id", "row_tail_q", "front", "n_front", "smart", "admitted", "layer_sync",
        "n_nodes", "node_token", "node_parent", "node_depth", "node_kind", "node_cand",
        "child_off", "child", "tail_n", "tail_id", "tail_q", "row_dense", "row_det", "node_row",
        "row_sync", "smart_cost", "total_bytes")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build()
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, u64, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                                 ctypes.c_size_t)
        P = ctypes.POINTER
        L.vrt_check_config.argtypes = [P(Config)]
        L.vrt_check_config.restype = i32
        L.vrt_tree_layout_of.argtypes = [P(Config), P(TreeLayout)]
        L.vrt_tree_layout_of.restype = i32
        L.vrt_tree_bytes.argtypes = [P(Config)]
        L.vrt_tree_bytes.restype = sz
        L.vrt_workspace_bytes.argtypes = [P(Config)]
        L.vrt_workspace_bytes.restype = sz
        L.vrt_build_tree.argtypes = [P(Config), i32, vp, i64, i64, u64, u64, vp, vp, sz, vp, vp]
        L.vrt_build_tree.restype = i32
        L.vrt_verify_tree.argtypes = [P(Config), vp, i64, i64, vp, u64, u64, vp, sz, vp, vp, vp, vp,
                                      vp, vp]
        L.vrt_verify_tree.restype = i32
        L.vrt_verify_tree_static.argtypes = [P(Config), vp, i64, i64, vp, u64, u64, vp, vp, vp, vp, vp, vp]
        L.vrt_verify_tree_static.restype = i32
        L.vrt_verify_dense.argtypes = [P(Config), vp, i64, i64, vp, i64, i64, vp, u64, u64, vp, sz, vp, vp,
                                       vp, vp, vp, vp]
        L.vrt_verify_dense.restype = i32
        L.vrt_verify_lazy.argtypes = [P(Config), vp, i64, i64, vp, u64, u64, vp, sz, vp, vp, vp, vp,
                                      vp, vp]
        L.vrt_verify_lazy.restype = i32
        L.vrt_verify_nodes.argtypes = [P(Config), vp, i64, i64, vp, u64, u64, vp, sz, vp, vp]
        L.vrt_verify_nodes.restype = i32
        L.vrt_verify_walk.argtypes = [P(Config), vp, vp, sz, vp, vp, vp, vp, vp, vp]
        L.vrt_verify_walk.restype = i32
        L.vrt_tree_mask.argtypes = [P(Config), vp, vp, vp, vp]
        L.vrt_tree_mask.restype = i32
        L.vrt_accepted_kv.argtypes = [P(Config), vp, vp, vp, vp, vp]
        L.vrt_accepted_kv.restype = i32
        L.vrt_support_coverage.argtypes = [P(Config), vp, i64, i64, i32, vp, vp]
        L.vrt_support_coverage.restype = i32
        L.vrt_read_probe.argtypes = [vp, sz, vp, vp]
        L.vrt_read_probe.restype = i32
        L.vrt_last_error.argtypes = []
        L.vrt_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


PROBE_FIRST, PROBE_LAST = 0, 1


def make_config(B, V, dtype=BF16, trunc=128, K=10, m=1, probe=1, D=8, W=0, R=60, mode=MODE_TOPR,
                budget=128, T=1.0, eps_m0=1e-6, alpha=1.0, lam=0.0, gamma=0.0, delta=0.0, rho=1.0,
                order=PROBE_FIRST, tree_base=0):
    return Config(B, V, dtype, trunc, K, m, probe, D, W, R, mode, budget, T, eps_m0, alpha, lam,
                  gamma, delta, rho, order, tree_base)


def last_error():
    return lib().vrt_last_error().decode()


def _check(code):
    if code != OK:
        raise VrtError(code, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(getattr(stream, "cuda_stream", stream))


def check_config(cfg):
    _check(lib().vrt_check_config(ctypes.byref(cfg)))


def tree_layout_of(cfg):
    L = TreeLayout()
    _check(lib().vrt_tree_layout_of(ctypes.byref(cfg), ctypes.byref(L)))
    return L


def tree_bytes(cfg):
    n = lib().vrt_tree_bytes(ctypes.byref(cfg))
    if n == 0:
        raise VrtError(EINVAL, last_error())
    return n


def workspace_bytes(cfg):
    n = lib().vrt_workspace_bytes(ctypes.byref(cfg))
    if n == 0:
        raise VrtError(EINVAL, last_error())
    return n


def build_tree(cfg, layer, draft_logits, ld, tree_stride, seed, step, tree, ws, stats=None,
               stream=None):
    """vrt_build_tree; draft_logits may be None for FINISH."""
    _check(lib().vrt_build_tree(ctypes.byref(cfg), layer, _ptr(draft_logits), ld, tree_stride, seed,
                                step, _ptr(tree), _ptr(ws), ws.numel() * ws.element_size(),
                                _ptr(stats), _stream(stream)))


def verify_tree(cfg, target_logits, ld, tree_stride, tree, seed, step, ws, out_tokens, out_nodes,
                out_len, stats, node_out=None, stream=None):
    """vrt_verify_tree."""
    _check(lib().vrt_verify_tree(ctypes.byref(cfg), _ptr(target_logits), ld, tree_stride, _ptr(tree),
                                 seed, step, _ptr(ws), ws.numel() * ws.element_size(),
                                 _ptr(out_tokens), _ptr(out_nodes), _ptr(out_len), _ptr(stats),
                                 _ptr(node_out), _stream(stream)))


def verify_tree_static(cfg, target_logits, ld, tree_stride, tree, seed, step, out_tokens, out_nodes, out_len,
                       stats, node_out=None, stream=None):
    """vrt_verify_tree_static: vrt_verify_tree on the library's static per-GPU workspace."""
    _check(lib().vrt_verify_tree_static(ctypes.byref(cfg), _ptr(target_logits), ld, tree_stride, _ptr(tree),
                                        seed, step, _ptr(out_tokens), _ptr(out_nodes), _ptr(out_len),
                                        _ptr(stats), _ptr(node_out), _stream(stream)))


def verify_dense(cfg, target_logits, ld, tree_stride, draft_layers, draft_ld, draft_tree_stride, tree, seed,
                 step, ws, out_tokens, out_nodes, out_len, stats, node_out=None, stream=None):
    """vrt_verify_dense: draft_layers is a list of D device tensors, layer l's draft rows as
    passed to build_tree."""
    ptrs = (ctypes.c_void_p * len(draft_layers))(*[t.data_ptr() for t in draft_layers])
    _check(lib().vrt_verify_dense(ctypes.byref(cfg), _ptr(target_logits), ld, tree_stride, ptrs, draft_ld,
                                  draft_tree_stride, _ptr(tree), seed, step, _ptr(ws),
                                  ws.numel() * ws.element_size(), _ptr(out_tokens), _ptr(out_nodes),
                                  _ptr(out_len), _ptr(stats), _ptr(node_out), _stream(stream)))


def verify_lazy(cfg, target_logits, ld, tree_stride, tree, seed, step, ws, out_tokens, out_nodes,
                out_len, stats, node_out=None, stream=None):
    """vrt_verify_lazy: vrt_verify_tree's outputs, deciding only the nodes the walk reaches."""
    _check(lib().vrt_verify_lazy(ctypes.byref(cfg), _ptr(target_logits), ld, tree_stride, _ptr(tree),
                                 seed, step, _ptr(ws), ws.numel() * ws.element_size(),
                                 _ptr(out_tokens), _ptr(out_nodes), _ptr(out_len), _ptr(stats),
                                 _ptr(node_out), _stream(stream)))


def verify_nodes(cfg, target_logits, ld, tree_stride, tree, seed, step, ws, node_out=None, stream=None):
    """vrt_verify_nodes: every node's decision (the first part of vrt_verify_tree)."""
    _check(lib().vrt_verify_nodes(ctypes.byref(cfg), _ptr(target_logits), ld, tree_stride, _ptr(tree),
                                  seed, step, _ptr(ws), ws.numel() * ws.element_size(), _ptr(node_out),
                                  _stream(stream)))


def verify_walk(cfg, tree, ws, out_tokens, out_nodes, out_len, stats, node_out=None, stream=None):
    """vrt_verify_walk: the walk over the decided nodes (the second part of vrt_verify_tree)."""
    _check(lib().vrt_verify_walk(ctypes.byref(cfg), _ptr(tree), _ptr(ws), ws.numel() * ws.element_size(),
                                 _ptr(out_tokens), _ptr(out_nodes), _ptr(out_len), _ptr(stats),
                                 _ptr(node_out), _stream(stream)))


def tree_mask(cfg, tree, mask, pos=None, stream=None):
    """vrt_tree_mask: mask is a device i32/u32 tensor [B, N, (N+31)//32], pos [B, N] or None."""
    _check(lib().vrt_tree_mask(ctypes.byref(cfg), _ptr(tree), _ptr(mask), _ptr(pos), _stream(stream)))


def accepted_kv(cfg, out_nodes, out_len, keep, keep_n, stream=None):
    """vrt_accepted_kv: keep [B, D+1], keep_n [B] (device i32 tensors)."""
    _check(lib().vrt_accepted_kv(ctypes.byref(cfg), _ptr(out_nodes), _ptr(out_len), _ptr(keep),
                                 _ptr(keep_n), _stream(stream)))


def support_coverage(cfg, draft_logits, ld, tree_stride, n_rows, coverage, stream=None):
    """vrt_support_coverage: coverage is a device f64 tensor [B, n_rows]."""
    _check(lib().vrt_support_coverage(ctypes.byref(cfg), _ptr(draft_logits), ld, tree_stride, n_rows,
                                      _ptr(coverage), _stream(stream)))


def read_probe(buf, sink, stream=None):
    """vrt_read_probe over the whole of `buf` (a device tensor); `sink` a device u32."""
    _check(lib().vrt_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                _stream(stream)))


# ---------------------------------------------------------------------------
# Views of the tree blob as typed tensors (no copies), following vrt_tree_layout.
_FIELDS = {
    # name: (dtype, shape per tree in terms of the layout capacities)
    "cand_token": ("i32", ("NC",)), "cand_parent": ("i32", ("NC",)), "cand_score": ("f32", ("NC",)),
    "cand_kind": ("i32", ("NC",)), "row_tail_n": ("i32", ("NR",)),
    "row_tail_id": ("i32", ("NR", "TC")), "row_tail_q": ("f32", ("NR", "TC")),
    "front": ("i32", ("FP",)), "n_front": ("i32", ()), "smart": ("f64", (8,)),
    "admitted": ("i32", ("N",)), "layer_sync": ("i32", ()), "n_nodes": ("i32", ()), "node_token": ("i32", ("N",)),
    "node_parent": ("i32", ("N",)), "node_depth": ("i32", ("N",)), "node_kind": ("i32", ("N",)),
    "node_cand": ("i32", ("N",)), "child_off": ("i32", ("N+1",)), "child": ("i32", ("N",)),
    "tail_n": ("i32", ("N",)), "tail_id": ("i32", ("N", "TC")), "tail_q": ("f32", ("N", "TC")),
    "row_dense": ("f64", ("NRd", 2)), "row_det": ("i32", ("NRd", 32)), "node_row": ("i32", ("Nd",)), "row_sync": ("i64", ("FP",)),
}


def tree_views(cfg, tree):
    """Dict of tensor views into the tree blob (a uint8 tensor of tree_bytes(cfg))."""
    import torch
    L = tree_layout_of(cfg)
    dt = {"i32": torch.int32, "f32": torch.float32, "f64": torch.float64, "i64": torch.int64}
    es = {"i32": 4, "f32": 4, "f64": 8, "i64": 8}
    out = {}
    for name, (t, shape) in _FIELDS.items():
        dims = []
        for d in shape:
            if isinstance(d, int):
                dims.append(d)
            elif d == "N+1":
                dims.append(L.N + 1)
            elif d in ("NRd", "Nd"):  # dense-row arrays: empty unless trunc = DENSE
                dims.append((L.NR if d == "NRd" else L.N) if cfg.trunc == DENSE else 0)
            else:
                dims.append(getattr(L, d))
        n = cfg.B
        for d in dims:
            n *= d
        off = getattr(L, name)
        out[name] = tree[off:off + n * es[t]].view(dt[t]).view(cfg.B, *dims)
    return out
