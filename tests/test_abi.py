"""The C ABI without a GPU: the library loads, exports every symbol include/vrt.h
declares, sizes buffers and rejects bad arguments with the documented codes."""
import ctypes
import os
import re

import pytest

from verify_row_top_amd import vrt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "vrt.h")).read()
    return sorted(set(re.findall(r"\b(vrt_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    L = ctypes.CDLL(vrt.LIB_PATH)
    names = _declared()
    assert set(names) == set(vrt.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_headline_sizes():
    c = vrt.make_config(B=32, V=128256, K=10, D=8, R=60)
    vrt.check_config(c)
    L = vrt.tree_layout_of(c)
    assert (L.NC, L.NR, L.N, L.TC, L.FP) == (710, 71, 61, 128, 10)
    assert vrt.tree_bytes(c) == L.total_bytes > 0
    assert vrt.workspace_bytes(c) > 0
    offs = [getattr(L, f) for f, _ in vrt.TreeLayout._fields_[5:-1]]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), vrt.EINVAL), (dict(V=0), vrt.EINVAL), (dict(V=(1 << 20) + 1), vrt.EINVAL),
    (dict(dtype=7), vrt.EDTYPE), (dict(trunc=-1), vrt.EINVAL), (dict(trunc=2048), vrt.EINVAL),
    (dict(K=0), vrt.EINVAL), (dict(K=31), vrt.EINVAL), (dict(m=10, K=10), vrt.EINVAL),
    (dict(m=-1), vrt.EINVAL), (dict(D=0), vrt.EINVAL), (dict(D=33), vrt.EINVAL),
    (dict(R=0), vrt.EINVAL), (dict(T=0.0), vrt.EINVAL), (dict(T=-1.0), vrt.EINVAL),
    (dict(T=float("nan")), vrt.EINVAL), (dict(T=1e-45), vrt.EINVAL), (dict(mode=5), vrt.EINVAL),
    (dict(mode=1, budget=0), vrt.EINVAL), (dict(mode=1, alpha=0.0), vrt.EINVAL),
    (dict(mode=1, gamma=float("inf")), vrt.EINVAL), (dict(W=200, K=30), vrt.EINVAL),
    (dict(eps_m0=-1.0), vrt.EINVAL), (dict(order=2), vrt.EINVAL), (dict(order=-1), vrt.EINVAL),
    (dict(tree_base=-1), vrt.EINVAL),
])
def test_bad_configs_are_rejected(kw, code):
    base = dict(B=2, V=1000, K=10, D=4, R=20)
    base.update(kw)
    c = vrt.make_config(**base)
    with pytest.raises(vrt.VrtError) as e:
        vrt.check_config(c)
    assert e.value.code == code
    assert vrt.last_error()
    assert vrt.lib().vrt_tree_bytes(ctypes.byref(c)) == 0


def test_m_equal_k_allowed_without_probe():
    vrt.check_config(vrt.make_config(B=1, V=100, K=4, m=4, probe=0, D=2, R=4))


class _FakeTensor:
    """Stands in for a tensor: a data pointer and a byte size, no GPU needed."""

    def __init__(self, ptr, nbytes=1 << 20):
        self.p, self.n = ptr, nbytes

    def data_ptr(self):
        return self.p

    def numel(self):
        return self.n

    def element_size(self):
        return 1


def _call_build(c, layer=0, logits=0x10000, ld=1024, stride=4096, tree=0x20000, ws=0x30000,
                ws_bytes=1 << 30):
    return vrt.lib().vrt_build_tree(ctypes.byref(c), layer, ctypes.c_void_p(logits), ld, stride, 1,
                                    0, ctypes.c_void_p(tree), ctypes.c_void_p(ws), ws_bytes, None,
                                    None)


def test_build_argument_errors_are_caught_before_any_launch():
    c = vrt.make_config(B=2, V=1000, K=4, D=3, R=10)
    assert _call_build(c, layer=3) == vrt.EINVAL
    assert _call_build(c, layer=-2) == vrt.EINVAL
    assert _call_build(c, logits=0) == vrt.EINVAL
    assert _call_build(c, logits=0x10004) == vrt.EINVAL            # not 16-byte aligned
    assert _call_build(c, ld=999) == vrt.EINVAL                    # ld < V
    assert _call_build(c, ld=1001) == vrt.EINVAL                   # ld not a multiple of 16 B
    assert _call_build(c, tree=0) == vrt.EINVAL
    assert _call_build(c, ws_bytes=16) == vrt.ENOMEM
    assert "workspace" in vrt.last_error()


def test_verify_argument_errors_are_caught_before_any_launch():
    c = vrt.make_config(B=2, V=1000, K=4, D=3, R=10)
    L = vrt.lib()
    good = dict(t=0x10000, ld=1024, stride=4096, tree=0x20000, ws=0x30000, wsb=1 << 30,
                o=0x40000, n=0x50000, ln=0x60000, st=0x70000)

    def call(**kw):
        a = dict(good, **kw)
        v = ctypes.c_void_p
        return L.vrt_verify_tree(ctypes.byref(c), v(a["t"]), a["ld"], a["stride"], v(a["tree"]), 1, 0,
                                 v(a["ws"]), a["wsb"], v(a["o"]), v(a["n"]), v(a["ln"]), v(a["st"]),
                                 None, None)
    assert call(t=0) == vrt.EINVAL
    assert call(o=0) == vrt.EINVAL
    assert call(st=0) == vrt.EINVAL
    assert call(wsb=8) == vrt.ENOMEM
    assert call(ld=10) == vrt.EINVAL
    assert call(stride=-16) == vrt.EINVAL


def test_dense_config_builds_but_probe_trees_are_not_verified():
    c = vrt.make_config(B=2, V=1000, K=4, D=3, R=10, trunc=vrt.DENSE)
    vrt.check_config(c)
    L = vrt.tree_layout_of(c)
    assert L.TC == 0 and vrt.tree_bytes(c) > 0
    v = ctypes.c_void_p
    r = vrt.lib().vrt_verify_tree(ctypes.byref(c), v(0x10000), 1024, 4096, v(0x20000), 1, 0,
                                  v(0x30000), 1 << 30, v(0x40000), v(0x50000), v(0x60000),
                                  v(0x70000), None, None)
    assert r == vrt.EINVAL and "VRT_DENSE" in vrt.last_error()
    r = vrt.lib().vrt_verify_nodes(ctypes.byref(c), v(0x10000), 1024, 4096, v(0x20000), 1, 0,
                                   v(0x30000), 1 << 30, None, None)
    assert r == vrt.EINVAL


def test_lazy_verify_argument_errors_are_caught_before_any_launch():
    c = vrt.make_config(B=2, V=1000, K=4, D=3, R=10)
    L = vrt.lib()
    good = dict(t=0x10000, ld=1024, stride=4096, tree=0x20000, ws=0x30000, wsb=1 << 30,
                o=0x40000, n=0x50000, ln=0x60000, st=0x70000)

    def call(**kw):
        a = dict(good, **kw)
        v = ctypes.c_void_p
        return L.vrt_verify_lazy(ctypes.byref(c), v(a["t"]), a["ld"], a["stride"], v(a["tree"]), 1, 0,
                                 v(a["ws"]), a["wsb"], v(a["o"]), v(a["n"]), v(a["ln"]), v(a["st"]),
                                 None, None)
    assert call(t=0) == vrt.EINVAL
    assert call(o=0) == vrt.EINVAL
    assert call(n=0) == vrt.EINVAL
    assert call(st=0) == vrt.EINVAL
    assert call(wsb=8) == vrt.ENOMEM
    assert call(ld=10) == vrt.EINVAL
    assert call(tree=0x20008) == vrt.EINVAL
    d = vrt.make_config(B=2, V=1000, K=4, D=3, R=10, trunc=vrt.DENSE)
    v = ctypes.c_void_p
    assert L.vrt_verify_lazy(ctypes.byref(d), v(0x10000), 1024, 4096, v(0x20000), 1, 0, v(0x30000),
                             1 << 30, v(0x40000), v(0x50000), v(0x60000), v(0x70000), None,
                             None) == vrt.EINVAL


def test_dense_verify_argument_errors_are_caught_before_any_launch():
    c = vrt.make_config(B=2, V=1000, K=4, D=3, R=10, trunc=vrt.DENSE)
    L = vrt.lib()
    v = ctypes.c_void_p
    good_layers = (ctypes.c_void_p * 3)(0x80000, 0x90000, 0xA0000)

    def call(cfg=c, layers=good_layers, dld=1024, dstride=4096 * 10, t=0x10000):
        return L.vrt_verify_dense(ctypes.byref(cfg), v(t), 1024, 4096, layers, dld, dstride, v(0x20000), 1, 0,
                                  v(0x30000), 1 << 30, v(0x40000), v(0x50000), v(0x60000), v(0x70000), None,
                                  None)
    assert call(layers=None) == vrt.EINVAL
    assert call(dld=10) == vrt.EINVAL
    assert call(layers=(ctypes.c_void_p * 3)(0x80000, 0x90008, 0xA0000)) == vrt.EINVAL
    assert call(layers=(ctypes.c_void_p * 3)(0x80000, None, 0xA0000)) == vrt.EINVAL
    assert call(t=0) == vrt.EINVAL
    truncated = vrt.make_config(B=2, V=1000, K=4, D=3, R=10)
    assert call(cfg=truncated) == vrt.EINVAL and "VRT_DENSE" in vrt.last_error()


def test_split_verify_argument_errors_are_caught_before_any_launch():
    c = vrt.make_config(B=2, V=1000, K=4, D=3, R=10)
    L = vrt.lib()
    v = ctypes.c_void_p
    # decisions: target rows are checked, outputs are not needed
    assert L.vrt_verify_nodes(ctypes.byref(c), v(0), 1024, 4096, v(0x20000), 1, 0, v(0x30000), 1 << 30,
                              None, None) == vrt.EINVAL
    assert L.vrt_verify_nodes(ctypes.byref(c), v(0x10000), 1024, 4096, v(0x20000), 1, 0, v(0x30000), 8,
                              None, None) == vrt.ENOMEM
    assert "workspace" in vrt.last_error()
    assert L.vrt_verify_nodes(ctypes.byref(c), v(0x10000), 10, 4096, v(0x20000), 1, 0, v(0x30000),
                              1 << 30, None, None) == vrt.EINVAL
    # the walk: outputs are checked, no logits
    good = dict(tree=0x20000, ws=0x30000, wsb=1 << 30, o=0x40000, n=0x50000, ln=0x60000, st=0x70000)

    def walk(**kw):
        a = dict(good, **kw)
        return L.vrt_verify_walk(ctypes.byref(c), v(a["tree"]), v(a["ws"]), a["wsb"], v(a["o"]), v(a["n"]),
                                 v(a["ln"]), v(a["st"]), None, None)
    assert walk(o=0) == vrt.EINVAL
    assert walk(st=0) == vrt.EINVAL
    assert walk(tree=0) == vrt.EINVAL
    assert walk(wsb=8) == vrt.ENOMEM
    assert walk(ws=0x30008) == vrt.EINVAL  # not 16-byte aligned


def test_mask_and_kv_argument_errors_are_caught_before_any_launch():
    c = vrt.make_config(B=2, V=1000, K=4, D=3, R=10)
    L = vrt.lib()
    v = ctypes.c_void_p
    assert L.vrt_tree_mask(ctypes.byref(c), v(0), v(0x40000), None, None) == vrt.EINVAL
    assert L.vrt_tree_mask(ctypes.byref(c), v(0x20000), v(0), None, None) == vrt.EINVAL
    assert L.vrt_tree_mask(ctypes.byref(c), v(0x20008), v(0x40000), None, None) == vrt.EINVAL
    assert L.vrt_tree_mask(ctypes.byref(c), v(0x20000), v(0x40002), None, None) == vrt.EINVAL
    assert L.vrt_accepted_kv(ctypes.byref(c), v(0x1000), v(0x2000), v(0), v(0x3000), None) == vrt.EINVAL
    assert L.vrt_accepted_kv(ctypes.byref(c), v(0x1000), v(0x2001), v(0x4000), v(0x3000), None) == vrt.EINVAL
    bad = vrt.make_config(B=2, V=1000, K=4, D=3, R=10)
    bad.B = 0
    assert L.vrt_tree_mask(ctypes.byref(bad), v(0x20000), v(0x40000), None, None) == vrt.EINVAL
