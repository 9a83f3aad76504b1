"""Seeded synthetic logits (the stand-in for draft and target models), host and device.

The same __host__ __device__ routines in synth.hip produce the rows on the CPU
(to feed the oracle) and on the GPU (to fill HBM for tests and the benchmark).
This module holds no tree-building or verification arithmetic.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libvrtsynth.so")

F32, BF16 = 0, 1
DRAFT, TARGET = 0, 1


class Params(ctypes.Structure):
    _fields_ = [("V", ctypes.c_int32), ("dtype", ctypes.c_int32), ("n_tables", ctypes.c_int32),
                ("split", ctypes.c_int32), ("draft_scale", ctypes.c_float),
                ("target_sigma", ctypes.c_float), ("seed", ctypes.c_uint64)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build()
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
        L.syn_node_key.argtypes = [u64, i32]
        L.syn_node_key.restype = u64
        L.syn_root_key.argtypes = [u64, i32]
        L.syn_root_key.restype = u64
        L.syn_rows_host.argtypes = [ctypes.POINTER(Params), vp, i32, vp, vp, vp, i64, i32]
        L.syn_rows_dev.argtypes = [ctypes.POINTER(Params), vp, i32, vp, vp, vp, i64, i32, vp]
        L.syn_rows_dev.restype = i32
        L.syn_frontier_keys_dev.argtypes = [i32, i32, i32, i32, vp, vp, vp, i32, vp, i32, vp, vp]
        L.syn_frontier_keys_dev.restype = i32
        L.syn_tree_keys_dev.argtypes = [i32, i32, vp, vp, vp, vp, vp, vp]
        L.syn_tree_keys_dev.restype = i32
        _lib = L
    return _lib


def zipf_table(V, a):
    """Zipf-shaped base logits z[r-1] = -a ln r, r = 1..V, computed in fp64 and rounded to fp32."""
    r = np.arange(1, V + 1, dtype=np.float64)
    return (-a * np.log(r)).astype(np.float32)


def tables(V, exponents):
    """Stacked Zipf tables [len(exponents), V] (empty when there is no Zipf base)."""
    if not exponents:
        return np.zeros((1, max(V, 1)), np.float32)
    return np.stack([zipf_table(V, a) for a in exponents]).astype(np.float32)


def node_key(parent, token):
    return lib().syn_node_key(parent, int(token))


def root_key(seed, b):
    return lib().syn_root_key(seed, int(b))


def path_key(root, tokens):
    k = root
    for t in tokens:
        k = node_key(k, t)
    return k


def decode_keys(root_keys, tokens):
    """Root keys of the next decode step: each tree's context extended by the tokens its
    step emitted (the node-key chain)."""
    return [path_key(int(k), [int(t) for t in toks]) for k, toks in zip(root_keys, tokens)]


def rows_host(p, zipf, keys, trees=None, which=DRAFT):
    """Rows for the given node keys on the CPU: uint16 (bf16 bits) or float32, shape [n, V]."""
    keys = np.ascontiguousarray(keys, dtype=np.uint64)
    n = keys.size
    out = np.zeros((n, p.V), np.uint16 if p.dtype == BF16 else np.float32)
    tr = None if trees is None else np.ascontiguousarray(trees, dtype=np.int32)
    zipf = np.ascontiguousarray(zipf, dtype=np.float32)
    lib().syn_rows_host(ctypes.byref(p), zipf.ctypes.data_as(ctypes.c_void_p), n,
                        keys.ctypes.data_as(ctypes.c_void_p),
                        None if tr is None else tr.ctypes.data_as(ctypes.c_void_p),
                        out.ctypes.data_as(ctypes.c_void_p), p.V, which)
    return out


def to_f32(rows):
    """Expand bf16 bit patterns (uint16) to float32 exactly; float32 passes through."""
    rows = np.asarray(rows)
    if rows.dtype == np.uint16:
        return (rows.astype(np.uint32) << 16).view(np.float32)
    return rows.astype(np.float32, copy=False)


def rows_dev(p, zipf_dev, keys_dev, trees_dev, out, which, stream):
    """Device rows into `out` (a [n, ld] tensor) for device keys; torch tensors, async on stream."""
    r = lib().syn_rows_dev(ctypes.byref(p), ctypes.c_void_p(zipf_dev.data_ptr()), keys_dev.numel(),
                           ctypes.c_void_p(keys_dev.data_ptr()),
                           None if trees_dev is None else ctypes.c_void_p(trees_dev.data_ptr()),
                           ctypes.c_void_p(out.data_ptr()), out.stride(-2) if out.dim() > 1 else p.V,
                           which, ctypes.c_void_p(stream))
    if r != 0:
        raise RuntimeError("synthetic row generation failed to launch")


def frontier_keys_dev(B, K, base, prev_keys, nxt, n_next, cand_token, out, stream):
    r = lib().syn_frontier_keys_dev(B, K, base, prev_keys.shape[-1], ctypes.c_void_p(prev_keys.data_ptr()),
                                    ctypes.c_void_p(nxt.data_ptr()), ctypes.c_void_p(n_next.data_ptr()),
                                    nxt.shape[-1], ctypes.c_void_p(cand_token.data_ptr()),
                                    cand_token.shape[-1], ctypes.c_void_p(out.data_ptr()),
                                    ctypes.c_void_p(stream))
    if r != 0:
        raise RuntimeError("frontier key kernel failed to launch")


def tree_keys_dev(B, N, root_keys, n_nodes, token, parent, out, stream):
    r = lib().syn_tree_keys_dev(B, N, ctypes.c_void_p(root_keys.data_ptr()),
                                ctypes.c_void_p(n_nodes.data_ptr()), ctypes.c_void_p(token.data_ptr()),
                                ctypes.c_void_p(parent.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                ctypes.c_void_p(stream))
    if r != 0:
        raise RuntimeError("tree key kernel failed to launch")
