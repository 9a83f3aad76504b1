"""GPU parity of the tree attention mask, position ids (vrt_tree_mask) and the kept KV
entries (vrt_accepted_kv) against the oracle, bit for bit.

Trees come from the oracle's own builds (small workloads) or from seeded random parent
arrays at the workloads' full node counts (61 for the headline, 129 for the stress and
SMART workloads), some with parents out of range; the oracle's reading of those is the
same tree with such parents cut (the path ends there).
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from synth import workloads
from tests.gpu_common import Lib, lib_config
from oracle.drive import OracleStep
from tests.test_gpu_build import _small
from verify_row_top_amd import vrt

pytestmark = pytest.mark.gpu


def _unpack(words, N):
    bits = np.unpackbits(words.view(np.uint8), bitorder="little").reshape(words.shape[0], -1)
    return bits[:, :N].astype(bool)


def _mask_of(L, b, N):
    W32 = (N + 31) // 32
    m = torch.zeros((L.cfg.B, N, W32), dtype=torch.int32, device=L.dev)
    pos = torch.zeros((L.cfg.B, N), dtype=torch.int32, device=L.dev)
    vrt.tree_mask(L.cfg, L.tree, m, pos)
    torch.cuda.synchronize()
    return m.cpu().numpy().view(np.uint32), pos.cpu().numpy()


@pytest.mark.parametrize("w", [_small(B=4, R=40, D=5), _small(B=3, m=3, K=8, R=50)], ids=["small", "m3"])
def test_mask_of_oracle_trees(gpu, w):
    steps = [OracleStep(w, 3, b, 1, verify=False) for b in range(w.B)]
    L = Lib(lib_config(w), gpu)
    for b, s in enumerate(steps):
        L.write_view(b, s.view)
    words, pos = _mask_of(L, 0, L.N)
    for b, s in enumerate(steps):
        n = s.view["n_nodes"]
        want, wpos = O.tree_mask(s.view["parent"])
        got = _unpack(words[b], L.N)
        np.testing.assert_array_equal(got[:n, :n], want)
        assert not got[n:].any() and not got[:, n:].any()
        np.testing.assert_array_equal(pos[b, :n], wpos)
        assert (pos[b, n:] == -1).all()


@pytest.mark.parametrize("name,w", [("headline", workloads.get("headline")),
                                    ("stress", workloads.get("stress")),
                                    ("smart", workloads.get("smart"))])
def test_mask_at_full_node_counts(gpu, name, w):
    rng = np.random.default_rng(11)
    L = Lib(lib_config(w), gpu)
    N, B = L.N, w.B
    n_nodes = rng.integers(1, N + 1, size=B).astype(np.int32)
    n_nodes[0], n_nodes[-1] = N, 1
    parents = np.full((B, N), -1, np.int32)
    for b in range(B):
        for i in range(1, N):
            parents[b, i] = rng.integers(0, i)
        if b % 3 == 1:  # some parents out of range: the path ends there
            bad = rng.integers(1, N, size=3)
            parents[b, bad] = np.array([N + 5, -3, 10**6])[: bad.size]
    L.views["n_nodes"].copy_(torch.from_numpy(n_nodes))
    L.views["node_parent"].copy_(torch.from_numpy(parents))
    words, pos = _mask_of(L, 0, N)
    for b in range(B):
        n = int(n_nodes[b])
        p = parents[b, :n].copy()
        for i in range(1, n):
            if not (0 <= p[i] < i):
                p[i] = -1
        # the oracle takes only well-formed trees: a cut path is a forest; mask it per root
        want = np.zeros((n, n), bool)
        wpos = np.zeros(n, np.int32)
        for i in range(n):
            a, d = i, -1
            while a >= 0:
                want[i, a] = True
                a, d = p[a] if a > 0 else -1, d + 1
            wpos[i] = d
        if (p[1:] >= 0).all():
            om, op = O.tree_mask(p)
            np.testing.assert_array_equal(om, want)
            np.testing.assert_array_equal(op, wpos)
        got = _unpack(words[b], N)
        np.testing.assert_array_equal(got[:n, :n], want)
        assert not got[n:].any() and not got[:, n:].any()
        np.testing.assert_array_equal(pos[b, :n], wpos)


def test_accepted_kv_matches_oracle(gpu):
    w = workloads.get("headline")
    cfg = lib_config(w)
    B, D = w.B, w.D
    rng = np.random.default_rng(5)
    out_len = rng.integers(1, D + 2, size=B).astype(np.int32)
    out_len[0], out_len[1] = 1, D + 1
    out_nodes = np.full((B, D), -1, np.int32)
    for b in range(B):
        out_nodes[b, : out_len[b] - 1] = np.sort(rng.choice(np.arange(1, 61), out_len[b] - 1, replace=False))
    on = torch.from_numpy(out_nodes).to(gpu)
    ol = torch.from_numpy(out_len).to(gpu)
    keep = torch.full((B, D + 1), 99, dtype=torch.int32, device=gpu)
    keep_n = torch.zeros(B, dtype=torch.int32, device=gpu)
    vrt.accepted_kv(cfg, on, ol, keep, keep_n)
    torch.cuda.synchronize()
    k, kn = keep.cpu().numpy(), keep_n.cpu().numpy()
    for b in range(B):
        want = O.accepted_kv(out_len[b], out_nodes[b])
        assert kn[b] == want.size
        np.testing.assert_array_equal(k[b, : want.size], want)
        assert (k[b, want.size:] == -1).all()
