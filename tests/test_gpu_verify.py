"""GPU parity of vrt_verify_tree against the oracle, on trees the oracle built.

The oracle builds each tree from generator rows, its verification view is written
into the library's tree blob, and both sides verify the same target rows with the
same Philox counters. Every node's outcome (accepted child or final token) must
match bit for bit unless the oracle flags one of that node's draws as within 1e-6
of its threshold; the residual mass W must agree to 1e-5; the emitted tokens must
match whenever the walk's path has no such draw.
"""
import numpy as np
import pytest
import torch

import synth
from synth import workloads
from tests.gpu_common import Lib, lib_config, to_device_rows
from oracle.drive import OracleStep

pytestmark = pytest.mark.gpu


def _small(**kw):
    base = dict(name="small", B=4, V=5000, dtype=synth.BF16, R=40, D=5, K=6, m=1, T=1.0,
                zipf=(1.1,), sigma=0.7)
    base.update(kw)
    return workloads.Workload(**base)


CASES = [
    ("tiny", workloads.get("tiny")),
    ("tiny_m0_T06", workloads.get("tiny").replace(m=0, T=0.6)),
    ("small_bf16_ragged", _small()),
    ("small_m3_K8", _small(m=3, K=8, R=50)),
    ("small_probe_off", _small(probe=0)),
    ("small_trunc4", _small(V=300, trunc=4, K=3, R=12, D=4)),
    ("small_T06_trunc256", _small(T=0.6, trunc=256, V=3000)),
    ("small_fp32_flat", _small(dtype=synth.F32, zipf=(0.8,), V=4100, R=30)),
    ("stress_mixed_m0", _small(B=4, V=9000, zipf=(1.5, 0.8), split=2, R=64, D=6, K=8, m=0)),
]


def run_case(w, seed, step, dev, lazy=False):
    steps = [OracleStep(w, seed, b, step) for b in range(w.B)]
    cfg = lib_config(w)
    L = Lib(cfg, dev)
    for b, s in enumerate(steps):
        L.write_view(b, s.view)
    target, ld = to_device_rows([s.target_rows for s in steps], w, L.N, dev)
    print(f"verify parity: {w.name} seed={seed} step={step} B={w.B} V={w.V} lazy={lazy}", flush=True)
    if lazy:
        L.node_out.fill_(-7)
        L.verify_lazy(target, ld, seed, step)
    else:
        L.verify(target, ld, seed, step)
    return steps, L


def check(steps, L, lazy=False):
    """Compare every node (lazy: every node the walk visits, the others untouched); a
    mismatch is allowed only at a node the oracle marks as having a draw within 1e-6 of
    its threshold. Returns (exempt, mismatched, nodes)."""
    node_out = L.node_out.cpu().numpy()
    out_tok = L.out_tokens.cpu().numpy()
    out_len = L.out_len.cpu().numpy()
    out_nodes = L.out_nodes.cpu().numpy()
    stats = L.stats.cpu().numpy()
    n_exempt = n_miss = n_nodes = 0
    for b, s in enumerate(steps):
        pn = s.per_node
        n = s.view["n_nodes"]
        assert stats[b, 0] == 0, f"status bits {stats[b, 0]:#x} on tree {b}"
        visit = set(range(n))
        if lazy:  # the nodes both walks visit (they part only after a near-threshold draw)
            visit = ({0} | set(s.out_nodes.tolist())) & ({0} | set(out_nodes[b, :out_len[b] - 1].tolist()))
            assert stats[b, 4] == len(s.out_tokens) or s.verify_exempt > 0
            assert stats[b, 1] == out_len[b] - 1
            untouched = [i for i in range(n) if i not in visit]
            if s.verify_exempt == 0:
                assert (node_out[b, untouched] == -7).all(), "lazy walk decided an unvisited node"
        for i in sorted(visit):
            n_nodes += 1
            g = node_out[b, i]
            same = g[0] == pn["accept"][i] and (pn["accept"][i] >= 0 or g[1] == pn["token"][i])
            if pn["exempt"][i]:
                n_exempt += 1
                n_miss += not same
                continue
            assert same, (b, i, g, pn[i])
            if pn["accept"][i] < 0:
                W = np.array([g[3]], np.int32).view(np.float32)[0]
                assert abs(W - pn["W"][i]) <= 1e-5, (b, i, W, pn["W"][i])
            assert (g[2] & 0xFF) == pn["n_tests"][i], (b, i, g, pn[i])
        L_ = len(s.out_tokens)
        same = out_len[b] == L_ and np.array_equal(out_tok[b, :L_], s.out_tokens) and \
            np.array_equal(out_nodes[b, :L_ - 1], s.out_nodes) and np.all(out_tok[b, L_:] == -1)
        assert same or s.verify_exempt > 0, (b, out_tok[b], s.out_tokens)
    return n_exempt, n_miss, n_nodes


@pytest.mark.parametrize("lazy", [False, True], ids=["all_nodes", "lazy"])
@pytest.mark.parametrize("name,w", CASES, ids=[c[0] for c in CASES])
def test_verify_matches_oracle(gpu, name, w, lazy):
    tot_ex = tot_miss = tot = 0
    for seed, step in [(1, 0), (2, 5), (3, 77)]:
        steps, L = run_case(w, seed, step, gpu, lazy)
        ex, miss, n = check(steps, L, lazy)
        tot_ex += ex
        tot_miss += miss
        tot += n
    print(f"{name}: {tot} nodes, {tot_ex} with a near-threshold draw, {tot_miss} of those differ")
    assert tot_miss <= max(1, tot_ex // 10), (tot_miss, tot_ex)


def test_verify_bad_target_rows_set_status(gpu):
    w = _small(B=3)
    steps = [OracleStep(w, 4, b, 0, verify=False) for b in range(w.B)]
    cfg = lib_config(w)
    L = Lib(cfg, gpu)
    for b, s in enumerate(steps):
        L.write_view(b, s.view)
    rows = [s.target_rows.copy() for s in steps]
    rows[0][0, 17] = 0x7FC0       # NaN in tree 0's root row
    rows[1][1, :] = 0xFF80        # tree 1: node 1's row entirely -inf
    target, ld = to_device_rows(rows, w, L.N, gpu)
    L.verify(target, ld, 4, 0)
    st = L.stats.cpu().numpy()[:, 0]
    assert st[0] & 0x4 and st[1] & 0x4 and st[2] == 0
    assert (L.out_len.cpu().numpy() >= 1).all()


def test_verify_empty_tree_is_a_bonus_sample(gpu):
    # a tree with only the root: one token drawn from p at the root
    w = _small(B=2)
    steps = [OracleStep(w, 9, b, 0) for b in range(w.B)]
    cfg = lib_config(w)
    L = Lib(cfg, gpu)
    for b, s in enumerate(steps):
        v = dict(s.view)
        v = {k: (a[:1] if isinstance(a, np.ndarray) and k not in ("child_off", "child") else a)
             for k, a in v.items()}
        v["n_nodes"] = 1
        v["child_off"] = np.zeros(2, np.int32)
        v["child"] = np.zeros(0, np.int32)
        v["tail_n"] = np.zeros(1, np.int32)
        L.write_view(b, v)
        from oracle import oracle as orc
        from oracle.drive import oracle_cfg
        tok, nodes, pn, ex = orc.verify(oracle_cfg(w), v, synth.to_f32(s.target_rows[:1]), 9, b, 0)
        s.bonus = (tok, ex)
    target, ld = to_device_rows([s.target_rows for s in steps], w, L.N, gpu)
    L.verify(target, ld, 9, 0)
    for b, s in enumerate(steps):
        tok, ex = s.bonus
        assert L.out_len[b].item() == 1
        if ex == 0:
            assert L.out_tokens[b, 0].item() == tok[0]


def test_lazy_walk_flags_a_bad_root_row(gpu):
    w = _small(B=2)
    steps = [OracleStep(w, 4, b, 0, verify=False) for b in range(w.B)]
    L = Lib(lib_config(w), gpu)
    for b, s in enumerate(steps):
        L.write_view(b, s.view)
    rows = [s.target_rows.copy() for s in steps]
    rows[0][0, 17] = 0x7FC0       # NaN in tree 0's root row
    target, ld = to_device_rows(rows, w, L.N, gpu)
    L.verify_lazy(target, ld, 4, 0)
    st = L.stats.cpu().numpy()[:, 0]
    assert st[0] & 0x4 and st[1] == 0
    assert (L.out_len.cpu().numpy() >= 1).all()
