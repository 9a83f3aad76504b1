"""SMART keep rule (SMART key designs 1-3) and the temperature limit of
RheoSampling's findings, pinned by hand-worked cases and invariants.

Readings (see the design notes): |P| is the number of root-to-leaf paths of
the current tree (its leaf count), the accumulated gain L starts at 0, |T|
counts the root, g = path probability / |P|. These readings are parity
unpinned beyond the hand-worked cases below.
"""
import numpy as np
import pytest

from oracle import oracle as orc
from synth import workloads
from oracle.drive import OracleStep, oracle_cfg


def _row(V, probs_at):
    """A logit row with softmax(row) = the given probabilities at the given ids (rest ~0)."""
    row = np.full(V, -200.0, np.float32)
    for tok, p in probs_at.items():
        row[tok] = np.log(p)
    return row


def _smart(V=4, K=4, D=1, budget=10, alpha=1.0, lam=1.0, gamma=0.0, delta=0.0, rho=1.0):
    return orc.make_cfg(V=V, trunc=V, K=K, m=1, probe=0, D=D, mode=orc.SMART, budget=budget,
                        alpha=alpha, lam=lam, gamma=gamma, delta=delta, rho=rho, T=1.0)


def _emitted(t):
    t.finish()
    v = t.view()
    return v["token"][1:].tolist(), v["parent"][1:].tolist()


def test_linear_cost_keeps_above_average_gain():
    # probabilities 0.5, 0.3, 0.15, 0.05 at ids 2, 0, 3, 1; gamma = 0 so the rule is
    # alpha * g * |T| > L:  0.5 kept (L = 0); 0.3 * 2 = 0.6 > 0.5 kept (root had a
    # child already, so |P| becomes 2); (0.15 / 2) * 3 = 0.225 < 0.8 rejected.
    t = orc.Tree(_smart(), 1, 0, 0)
    t.expand_layer(0, _row(4, {2: 0.5, 0: 0.3, 3: 0.15, 1: 0.05})[None])
    toks, pars = _emitted(t)
    assert toks == [2, 0] and pars == [0, 0]


def test_discount_alpha_prunes_more():
    # alpha = 0.5: 0.5 * 0.3 * 2 = 0.3 < 0.5, so only the first candidate is kept
    t = orc.Tree(_smart(alpha=0.5), 1, 0, 0)
    t.expand_layer(0, _row(4, {2: 0.5, 0: 0.3, 3: 0.15, 1: 0.05})[None])
    assert _emitted(t)[0] == [2]


def test_superlinear_verify_cost_prunes_more():
    # lambda = 0, gamma = delta = rho = 1: C(n) = e^n - 1, C'(n) = e^n, the rule is
    # g (1 - e^-n) > L: 0.3 (1 - e^-2) = 0.26 < 0.5, so the second candidate goes.
    t = orc.Tree(_smart(lam=0.0, gamma=1.0, delta=1.0, rho=1.0), 1, 0, 0)
    t.expand_layer(0, _row(4, {2: 0.5, 0: 0.3, 3: 0.15, 1: 0.05})[None])
    assert _emitted(t)[0] == [2]


def test_budget_caps_admissions():
    t = orc.Tree(_smart(budget=1), 1, 0, 0)
    t.expand_layer(0, _row(4, {2: 0.5, 0: 0.3, 3: 0.15, 1: 0.05})[None])
    assert _emitted(t)[0] == [2]


def test_two_layers_hand_worked():
    # layer 1: 0.9 kept (L = 0.9, |T| = 2, |P| = 1); 0.06 * 2 = 0.12 < 0.9 rejected.
    # layer 2 under the 0.9 node (a leaf, so |P| stays 1): path 0.9 * 0.95 = 0.855,
    # 0.855 * 2 = 1.71 > 0.9 kept (L = 1.755, |T| = 3); 0.9 * 0.03 * 3 = 0.081 < 1.755.
    cfg = _smart(D=2)
    t = orc.Tree(cfg, 1, 0, 0)
    t.expand_layer(0, _row(4, {1: 0.9, 0: 0.06, 2: 0.03, 3: 0.01})[None])
    front = t.frontier()
    assert len(front) == 1 and t.cands()[front[0]]["token"] == 1
    t.expand_layer(1, _row(4, {2: 0.95, 1: 0.03, 0: 0.01, 3: 0.01})[None])
    toks, pars = _emitted(t)
    assert toks == [1, 2] and pars == [0, 1]


def test_first_rejection_ends_the_layer_and_invariants_hold():
    w = workloads.get("tiny").replace(mode=orc.SMART, budget=24, D=5, K=6, W=0, alpha=1.0,
                                      lam=0.02, gamma=0.01, delta=0.004, rho=1.3)
    for seed in range(6):
        s = OracleStep(w, seed, 0, seed, verify=False)
        v = s.view
        n = v["n_nodes"]
        assert 1 <= n <= w.budget + 1
        assert np.all(v["parent"][1:] < np.arange(1, n))
        assert v["depth"].max() <= w.D
        # admitted nodes of each layer are a best-first prefix of that layer's candidates
        cands = s.cands
        for layer in range(w.D):
            base = s.tree.layer_base(layer)
            span = (1 if layer == 0 else w.budget) * w.K
            sl = np.arange(base, base + span)
            sl = sl[cands["live"][sl] == 1]
            if sl.size == 0:
                continue
            order = sl[np.lexsort((sl, -cands["score"][sl].astype(np.float64)))]
            adm = [c for c in v["cand"][1:] if base <= c < base + span]
            assert list(order[:len(adm)]) == adm


def test_temperature_to_zero_m0_equals_topk_tree():
    # RheoSampling findings: at T -> 0, m = 0 collapses to the deterministic top-K tree
    w = workloads.get("tiny")
    for seed in range(12):
        a = OracleStep(w, seed, 0, seed, cfg=oracle_cfg(w, m=0, T=1e-3), verify=False)
        b = OracleStep(w, seed, 0, seed, cfg=oracle_cfg(w, probe=0, T=1e-3), verify=False)
        assert set(a.node_keys.tolist()) == set(b.node_keys.tolist())


def test_temperature_to_zero_m1_keeps_topk_tokens_but_not_structure():
    # m = 1: every parent's children are still the top-K tokens (the probe, when the
    # tempered tail mass has not underflowed to 0, is the second-ranked token), but its
    # proxy score differs from q(x_2), so the prune keeps a different tree
    w = workloads.get("tiny")
    differ = 0
    for seed in range(12):
        a = OracleStep(w, seed, 0, seed, cfg=oracle_cfg(w, m=1, T=1e-3), verify=False)
        b = OracleStep(w, seed, 0, seed, cfg=oracle_cfg(w, probe=0, T=1e-3), verify=False)
        for r in range(a.tree.n_rows()):
            e = a.tree.row(r)
            if e.n_sup == 0:
                continue
            assert e.probe_rank in (-1, 1)
        differ += set(a.node_keys.tolist()) != set(b.node_keys.tolist())
    assert differ >= 1
