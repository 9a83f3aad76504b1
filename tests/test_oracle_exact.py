"""Exact enumeration pins of the oracle's build and verification (RheoSampling
highlights: the step is lossless for any prune budget R; key design 3: probe-first
optimal-transport verification).

orc_exact_law runs the oracle's own expansion and decision code with every probe draw,
every accept/reject test and every final sample taken as a branch weighted by its
probability (u uniform on [0, 1)), on small context-table models (V <= 8, depth <= 3).
Losslessness then fixes the result exactly, independently of the oracle:
  * the first emitted token's law is the tempered target softmax at the root context;
  * the law of the first two emitted tokens is p(a) p(b | a), whether the second token
    comes from the same tree or from the next step;
to 1e-12, for probe first and probe last, m in {0, 1, 3}, supports shorter than V, the
dense support (the whole vocabulary, the probe drawn in token-id order), prune budgets
below K, the plain top-K tree and trees shaped by SMART's keep rule (which the laws do
not pin: any kept subtree is verified losslessly). At depth 1 the probability that the first token comes
from the tree must also equal the closed forms derived from key design 3
(tests/test_oracle_lossless.py, tests/test_oracle_rrsw.py) to 1e-12; for the dense
support the closed form is that of a truncated support holding all V tokens, since the
probe's law does not depend on the order its inverse CDF walks.
"""
import numpy as np
import pytest

from oracle import oracle as orc
from tests.test_oracle_lossless import _depth1_acceptance
from tests.test_oracle_rrsw import _depth1_rrsw

TOL = 1e-12


def tables(V, D, seed):
    """Draft and target rows for every context path of length <= D + 1."""
    n = sum(V ** k for k in range(D + 2))
    rng = np.random.default_rng(seed)
    dt = (rng.normal(size=(n, V)) * 1.5).astype(np.float32)
    tt = (dt + rng.normal(size=(n, V)) * 0.8).astype(np.float32)
    return dt, tt


def softmax(x, T):
    invT = np.float64(np.float32(1.0) / np.float32(T))
    e = np.exp((x.astype(np.float64) - np.float64(x.max())) * invT)
    return e / e.sum()


CONFIGS = [
    ("m1_fillers_D3", dict(V=8, trunc=8, K=3, m=1, D=3, W=2, R=6, T=1.0), 1),
    ("m0_T06", dict(V=8, trunc=8, K=3, m=0, D=2, W=2, R=5, T=0.6), 2),
    ("m3_K4", dict(V=6, trunc=6, K=4, m=3, D=2, W=1, R=5, T=1.0), 3),
    ("trunc4_lt_V8", dict(V=8, trunc=4, K=3, m=1, D=3, W=2, R=6, T=0.8), 4),
    ("probe_last_D3", dict(V=7, trunc=7, K=3, m=1, D=3, W=2, R=5, T=1.0, order=orc.PROBE_LAST), 5),
    ("probe_last_trunc5_T06", dict(V=8, trunc=5, K=3, m=0, D=2, W=3, R=4, T=0.6, order=orc.PROBE_LAST), 6),
    ("probe_off_topk", dict(V=8, trunc=8, K=3, m=0, probe=0, D=3, W=2, R=6, T=1.0), 7),
    ("K1_m0_chain", dict(V=6, trunc=6, K=1, m=0, D=3, W=1, R=3, T=1.0), 8),
    ("R2_lt_K3", dict(V=8, trunc=8, K=3, m=1, D=3, W=3, R=2, T=1.0), 9),
    ("dense_m1_D3", dict(V=6, trunc=orc.DENSE, K=3, m=1, D=3, W=2, R=6, T=1.0), 41),
    ("dense_m0_T06", dict(V=7, trunc=orc.DENSE, K=3, m=0, D=2, W=2, R=5, T=0.6), 42),
    ("dense_m3_K4_T08", dict(V=6, trunc=orc.DENSE, K=4, m=3, D=2, W=1, R=5, T=0.8), 43),
    ("dense_probe_last_D3", dict(V=6, trunc=orc.DENSE, K=3, m=1, D=3, W=2, R=5, T=1.0,
                                 order=orc.PROBE_LAST), 44),
    # SMART's keep rule shapes the tree (a parent keeps some of its children, the frontier
    # varies); the step stays lossless whatever the rule keeps
    ("smart_budget4", dict(V=6, trunc=6, K=3, m=1, D=3, mode=orc.SMART, budget=4, T=1.0,
                           alpha=1.0, lam=0.02, gamma=0.01, delta=0.004, rho=1.3), 51),
    ("smart_budget6_m0_T06", dict(V=6, trunc=6, K=3, m=0, D=3, mode=orc.SMART, budget=6, T=0.6,
                                  alpha=50.0, lam=0.02, gamma=0.01, delta=0.004, rho=1.3), 52),
    ("smart_dense_alpha08", dict(V=6, trunc=orc.DENSE, K=3, m=1, D=3, mode=orc.SMART, budget=5,
                                 T=1.0, alpha=0.8, lam=0.02, gamma=0.01, delta=0.004, rho=1.3), 53),
]


def laws_match(kw, seed):
    """(max |law1 - p|, max |law2 - p x p(.|a)|, sum of law1) for one configuration."""
    V, D, T = kw["V"], kw["D"], kw["T"]
    cfg = orc.make_cfg(**kw)
    dt, tt = tables(V, D, seed)
    law1, law2, _ = orc.exact_law(cfg, D + 1, dt, tt)
    p = softmax(tt[0], T)
    pc = np.stack([softmax(tt[orc.ctx_index(V, [a])], T) for a in range(V)])
    return float(np.abs(law1 - p).max()), float(np.abs(law2 - p[:, None] * pc).max()), float(law1.sum())


@pytest.mark.parametrize("name,kw,seed", CONFIGS, ids=[c[0] for c in CONFIGS])
def test_exact_first_and_two_token_laws_are_the_target(name, kw, seed):
    e1, e2, tot = laws_match(kw, seed)
    assert abs(tot - 1.0) <= TOL, tot
    assert e1 <= TOL, e1
    assert e2 <= TOL, e2


DEPTH1 = [
    ("probe_first_m1", dict(V=8, trunc=8, K=3, m=1, T=1.0), 11),
    ("probe_first_m0_T06", dict(V=8, trunc=8, K=3, m=0, T=0.6), 12),
    ("probe_first_m3_trunc6", dict(V=8, trunc=6, K=4, m=3, T=1.0), 13),
    ("probe_first_trunc4", dict(V=7, trunc=4, K=3, m=1, T=0.8), 14),
    ("probe_off", dict(V=8, trunc=8, K=3, m=0, probe=0, T=1.0), 15),
    ("probe_last_m1", dict(V=8, trunc=8, K=3, m=1, T=1.0, order=orc.PROBE_LAST), 16),
    ("probe_last_trunc5_T06", dict(V=8, trunc=5, K=3, m=0, T=0.6, order=orc.PROBE_LAST), 17),
    ("dense_m1", dict(V=8, trunc=orc.DENSE, K=3, m=1, T=1.0), 18),
    ("dense_m0_T06", dict(V=7, trunc=orc.DENSE, K=4, m=0, T=0.6), 19),
    ("dense_probe_last", dict(V=8, trunc=orc.DENSE, K=3, m=1, T=0.8, order=orc.PROBE_LAST), 20),
]


def depth1_gap(kw, seed):
    """|exact P(first token from the tree) - closed form| at depth 1 (every child kept)."""
    cfg = orc.make_cfg(D=1, W=0, R=kw["K"], **kw)
    dt, tt = tables(kw["V"], 1, seed)
    _, _, acc = orc.exact_law(cfg, 2, dt, tt, two=False)
    if kw["trunc"] == orc.DENSE:  # the closed form's support: every token
        cfg = orc.make_cfg(D=1, W=0, R=kw["K"], **dict(kw, trunc=kw["V"]))
    closed = _depth1_rrsw(cfg, dt[0], tt[0]) if kw.get("order") == orc.PROBE_LAST else \
        _depth1_acceptance(cfg, dt[0], tt[0])
    return abs(acc - closed), acc


@pytest.mark.parametrize("name,kw,seed", DEPTH1, ids=[c[0] for c in DEPTH1])
def test_exact_depth1_acceptance_is_the_closed_form(name, kw, seed):
    gap, acc = depth1_gap(kw, seed)
    assert 0.0 < acc <= 1.0
    assert gap <= TOL, (gap, acc)


def test_acceptance_rises_with_the_tree():
    """Not a law: a deeper, wider tree accepts at least as often at the root as its
    depth-1 top slice does here (more kept children at the root under the same prune)."""
    kw = dict(V=8, trunc=8, K=3, m=1, T=1.0)
    dt, tt = tables(8, 3, 21)
    _, _, a1 = orc.exact_law(orc.make_cfg(D=1, W=0, R=1, **kw), 4, dt, tt, two=False)
    _, _, a3 = orc.exact_law(orc.make_cfg(D=1, W=0, R=3, **kw), 4, dt, tt, two=False)
    assert a3 >= a1 - TOL


def exact_ok():
    """The exact pins on a few configurations (for the planted-mistake tests)."""
    for name, kw, seed in (CONFIGS[0], CONFIGS[1], CONFIGS[4], CONFIGS[5], CONFIGS[9], CONFIGS[12]):
        e1, e2, tot = laws_match(kw, seed)
        if not (abs(tot - 1.0) <= TOL and e1 <= TOL and e2 <= TOL):
            return False
    for name, kw, seed in DEPTH1:
        if depth1_gap(kw, seed)[0] > TOL:
            return False
    return True
