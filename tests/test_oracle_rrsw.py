"""Pins of the oracle's probe-last order: the RRSw baseline of RheoSampling's key design 3
(recursive rejection without replacement: the deterministic kept children first, the probe
last) and its verification ablation (Top-K vanilla < Rheo + RRSw < Rheo +
RheoVerification).

Reading stated here (the pages fix the order, not the layout): with fillers, the probe is
drawn from the ranks after them (fillers chosen first), so no kept deterministic child lies
in the probe's tail; its proxy is min{q(last deterministic), mass after it}.

* Chi-square (p > 0.01, 10^6 trials, V = 16): first token, and first two tokens, follow the
  target softmax (losslessness).
* Closed form at depth 1, derived here: the deterministic set D (top m, then fillers) is
  accepted with total probability p(D) (point masses, each rejection renormalising); the
  probe s ~ q~' (tempered tail after D) with min(1, p_D(s)/q~'(s)), p_D = p / (1 - p(D)) off D:
  P = p(D) + sum_s min((1 - p(D)) q~'(s), p(s)). z-test.
* With no fillers (K = m + 1) both orders share one tree; probe first accepts at least as
  often as probe last (closed forms on random instances), and probe last beats the
  point-mass top-K tree.
* Draft = target: probe last always accepts.
"""
import numpy as np
import pytest

from oracle import oracle as orc
from tests.test_oracle_lossless import V, N_TRIALS, _tables, _softmax, _chi2, _depth1_acceptance

LAST = orc.PROBE_LAST


def _depth1_rrsw(cfg, draft, target):
    T, m, K, trunc = cfg.T, cfg.m, cfg.K, cfg.trunc
    V = draft.size
    order = np.lexsort((np.arange(V), -draft.astype(np.float64)))[:min(trunc, V)]
    lv = draft[order].astype(np.float64)
    invT = np.float64(np.float32(1.0) / np.float32(T))
    qT = np.exp((lv - lv.max()) * invT)
    qT /= qT.sum()
    p = _softmax(target, T)
    t0 = min(K - 1, order.size)
    pD = p[order[:t0]].sum()
    tail = order[t0:]
    if tail.size == 0:
        return pD
    qt = qT[t0:] / qT[t0:].sum()
    return pD + np.minimum((1.0 - pD) * qt, p[tail]).sum()


LOSSLESS = [
    ("fillers_m1", dict(trunc=16, K=4, m=1, D=3, W=3, R=8, T=1.0), 70),
    ("fillers_m0_T06", dict(trunc=16, K=3, m=0, D=3, W=3, R=8, T=0.6), 71),
    ("no_fillers_m2", dict(trunc=16, K=3, m=2, D=2, W=3, R=6, T=1.0), 72),
    ("trunc4", dict(trunc=4, K=3, m=1, D=3, W=2, R=6, T=1.0), 73),
    ("K1_m0", dict(trunc=16, K=1, m=0, D=3, W=1, R=3, T=0.8), 74),
]


@pytest.mark.slow
@pytest.mark.parametrize("name,kw,seed", LOSSLESS, ids=[c[0] for c in LOSSLESS])
def test_probe_last_first_token_follows_target_softmax(name, kw, seed):
    cfg = orc.make_cfg(V=V, order=LAST, **kw)
    dt, tt = _tables(kw["D"], seed)
    out, nf, ne = orc.table_trials(cfg, kw["D"], dt, tt, 7000 + seed, 0, 0, N_TRIALS)
    p = _softmax(tt[orc.ctx_index(V, [])], kw["T"])
    obs = np.bincount(out[:, 0], minlength=V).astype(np.float64)
    assert _chi2(obs, p * N_TRIALS) > 0.01, name
    assert nf.mean() > 0.3


@pytest.mark.slow
def test_probe_last_first_two_tokens_follow_target_chain():
    kw = dict(trunc=16, K=4, m=1, D=2, W=3, R=6, T=1.0)
    cfg = orc.make_cfg(V=V, order=LAST, **kw)
    dt, tt = _tables(2, 77)
    out, nf, ne = orc.table_trials(cfg, 3, dt, tt, 7700, 0, 0, N_TRIALS, two=True)
    p1 = _softmax(tt[orc.ctx_index(V, [])], 1.0)
    joint = np.zeros((V, V))
    for a in range(V):
        joint[a] = p1[a] * _softmax(tt[orc.ctx_index(V, [a])], 1.0)
    obs = np.zeros((V, V))
    np.add.at(obs, (out[:, 0], out[:, 1]), 1)
    assert _chi2(obs.ravel(), joint.ravel() * N_TRIALS) > 0.01


@pytest.mark.slow
@pytest.mark.parametrize("kw,seed", [(dict(trunc=16, K=4, m=1, T=1.0), 81),
                                     (dict(trunc=16, K=3, m=0, T=0.6), 82),
                                     (dict(trunc=8, K=5, m=2, T=1.0), 83)])
def test_probe_last_depth1_acceptance_matches_closed_form(kw, seed):
    cfg = orc.make_cfg(V=V, D=1, W=0, R=kw["K"], order=LAST, **kw)
    dt, tt = _tables(1, seed)
    out, nf, ne = orc.table_trials(cfg, 1, dt, tt, 8000 + seed, 0, 0, N_TRIALS)
    phat = (nf >= 1).mean()
    P = _depth1_rrsw(cfg, dt[0], tt[0])
    z = (phat - P) / np.sqrt(P * (1 - P) / N_TRIALS)
    assert abs(z) < 4.0, (phat, P, z)


def test_without_fillers_probe_first_dominates_probe_last():
    wins = ties = 0
    for seed in range(60):
        dt, tt = _tables(1, 900 + seed)
        for m, T in [(1, 1.0), (2, 0.6), (0, 1.0)]:
            K = m + 1
            first = _depth1_acceptance(orc.make_cfg(V=V, trunc=16, K=K, m=m, D=1, R=K, T=T), dt[0], tt[0])
            last = _depth1_rrsw(orc.make_cfg(V=V, trunc=16, K=K, m=m, D=1, R=K, T=T, order=LAST), dt[0], tt[0])
            assert first >= last - 1e-12, (seed, m, first, last)
            wins += first > last + 1e-12
            ties += abs(first - last) <= 1e-12
    assert wins >= 100  # m = 0 ties (no deterministic prefix): 60 of 180


def test_probe_last_beats_point_mass_topk():
    wins = 0
    for seed in range(40):
        dt, tt = _tables(1, 1000 + seed)
        last = _depth1_rrsw(orc.make_cfg(V=V, trunc=16, K=3, m=1, D=1, R=3, T=1.0, order=LAST), dt[0], tt[0])
        top = _depth1_acceptance(orc.make_cfg(V=V, trunc=16, K=3, m=1, probe=0, D=1, R=3, T=1.0), dt[0], tt[0])
        wins += last > top
    assert wins >= 30


def test_probe_last_identity_always_accepts():
    for m, K in [(1, 3), (0, 3), (2, 3)]:
        cfg = orc.make_cfg(V=V, trunc=16, K=K, m=m, D=1, R=K, T=1.0, order=LAST)
        dt, tt = _tables(1, 60 + m, identity=True)
        out, nf, ne = orc.table_trials(cfg, 1, dt, tt, 6000 + m, 0, 0, 100_000)
        assert (nf >= 1).all()


def test_probe_last_tree_layout():
    """Slots: top m DET, then the fillers (ranks m .. K-2), then the probe from ranks >= K-1;
    the proxy is min{q(x_{K-1}), the raw mass after it}."""
    rng = np.random.default_rng(3)
    row = (rng.normal(size=V) * 2).astype(np.float32)
    cfg = orc.make_cfg(V=V, trunc=16, K=5, m=1, D=1, R=5, T=1.0, order=LAST)
    t = orc.Tree(cfg, seed=9, b=0, step=0)
    t.expand_layer(0, row[None, :])
    cands = t.cands()
    kinds = [int(c["kind"]) for c in cands[:5]]
    assert kinds == [orc.DET, orc.FILL, orc.FILL, orc.FILL, orc.PROBE]
    ids, vals = orc.support(row, 16)
    assert [int(c["token"]) for c in cands[:4]] == list(ids[:4])
    assert int(cands[4]["token"]) in set(ids[4:].tolist())
    ex = t.row(0)
    qr = np.array(ex.q_raw[:16], np.float32)
    z = np.float32(ex.z_raw)
    assert np.float32(ex.proxy) == min(qr[3], z)
    assert abs(float(z) - float(qr[4:].sum())) < 1e-6
