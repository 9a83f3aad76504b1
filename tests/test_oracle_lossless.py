"""Losslessness and acceptance pins for the oracle's tree build + verification.

* Chi-square (p > 0.01, 10^6 trials, V = 16): the first emitted token follows the
  target softmax at the root, and the first two tokens follow the product of the
  target softmaxes at the root and at the first token's context (RheoSampling:
  losslessness for any prune budget R, in its highlights and summary).
* Closed-form depth-1 acceptance, derived here from key design 3: the probe is
  accepted with min(1, p/q~); after a rejection the kept siblings are accepted
  with total probability sum_{x in D(s)} w(x)/W0, w = max(0, p - q~) on the tail
  and p elsewhere, W0 = 1 - sum_tail min(p, q~). Compared by a z-test.
* Special cases: K=1, m=0 is textbook speculative sampling (acceptance
  sum_v min(p, q)); draft = target gives acceptance 1; probe off is the
  point-mass top-K verifier (acceptance p(D)).
"""
import numpy as np
import pytest
from scipy.stats import chisquare

from oracle import oracle as orc

V = 16
N_TRIALS = 1_000_000


def _tables(D, seed, scale=1.5, noise=0.8, identity=False):
    n = sum(V ** k for k in range(D + 2))
    rng = np.random.default_rng(seed)
    dt = (rng.normal(size=(n, V)) * scale).astype(np.float32)
    tt = dt.copy() if identity else (dt + rng.normal(size=(n, V)) * noise).astype(np.float32)
    return dt, tt


def _softmax(x, T):
    invT = np.float64(np.float32(1.0) / np.float32(T))
    e = np.exp((x.astype(np.float64) - np.float64(x.max())) * invT)
    return e / e.sum()


def _chi2(obs, exp):
    keep = exp >= 5
    o = np.append(obs[keep], obs[~keep].sum())
    e = np.append(exp[keep], exp[~keep].sum())
    if e[-1] == 0:
        o, e = o[:-1], e[:-1]
    return chisquare(o, e * (o.sum() / e.sum())).pvalue


LOSSLESS_CASES = [
    # name, cfg kwargs, table seed
    ("m1_T1", dict(trunc=16, K=3, m=1, D=3, W=3, R=8, T=1.0), 10),
    ("m0_T06", dict(trunc=16, K=3, m=0, D=3, W=3, R=8, T=0.6), 11),
    ("m3_T1", dict(trunc=16, K=5, m=3, D=2, W=3, R=8, T=1.0), 12),
    ("trunc4_m1", dict(trunc=4, K=3, m=1, D=3, W=2, R=6, T=1.0), 13),
    ("trunc4_m0_T06", dict(trunc=4, K=2, m=0, D=3, W=2, R=5, T=0.6), 14),
    ("probe_off", dict(trunc=16, K=3, m=1, probe=0, D=3, W=3, R=8, T=1.0), 15),
    ("tiny_R", dict(trunc=8, K=4, m=1, D=3, W=4, R=2, T=1.0), 16),
]


@pytest.mark.slow
@pytest.mark.parametrize("name,kw,seed", LOSSLESS_CASES, ids=[c[0] for c in LOSSLESS_CASES])
def test_first_token_follows_target_softmax(name, kw, seed):
    cfg = orc.make_cfg(V=V, **kw)
    dt, tt = _tables(kw["D"], seed)
    out, nf, ne = orc.table_trials(cfg, kw["D"], dt, tt, 1000 + seed, 0, 0, N_TRIALS)
    p = _softmax(tt[orc.ctx_index(V, [])], kw["T"])
    obs = np.bincount(out[:, 0], minlength=V).astype(np.float64)
    pv = _chi2(obs, p * N_TRIALS)
    assert pv > 0.01, (name, pv)
    assert nf.mean() > 0.3  # the tree actually contributes tokens


@pytest.mark.slow
@pytest.mark.parametrize("kw,seed", [(dict(trunc=16, K=3, m=1, D=2, W=3, R=6, T=1.0), 21),
                                     (dict(trunc=4, K=3, m=0, D=2, W=2, R=5, T=0.6), 22)])
def test_first_two_tokens_follow_target_chain(kw, seed):
    cfg = orc.make_cfg(V=V, **kw)
    D = kw["D"]
    dt, tt = _tables(D, seed)
    out, nf, ne = orc.table_trials(cfg, D + 1, dt, tt, 2000 + seed, 0, 0, N_TRIALS, two=True)
    p1 = _softmax(tt[orc.ctx_index(V, [])], kw["T"])
    joint = np.zeros((V, V))
    for a in range(V):
        joint[a] = p1[a] * _softmax(tt[orc.ctx_index(V, [a])], kw["T"])
    obs = np.zeros((V, V))
    np.add.at(obs, (out[:, 0], out[:, 1]), 1)
    pv = _chi2(obs.ravel(), joint.ravel() * N_TRIALS)
    assert pv > 0.01, pv


def _depth1_acceptance(cfg, draft, target):
    """Closed-form P(first token comes from the tree) at the root, depth 1."""
    T, m, K, trunc, probe = cfg.T, cfg.m, cfg.K, cfg.trunc, cfg.probe
    V = draft.size
    order = np.lexsort((np.arange(V), -draft.astype(np.float64)))[:min(trunc, V)]
    lv = draft[order].astype(np.float64)
    invT = np.float64(np.float32(1.0) / np.float32(T))
    qT = np.exp((lv - lv.max()) * invT)
    qT /= qT.sum()
    p = _softmax(target, T)
    if not probe:
        return p[order[:K]].sum()
    tail = order[m:]
    zT = qT[m:].sum()
    qt = np.zeros(V)
    qt[tail] = qT[m:] / zT
    w = np.where(qt > 0, np.maximum(0.0, p - qt), p)
    W0 = 1.0 - np.minimum(p, qt)[tail].sum()
    total = 0.0
    for j, s in enumerate(tail):
        fillers = [t for t in tail if t != s][:K - m - 1]
        Dset = list(order[:m]) + fillers
        a = min(1.0, p[s] / qt[s])
        total += qt[s] * (a + (1 - a) * sum(w[x] for x in Dset) / W0)
    return total


def _z_test(cfg, dt, tt, seed):
    out, nf, ne = orc.table_trials(cfg, 1, dt, tt, seed, 0, 0, N_TRIALS)
    phat = (nf >= 1).mean()
    P = _depth1_acceptance(cfg, dt[0], tt[0])
    if P >= 1.0 - 1e-12:
        return phat, P, 0.0
    z = (phat - P) / np.sqrt(P * (1 - P) / N_TRIALS)
    return phat, P, z


@pytest.mark.slow
@pytest.mark.parametrize("kw,seed", [
    (dict(trunc=16, K=4, m=1, T=1.0), 31),
    (dict(trunc=16, K=4, m=0, T=0.6), 32),
    (dict(trunc=8, K=5, m=3, T=1.0), 33),
    (dict(trunc=6, K=3, m=1, T=1.0), 34),
    (dict(trunc=16, K=4, m=1, probe=0, T=1.0), 35),
])
def test_depth1_acceptance_matches_closed_form(kw, seed):
    cfg = orc.make_cfg(V=V, D=1, W=0, R=kw["K"], **kw)
    dt, tt = _tables(1, seed)
    phat, P, z = _z_test(cfg, dt, tt, 3000 + seed)
    assert abs(z) < 4.0, (phat, P, z)


@pytest.mark.slow
def test_textbook_speculative_sampling_case():
    # one probe slot and m = 0: the probe is a plain draft sample, accepted with
    # total probability sum_v min(p(v), q(v)) (standard speculative sampling)
    cfg = orc.make_cfg(V=V, trunc=16, K=1, m=0, D=1, R=1, T=0.8)
    dt, tt = _tables(1, 41)
    out, nf, ne = orc.table_trials(cfg, 1, dt, tt, 4100, 0, 0, N_TRIALS)
    q = _softmax(dt[0], 0.8)
    p = _softmax(tt[0], 0.8)
    P = np.minimum(p, q).sum()
    phat = (nf >= 1).mean()
    assert abs(phat - P) / np.sqrt(P * (1 - P) / N_TRIALS) < 4.0, (phat, P)
    obs = np.bincount(out[:, 0], minlength=V).astype(np.float64)
    assert _chi2(obs, p * N_TRIALS) > 0.01


def test_identity_draft_equals_target_always_accepts():
    for m, K in [(1, 3), (2, 4), (1, 2)]:
        cfg = orc.make_cfg(V=V, trunc=16, K=K, m=m, D=1, R=K, T=1.0)
        dt, tt = _tables(1, 50 + m, identity=True)
        out, nf, ne = orc.table_trials(cfg, 1, dt, tt, 5000 + m, 0, 0, 100_000)
        assert (nf >= 1).all()


def test_rheo_verification_beats_point_mass_topk_at_depth1():
    # qualitative ordering of the depth-1 controlled experiment: probe-first
    # verification accepts more than the deterministic top-K tree of equal size
    wins = 0
    for seed in range(40):
        dt, tt = _tables(1, 600 + seed)
        on = _depth1_acceptance(orc.make_cfg(V=V, trunc=16, K=3, m=1, D=1, R=3, T=1.0), dt[0], tt[0])
        off = _depth1_acceptance(orc.make_cfg(V=V, trunc=16, K=3, m=1, probe=0, D=1, R=3, T=1.0),
                                 dt[0], tt[0])
        wins += on > off
    assert wins >= 30
