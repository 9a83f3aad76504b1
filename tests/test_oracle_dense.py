"""Pins of the oracle's dense baseline and support coverage (RheoSampling, the
support-size ablation: full-vocabulary softmax and sampling against truncation to the
top 128/256/512/1024 logits).

The dense expansion is pinned against fp64 numpy softmaxes and a lexsort of the row,
its probe draw by a chi-square test against the tempered tail, its verification by
losslessness on a context-table model, and its topology by the truncated path with a
support of the whole row (probe off). Coverage is pinned by closed forms (uniform and
geometric rows) and by a numpy sort."""
import numpy as np
import pytest
from scipy.stats import chisquare

from oracle import oracle as orc

DENSE = orc.DENSE


def _bf16(x):
    b = np.asarray(x, np.float32).view(np.uint32)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(np.float32)


def _ranks(row):
    return np.lexsort((np.arange(row.size), -row.astype(np.float64)))


def _softmax(x, T=1.0):
    invT = np.float64(np.float32(1.0) / np.float32(T))
    e = np.exp((x.astype(np.float64) - x.max()) * invT)
    return e / e.sum()


def _root(row, K, m, T=1.0, seed=7, step=0, order=orc.PROBE_FIRST, probe=1, trunc=DENSE):
    cfg = orc.make_cfg(V=row.size, trunc=trunc, K=K, m=m, probe=probe, D=1, R=K, T=T, order=order)
    t = orc.Tree(cfg, seed, 0, step)
    t.expand_layer(0, row[None])
    t.finish()
    return t


# ---------------------------------------------------------------------------------
# coverage

@pytest.mark.parametrize("V,trunc", [(1000, 128), (5000, 1024), (300, 512), (7, 128)])
def test_coverage_of_a_uniform_row_is_the_support_share(V, trunc):
    row = np.full(V, 0.25, np.float32)
    assert abs(orc.support_mass(row, trunc) - min(trunc, V) / V) < 1e-14


def test_coverage_of_a_geometric_row():
    # logits -a*k at a random permutation: the top n hold (1 - r^n) / (1 - r^V), r = e^-a
    rng = np.random.default_rng(3)
    V, a = 4000, 0.01
    ids = rng.permutation(V)
    row = np.empty(V, np.float32)
    row[ids] = (-a * np.arange(V)).astype(np.float32)
    k = -row[ids].astype(np.float64)  # the exact exponents the row holds
    for n in (128, 256, 512, 1024):
        r = np.exp(-k)
        ref = r[:n].sum() / r.sum()
        assert abs(orc.support_mass(row, n) - ref) < 1e-12
        closed = (1 - np.exp(-a * n)) / (1 - np.exp(-a * V))
        assert abs(orc.support_mass(row, n) - closed) < 1e-6  # float32 logits


def test_coverage_matches_a_sort_and_edge_rows():
    rng = np.random.default_rng(4)
    for it in range(20):
        V = int(rng.integers(50, 6000))
        row = _bf16(rng.normal(size=V) * float(rng.choice([0.5, 2.0, 6.0])))
        p = _softmax(row)
        for n in (1, 128, 1024):
            ref = np.sort(p)[::-1][:n].sum()
            assert abs(orc.support_mass(row, n) - ref) < 1e-12
    row = np.full(10, -np.inf, np.float32)
    assert orc.support_mass(row, 4) == 0.0
    row[3] = 1.0
    assert orc.support_mass(row, 1) == 1.0
    row = np.array([0.0, -np.inf, 0.0, -np.inf], np.float32)
    assert abs(orc.support_mass(row, 1) - 0.5) < 1e-15


# ---------------------------------------------------------------------------------
# dense expansion

@pytest.mark.parametrize("m,T,order", [(1, 1.0, 0), (0, 1.0, 0), (3, 0.6, 0), (1, 1.0, 1), (2, 0.6, 1)])
def test_dense_probabilities_slots_and_proxy(m, T, order):
    rng = np.random.default_rng(10 + m)
    K = 8
    for seed in range(15):
        V = int(rng.integers(200, 3000))
        row = _bf16(rng.normal(size=V) * 2.0)
        t = _root(row, K, m, T, seed=seed, step=seed, order=order)
        e = t.row(0)
        assert e.n_sup == V
        ids = _ranks(row)
        np.testing.assert_array_equal(np.array(e.sup_id[:min(V, orc.MAXSUP)]), ids[:orc.MAXSUP])
        p = _softmax(row)
        pT = _softmax(row, T)
        keep = min(V, orc.MAXSUP)
        np.testing.assert_allclose(np.array(e.q_raw[:keep], np.float64), p[ids[:keep]], rtol=3e-6,
                                   atol=1e-12)
        np.testing.assert_allclose(np.array(e.q_T[:keep]), pT[ids[:keep]], rtol=1e-12)
        t0 = K - 1 if order == orc.PROBE_LAST else m
        det = ids[:t0]
        tail = np.setdiff1d(np.arange(V), det)
        assert abs(e.z_raw - p[tail].sum()) < 3e-6
        assert abs(e.z_T - pT[tail].sum()) < 1e-12
        kids = t.cands()[:K]
        kids = kids[kids["live"] == 1]
        toks = kids["token"]
        s = e.probe_token
        assert s >= 0 and s not in det.tolist()
        if order == orc.PROBE_LAST:
            assert kids["kind"].tolist() == [orc.DET] * m + [orc.FILL] * (K - 1 - m) + [orc.PROBE]
            np.testing.assert_array_equal(toks[:K - 1], ids[:K - 1])
            assert toks[K - 1] == s
        else:
            assert kids["kind"].tolist() == [orc.DET] * m + [orc.PROBE] + [orc.FILL] * (K - m - 1)
            np.testing.assert_array_equal(toks[:m], ids[:m])
            assert toks[m] == s
            fill = [v for v in ids[m:] if v != s][:K - m - 1]
            np.testing.assert_array_equal(toks[m + 1:], fill)
        assert len(set(toks.tolist())) == len(toks)
        qr = np.array(e.q_raw[:K], np.float32)
        if t0 >= 1:
            assert e.proxy == min(qr[t0 - 1], np.float32(e.z_raw))
        else:
            assert e.proxy == min(np.float32(1.0), np.float32(qr[0] + np.float32(1e-6)))
        probe_kid = kids[kids["kind"] == orc.PROBE]
        assert probe_kid["score"][0] == np.float32(e.proxy)
        other = kids[kids["kind"] != orc.PROBE]
        np.testing.assert_array_equal(other["score"], np.array(e.q_raw[:len(other) + 1], np.float32)[
            [list(ids[:len(other) + 1]).index(x) for x in other["token"]]])


@pytest.mark.parametrize("T,order", [(1.0, 0), (0.6, 0), (1.0, 1)])
def test_dense_probe_draw_follows_the_tempered_tail(T, order):
    rng = np.random.default_rng(20)
    V, K, m = 40, 4, 1
    row = _bf16(rng.normal(size=V) * 1.5)
    t0 = K - 1 if order == orc.PROBE_LAST else m
    ids = _ranks(row)
    pT = _softmax(row, T)
    pT[ids[:t0]] = 0.0
    pT /= pT.sum()
    n = 20000
    obs = np.zeros(V)
    for step in range(n):
        e = _root(row, K, m, T, seed=99, step=step, order=order).row(0)
        obs[e.probe_token] += 1
    assert obs[ids[:t0]].sum() == 0
    live = pT > 0
    assert chisquare(obs[live], pT[live] * n).pvalue > 0.001


def test_dense_draw_is_inverse_cdf_in_token_order():
    # the draw is the first tail token (ascending id) whose cumulative tempered mass
    # exceeds u * z_T
    rng = np.random.default_rng(21)
    V, K, m = 300, 5, 2
    row = _bf16(rng.normal(size=V))
    ids = _ranks(row)
    for step in range(200):
        t = _root(row, K, m, 1.0, seed=5, step=step)
        e = t.row(0)
        w = _softmax(row)
        w[ids[:m]] = 0.0
        cdf = np.cumsum(w) / w.sum()
        ref = int(np.searchsorted(cdf, e.u, side="right"))
        if min(abs(cdf[max(ref - 1, 0)] - e.u), abs(cdf[min(ref, V - 1)] - e.u)) > 1e-9:
            assert e.probe_token == ref


def test_dense_without_probe_equals_the_whole_row_support():
    # probe off: the children are the top K of the row; a truncated support of all V
    # tokens gives the same tokens, and scores equal up to the pairwise sum's order
    rng = np.random.default_rng(22)
    for it in range(20):
        V = int(rng.integers(20, 1000))
        row = _bf16(rng.normal(size=V) * 2.0)
        a = _root(row, 10, 0, probe=0).cands()[:10]
        b = _root(row, 10, 0, probe=0, trunc=1024).cands()[:10]
        np.testing.assert_array_equal(a["token"], b["token"])
        np.testing.assert_array_equal(a["kind"], b["kind"])
        np.testing.assert_allclose(a["score"], b["score"], rtol=2e-6)
        np.testing.assert_array_equal(a["token"][a["live"] == 1], _ranks(row)[:min(10, V)])


def test_dense_view_holds_the_whole_tail():
    rng = np.random.default_rng(23)
    V, K, m, T = 200, 6, 1, 0.6
    row = _bf16(rng.normal(size=V))
    t = _root(row, K, m, T, seed=3)
    v = t.view()
    i = 0  # the root holds the probe's tail
    n = v["tail_n"][i]
    assert n == V - m
    ids = v["tail_id"][i, :n]
    q = v["tail_q"][i, :n]
    np.testing.assert_array_equal(ids, np.setdiff1d(np.arange(V), _ranks(row)[:m]))
    ref = _softmax(row, T)[ids]
    np.testing.assert_allclose(q, ref / ref.sum(), rtol=1e-12)


def _tables(D, seed, V):
    n = sum(V ** k for k in range(D + 2))
    rng = np.random.default_rng(seed)
    dt = (rng.normal(size=(n, V)) * 1.5).astype(np.float32)
    tt = (dt + rng.normal(size=(n, V)) * 0.8).astype(np.float32)
    return dt, tt


@pytest.mark.parametrize("T,order", [(1.0, 0), (0.6, 1)])
def test_dense_trees_verify_losslessly(T, order):
    V = 12
    cfg = orc.make_cfg(V=V, trunc=DENSE, K=4, m=1, D=2, W=3, R=6, T=T, order=order)
    dt, tt = _tables(2, 8, V)
    trials = 100_000
    out, nf, _ = orc.table_trials(cfg, 2, dt, tt, 777, 0, 0, trials)
    p = _softmax(tt[0], T)
    obs = np.bincount(out[:, 0], minlength=V).astype(np.float64)
    assert chisquare(obs, p * obs.sum()).pvalue > 0.001
    assert (nf >= 1).mean() > 0.3  # the tree is used
