"""The pins have power: each test plants one plausible mistake in a copy of the
oracle's source (on the CPU), builds it, and checks that a pin now fails while
the unmodified oracle passes the same check."""
import os
import shutil

import numpy as np
import pytest
from scipy.stats import chisquare

from oracle import build as obuild
from oracle import oracle as orc

SRC = os.path.join(os.path.dirname(obuild.__file__), "vrt_oracle.c")
V = 16


def _tables(D, seed):
    n = sum(V ** k for k in range(D + 2))
    rng = np.random.default_rng(seed)
    dt = (rng.normal(size=(n, V)) * 1.5).astype(np.float32)
    tt = (dt + rng.normal(size=(n, V)) * 0.8).astype(np.float32)
    return dt, tt


def _softmax(x, T):
    invT = np.float64(np.float32(1.0) / np.float32(T))
    e = np.exp((x.astype(np.float64) - x.max()) * invT)
    return e / e.sum()


def lossless_ok(T=1.0, m=1, trials=200_000):
    cfg = orc.make_cfg(V=V, trunc=16, K=3, m=m, D=2, W=3, R=6, T=T)
    dt, tt = _tables(2, 5)
    out, nf, _ = orc.table_trials(cfg, 2, dt, tt, 4242, 0, 0, trials)
    p = _softmax(tt[0], T)
    obs = np.bincount(out[:, 0], minlength=V).astype(np.float64)
    return chisquare(obs, p * obs.sum()).pvalue > 0.01


def acceptance_ok(trials=200_000):
    from tests.test_oracle_lossless import _depth1_acceptance
    cfg = orc.make_cfg(V=V, trunc=16, K=4, m=1, D=1, R=4, T=1.0)
    dt, tt = _tables(1, 78)
    out, nf, _ = orc.table_trials(cfg, 1, dt, tt, 4343, 0, 0, trials)
    P = _depth1_acceptance(cfg, dt[0], tt[0])
    z = ((nf >= 1).mean() - P) / np.sqrt(P * (1 - P) / trials)
    return abs(z) < 4.0


def rrsw_lossless_ok(trials=200_000):
    cfg = orc.make_cfg(V=V, trunc=16, K=4, m=1, D=2, W=3, R=6, T=1.0, order=orc.PROBE_LAST)
    dt, tt = _tables(2, 6)
    out, nf, _ = orc.table_trials(cfg, 2, dt, tt, 4545, 0, 0, trials)
    p = _softmax(tt[0], 1.0)
    obs = np.bincount(out[:, 0], minlength=V).astype(np.float64)
    return chisquare(obs, p * obs.sum()).pvalue > 0.01


def rrsw_acceptance_ok(trials=200_000):
    from tests.test_oracle_rrsw import _depth1_rrsw
    cfg = orc.make_cfg(V=V, trunc=16, K=4, m=1, D=1, R=4, T=1.0, order=orc.PROBE_LAST)
    dt, tt = _tables(1, 79)
    out, nf, _ = orc.table_trials(cfg, 1, dt, tt, 4646, 0, 0, trials)
    P = _depth1_rrsw(cfg, dt[0], tt[0])
    z = ((nf >= 1).mean() - P) / np.sqrt(P * (1 - P) / trials)
    return abs(z) < 4.0


def slots_ok():
    from tests.test_oracle_units import test_expansion_probabilities_and_slots
    try:
        for m in (0, 1, 3):
            test_expansion_probabilities_and_slots(m, 1.0)
    except AssertionError:
        return False
    return True


def support_ok():
    from tests.test_oracle_units import test_support_matches_lexsort
    try:
        test_support_matches_lexsort(1000, 128)
    except AssertionError:
        return False
    return True


def smart_ok():
    from tests import test_oracle_smart as ts
    try:
        ts.test_linear_cost_keeps_above_average_gain()
        ts.test_two_layers_hand_worked()
    except AssertionError:
        return False
    return True


def topr_ok():
    from tests import test_oracle_topr as tt
    return all(tt.hand_case_ok(n) for n in tt.CASES) and tt.invariants_ok(200)


def dense_ok():
    from tests import test_oracle_dense as td
    try:
        td.test_dense_probabilities_slots_and_proxy(1, 1.0, 0)
        td.test_dense_probabilities_slots_and_proxy(1, 1.0, 1)
        td.test_dense_probe_draw_follows_the_tempered_tail(1.0, 0)
    except AssertionError:
        return False
    return True


MUTANTS = [
    ("residual_mass_ignores_overlap", "    W = 1.0 - overlap;", "    W = 1.0;",
     lambda: lossless_ok() and acceptance_ok()),
    ("probe_ratio_inverted", "const double a = w[token[probe]] / qs;",
     "const double a = qs / w[token[probe]];", lambda: lossless_ok() and acceptance_ok()),
    ("tail_residual_not_clipped",
     "      overlap += (p < q) ? p : q;\n      w[y] = (p > q) ? p - q : 0.0;\n    }\n    W = 1.0 - overlap;",
     "      overlap += (p < q) ? p : q;\n      w[y] = p;\n    }\n    W = 1.0 - overlap;",
     lambda: lossless_ok() and acceptance_ok()),
    ("rejected_sibling_not_removed", "    W -= wx;\n    w[xt] = 0.0;", "    W -= wx;",
     lambda: lossless_ok() and acceptance_ok()),
    ("verify_ignores_temperature", "w[v] = exp(((double)x[v] - (double)M) * invT);",
     "w[v] = exp((double)x[v] - (double)M);", lambda: lossless_ok(T=0.6)),
    ("tail_mass_includes_top_m", "for (int32_t i = t0; i < n; ++i) zT += e->q_T[i];",
     "for (int32_t i = 0; i < n; ++i) zT += e->q_T[i];", lambda: slots_ok() and lossless_ok()),
    ("proxy_takes_max", "return e->q_raw[t0 - 1] < e->z_raw ? e->q_raw[t0 - 1] : e->z_raw;",
     "return e->q_raw[t0 - 1] > e->z_raw ? e->q_raw[t0 - 1] : e->z_raw;", slots_ok),
    # probe last (the RRSw baseline)
    ("probe_last_ratio_ignores_residual_mass", "const double a = w[token[probe]] / (W * qs);",
     "const double a = w[token[probe]] / qs;", lambda: rrsw_lossless_ok() and rrsw_acceptance_ok()),
    ("probe_last_tail_not_scaled", "const double q = W * tail_q[(int64_t)i * tail_cap + k];",
     "const double q = tail_q[(int64_t)i * tail_cap + k];",
     lambda: rrsw_lossless_ok() and rrsw_acceptance_ok()),
    ("probe_last_tail_includes_fillers",
     "const int32_t t0 = c->order == ORC_PROBE_LAST ? (c->K - 1 < n ? c->K - 1 : n) : m;",
     "const int32_t t0 = m;", lambda: rrsw_lossless_ok() and rrsw_acceptance_ok()),
    ("fillers_repeat_probe", "if (i != js) add_child", "if (i >= 0) add_child", slots_ok),
    ("support_tie_break_reversed", "return (x->id < y->id) ? -1 : (x->id > y->id);",
     "return (x->id > y->id) ? -1 : (x->id < y->id);", support_ok),
    # the dense baseline (support = the whole vocabulary)
    ("dense_tail_includes_deterministic", "for (int32_t i = 0; i < t0; ++i) det[ids[i]] = 1;",
     "for (int32_t i = 0; i < 0; ++i) det[ids[i]] = 1;", dense_ok),
    ("dense_raw_tail_mass_is_everything", "e->z_raw = pairwise(tx, V) / E;",
     "e->z_raw = pairwise(ex, V) / E;", dense_ok),
    ("dense_draw_walks_deterministic_tokens", "      if (det[v]) continue;\n      before = cum;",
     "      before = cum;", dense_ok),
    ("dense_fillers_repeat_probe", "if (ids[i] != s) add_child", "if (ids[i] >= 0) add_child",
     dense_ok),
    ("dense_tail_q_not_renormalised",
     "for (int32_t v = 0; v < V; ++v) e->dense_q[v] = det[v] ? 0.0 : et[v] / zT;",
     "for (int32_t v = 0; v < V; ++v) e->dense_q[v] = det[v] ? 0.0 : et[v] / Z;", lambda: exact_ok()),
    ("dense_tail_mass_includes_deterministic", "    if (!det[v]) zT += et[v];", "    zT += et[v];",
     dense_ok),
    ("dense_view_tail_shifted", "        tail_q[(int64_t)i * tail_cap + k] = e->dense_q[v];",
     "        tail_q[(int64_t)i * tail_cap + k] = e->dense_q[(v + 1) % t->cfg.V];", lambda: exact_ok()),
    # the per-layer beam and the global top-R prune (every check stops at the first wrong
    # frontier, so a frontier longer than W is never expanded)
    ("node_tie_break_reversed", "  return (x < y) ? -1 : (x > y);",
     "  return (x > y) ? -1 : (x < y);", topr_ok),
    ("beam_frontier_one_extra", "k < n && k < W; ++k", "k < n && k <= W; ++k", topr_ok),
    ("beam_ranks_earlier_layers", "  const int32_t base = orc_layer_base(t, layer);",
     "  const int32_t base = 0;", topr_ok),
    ("prune_keeps_one_extra", "k < n && k < c->R; ++k", "k < n && k <= c->R; ++k", topr_ok),
    ("smart_leaf_count_inverted", "if (t->has_child[par + 1]) t->n_paths += 1;",
     "if (!t->has_child[par + 1]) t->n_paths += 1;", smart_ok),
]


def exact_ok():
    from tests.test_oracle_exact import exact_ok as ok
    return ok()


# the verification mistakes (and the build's tail mass and the dense probe's tail, which
# the probe's law and its test depend on), each also caught by the exact enumeration of the
# first- and two-token laws and of the depth-1 acceptance: no statistics involved
EXACT = ["residual_mass_ignores_overlap", "probe_ratio_inverted", "tail_residual_not_clipped",
         "rejected_sibling_not_removed", "verify_ignores_temperature",
         "probe_last_ratio_ignores_residual_mass", "probe_last_tail_not_scaled",
         "probe_last_tail_includes_fillers", "tail_mass_includes_top_m",
         "dense_tail_q_not_renormalised", "dense_tail_mass_includes_deterministic",
         "dense_view_tail_shifted"]


def _planted(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, name
    mut = tmp_path / "vrt_oracle.c"
    mut.write_text(src.replace(old, new))
    shutil.copy(os.path.join(os.path.dirname(SRC), "vrt_oracle.h"), tmp_path / "vrt_oracle.h")
    return obuild.build(src=str(mut), out=str(tmp_path / f"liboracle_{name}.so"))


@pytest.mark.parametrize("name", EXACT)
def test_exact_law_catches_planted_mistake(tmp_path, name):
    old, new = {m[0]: (m[1], m[2]) for m in MUTANTS}[name]
    assert exact_ok(), "the unmodified oracle must pass the exact pins"
    with orc.using(_planted(tmp_path, name, old, new)):
        assert not exact_ok(), f"planted mistake {name} went unnoticed by the exact enumeration"


@pytest.mark.parametrize("name,old,new,check", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pin_catches_planted_mistake(tmp_path, name, old, new, check):
    src = open(SRC).read()
    assert src.count(old) == 1, name
    assert check(), "the unmodified oracle must pass the check"
    mut = tmp_path / "vrt_oracle.c"
    mut.write_text(src.replace(old, new))
    shutil.copy(os.path.join(os.path.dirname(SRC), "vrt_oracle.h"), tmp_path / "vrt_oracle.h")
    lib = obuild.build(src=str(mut), out=str(tmp_path / f"liboracle_{name}.so"))
    with orc.using(lib):
        assert not check(), f"planted mistake {name} went unnoticed"
