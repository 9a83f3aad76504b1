"""Pins of the oracle's per-layer beam and global top-R prune (RheoSampling framework
flowchart: the tree grows layer by layer from the current candidates and is cut to the
R best nodes by path score; its settings use R = 60 at depth 8).

Two kinds of pin, neither of which reuses the oracle's own sort:
  * hand-worked trees whose draft rows put exactly 1, 2 or 4 tokens at the row maximum and
    the rest at -inf, so every ranking probability is 1, 1/2 or 1/4, every path product is
    exact and the probe draw has a single possible outcome; the expected frontiers and the
    emitted tree (creation indices, tokens, parents, child lists, tails) are written out by
    hand below, including score ties broken by creation index, W < K, an R that cuts
    inside a layer and R < K;
  * invariants over 10^4 random small configurations with tie-heavy rows: each layer's
    frontier is the first min(W, n) of that layer's candidates in (score desc, creation
    index asc) order as numpy's lexsort gives it, the emitted nodes are the first R of all
    candidates in that order, every kept node's parent is kept and precedes it, a child's
    score never exceeds its parent's, siblings carry distinct tokens, child lists follow
    slot order and tails belong exactly to nodes whose probe child is kept.
"""
import numpy as np
import pytest

from oracle import oracle as orc

NEG = -np.inf


def _row(V, top):
    """A draft row with logit 0 at the given token ids and -inf elsewhere."""
    r = np.full(V, NEG, np.float32)
    r[list(top)] = 0.0
    return r


def _path(cands, c):
    out = []
    while c >= 0:
        out.append(int(cands[c]["token"]))
        c = int(cands[c]["parent"])
    return tuple(reversed(out))


def build(cfg, row_of_path, expect_fronts=None):
    """Build one tree layer by layer; row_of_path(path) gives the draft row of the node
    reached by that token path (the root: ()). With expect_fronts, stop at the first
    frontier that differs (so that a wrong frontier is never expanded) and return None."""
    t = orc.Tree(cfg, 7, 0, 0)
    front = [-1]
    fronts = []
    for layer in range(cfg.D):
        if not front:
            break
        cands = t.cands()
        rows = np.stack([row_of_path(_path(cands, c)) for c in front])
        t.expand_layer(layer, rows)
        front = [int(x) for x in t.frontier()]
        fronts.append(front)
        if expect_fronts is not None and (layer >= len(expect_fronts) or front != expect_fronts[layer]):
            return None, fronts
    t.finish()
    return t, fronts


# ---------------------------------------------------------------------------------
# Hand-worked trees

def _case_a():
    """Probe off, V=8, K=3, W=2, D=3, R=7.

    root () : tokens {2, 5} at 0    -> c0 (2, 1/2), c1 (5, 1/2), c2 (0, 0)
    beam    : c0, c1 tie at 1/2     -> front [0, 1] (creation index breaks the tie)
    (2)     : tokens {1, 3, 4, 6}   -> c3 (1, 1/8), c4 (3, 1/8), c5 (4, 1/8)
    (5)     : token {7}             -> c6 (7, 1/2), c7 (0, 0), c8 (1, 0)
    beam    : c6 1/2 > c3 1/8 = c4 = c5 -> front [6, 3]
    (5, 7)  : tokens {0, 7}         -> c9 (0, 1/4), c10 (7, 1/4), c11 (1, 0)
    (2, 1)  : token {3}             -> c12 (3, 1/8), c13 (0, 0), c14 (1, 0)
    prune   : c0 c1 c6 (1/2), c9 c10 (1/4), c3 c4 | c5 c12 (1/8), zeros -> R = 7 cuts the
              1/8 ties after c4.
    """
    V = 8
    rows = {(): [2, 5], (2,): [1, 3, 4, 6], (5,): [7], (5, 7): [0, 7], (2, 1): [3]}
    cfg = orc.make_cfg(V=V, trunc=8, K=3, m=0, probe=0, D=3, W=2, R=7)
    expect = dict(
        fronts=[[0, 1], [6, 3], []],
        cand=[-1, 0, 1, 6, 9, 10, 3, 4],
        token=[-1, 2, 5, 7, 0, 7, 1, 3],
        parent=[-1, 0, 0, 2, 3, 3, 1, 1],
        depth=[0, 1, 1, 2, 3, 3, 2, 2],
        kind=[orc.ROOT] + [orc.DET] * 7,
        child_off=[0, 2, 4, 5, 7, 7, 7, 7, 7],
        child=[1, 2, 6, 7, 3, 4, 5],
        scores={0: 0.5, 1: 0.5, 2: 0.0, 3: 0.125, 4: 0.125, 5: 0.125, 6: 0.5, 9: 0.25, 10: 0.25,
                12: 0.125},
        tails={},
    )
    return cfg, (lambda p: _row(V, rows[p])), expect


def _case_b():
    """Probe on (m=1), V=8, K=3, W=2, D=2, R=2 < K.

    root () : tokens {3, 6}         -> DET c0 (3, 1/2); the tempered tail after rank 1 holds
              mass only at token 6, so the probe is c1 (6) whatever the draw, with proxy
              min(q(x_1), z) = min(1/2, 1/2); filler c2 = the next rank, token 0 (score 0)
    beam    : front [0, 1]
    (3)     : tokens {1, 5}         -> c3 (1, 1/4 DET), c4 (5, 1/4 PROBE), c5 (0, 0 FILL)
    (6)     : token {4}             -> no tail mass: no probe; c6 (4, 1/2 DET), c7 (0), c8 (1)
    prune   : c0, c1, c6 tie at 1/2; R = 2 keeps c0 and c1 (two of the root's three
              children). The root's probe child is kept: its tail is ranks 1..7 of the root
              support (token 6 with q~ = 1, then tokens 0, 1, 2, 4, 5, 7 with q~ = 0).
    """
    V = 8
    rows = {(): [3, 6], (3,): [1, 5], (6,): [4]}
    cfg = orc.make_cfg(V=V, trunc=8, K=3, m=1, probe=1, D=2, W=2, R=2)
    expect = dict(
        fronts=[[0, 1], []],
        cand=[-1, 0, 1],
        token=[-1, 3, 6],
        parent=[-1, 0, 0],
        depth=[0, 1, 1],
        kind=[orc.ROOT, orc.DET, orc.PROBE],
        child_off=[0, 2, 2, 2],
        child=[1, 2],
        scores={0: 0.5, 1: 0.5, 2: 0.0, 3: 0.25, 4: 0.25, 5: 0.0, 6: 0.5, 7: 0.0, 8: 0.0},
        tails={0: ([6, 0, 1, 2, 4, 5, 7], [1, 0, 0, 0, 0, 0, 0])},
    )
    return cfg, (lambda p: _row(V, rows[p])), expect


def _case_c():
    """Probe on (m=1), trunc=4 < V=8, K=2, W=1 (a greedy chain), D=3, R=4.

    root ()   : tokens {2, 5}; support (2, 5, 0, 1) -> c0 (2, 1/2 DET), c1 (5, 1/2 PROBE)
    beam      : c0, c1 tie -> front [0]
    (2)       : token {7}: no tail mass -> c2 (7, 1/2 DET), c3 (0, 0 FILL)
    beam      : front [2]
    (2, 7)    : tokens {1, 3} -> c4 (1, 1/4 DET), c5 (3, 1/4 PROBE)
    prune     : c0 c1 c2 (1/2), c4 c5 (1/4), c3 (0) -> R = 4 keeps c0 c1 c2 c4, so c4's
                sibling probe c5 is cut. The root's tail: support ranks 1..3 = tokens
                (5, 0, 1) with q~ (1, 0, 0); node c2 keeps no probe child, so no tail.
    """
    V = 8
    rows = {(): [2, 5], (2,): [7], (2, 7): [1, 3]}
    cfg = orc.make_cfg(V=V, trunc=4, K=2, m=1, probe=1, D=3, W=1, R=4)
    expect = dict(
        fronts=[[0], [2], []],
        cand=[-1, 0, 1, 2, 4],
        token=[-1, 2, 5, 7, 1],
        parent=[-1, 0, 0, 1, 3],
        depth=[0, 1, 1, 2, 3],
        kind=[orc.ROOT, orc.DET, orc.PROBE, orc.DET, orc.DET],
        child_off=[0, 2, 3, 3, 4, 4],
        child=[1, 2, 3, 4],
        scores={0: 0.5, 1: 0.5, 2: 0.5, 3: 0.0, 4: 0.25, 5: 0.25},
        tails={0: ([5, 0, 1], [1, 0, 0])},
    )
    return cfg, (lambda p: _row(V, rows[p])), expect


CASES = {"a_ties_W_lt_K_R_cuts_layer": _case_a, "b_probe_R_lt_K": _case_b, "c_chain_trunc_lt_V": _case_c}


def hand_case_ok(name):
    """Whether the oracle reproduces hand-worked tree `name` (False at the first
    difference; a wrong frontier is never expanded further)."""
    cfg, row_of, e = CASES[name]()
    t, fronts = build(cfg, row_of, e["fronts"])
    if t is None:
        return False
    cands = t.cands()
    for c, s in e["scores"].items():
        if cands[c]["score"] != np.float32(s):
            return False
    v = t.view()
    if v["n_nodes"] != len(e["cand"]):
        return False
    for k in ("cand", "token", "parent", "depth", "kind", "child_off", "child"):
        if v[k].tolist() != e[k]:
            return False
    for i in range(v["n_nodes"]):
        n = int(v["tail_n"][i])
        if i in e["tails"]:
            ids, q = e["tails"][i]
            if v["tail_id"][i, :n].tolist() != ids or v["tail_q"][i, :n].tolist() != q:
                return False
        elif n != 0:
            return False
    return True


@pytest.mark.parametrize("name", list(CASES))
def test_hand_worked_tree(name):
    assert hand_case_ok(name)


# ---------------------------------------------------------------------------------
# Invariants over random small configurations

def _random_config(rng):
    V = int(rng.integers(3, 21))
    K = int(rng.integers(1, 6))
    probe = int(rng.integers(0, 2))
    m = int(rng.integers(0, K)) if probe else 0
    return dict(V=V, trunc=int(rng.integers(1, V + 1)), K=K, m=m, probe=probe,
                D=int(rng.integers(1, 5)), W=int(rng.integers(1, 2 * K + 1)),
                R=int(rng.integers(1, 31)), T=float(rng.choice([0.6, 1.0])),
                order=int(rng.integers(0, 2)) if probe else 0)


def _tie_rows(rng, V):
    """Rows of a random context model, cached by path: logits on a coarse grid (many exact
    ties) with some -inf entries."""
    cache = {}

    def row_of(path):
        if path not in cache:
            r = (np.round(rng.normal(size=V) * 1.5) * 0.5).astype(np.float32)
            r[rng.random(V) < 0.15] = NEG
            if not np.isfinite(r).any():
                r[int(rng.integers(0, V))] = 0.0
            cache[path] = r
        return cache[path]
    return row_of


def _key_order(idx, score):
    """idx sorted by (score desc, index asc): numpy's lexsort, not the oracle's sort."""
    idx = np.asarray(idx)
    return idx[np.lexsort((idx, -score[idx].astype(np.float64)))]


def check_invariants(kw, seed):
    """Every invariant for one random configuration; returns a failure message or None."""
    rng = np.random.default_rng(seed)
    cfg = orc.make_cfg(**kw)
    row_of = _tie_rows(rng, kw["V"])
    K, W, D, R = kw["K"], kw["W"], kw["D"], kw["R"]
    t = orc.Tree(cfg, seed, 0, seed)
    front = [-1]
    for layer in range(D):
        if not front:
            break
        cands = t.cands()
        t.expand_layer(layer, np.stack([row_of(_path(cands, c)) for c in front]))
        cands = t.cands()
        base = t.layer_base(layer)
        span = (1 if layer == 0 else W) * K
        live = [c for c in range(base, base + span) if cands[c]["live"]]
        # children of each expanded node: their parent, depth, score bound, distinct tokens
        for pos, f in enumerate(front):
            kids = [c for c in range(base + pos * K, base + pos * K + K) if cands[c]["live"]]
            e = t.row(t.row_base(layer) + pos)
            n_sup = min(kw["trunc"], kw["V"])
            if e.n_sup != n_sup:
                return f"layer {layer} pos {pos}: support of {e.n_sup}"
            # probe last without tail mass leaves the probe's slot empty; otherwise the
            # slots take min(K, support) distinct ranks
            want_n = min(K, n_sup)
            if kw["probe"] and kw["order"] == orc.PROBE_LAST:
                want_n = min(K - 1, n_sup) + (1 if e.probe_rank >= 0 else 0)
            if len(kids) != want_n:
                return f"layer {layer} pos {pos}: {len(kids)} children, want {want_n}"
            if kids != list(range(base + pos * K, base + pos * K + len(kids))):
                return f"layer {layer} pos {pos}: slots not filled in order"
            toks = [int(cands[c]["token"]) for c in kids]
            if len(set(toks)) != len(toks):
                return f"layer {layer} pos {pos}: repeated sibling token"
            ps = np.float32(1.0) if f < 0 else cands[f]["score"]
            pd = 0 if f < 0 else int(cands[f]["depth"])
            for c in kids:
                if cands[c]["parent"] != f or cands[c]["depth"] != pd + 1 or cands[c]["score"] > ps:
                    return f"layer {layer} cand {c}: parent/depth/score"
        nxt = [int(x) for x in t.frontier()]
        want = _key_order(live, cands["score"])[:min(W, len(live))].tolist() if layer + 1 < D else []
        if nxt != want:
            return f"layer {layer}: frontier {nxt} != {want}"
        front = nxt
    t.finish()
    cands = t.cands()
    allc = [c for c in range(len(cands)) if cands[c]["live"]]
    kept = _key_order(allc, cands["score"])[:R].tolist()
    v = t.view()
    n = v["n_nodes"]
    if n != 1 + len(kept) or v["cand"][1:].tolist() != kept:
        return f"emitted {v['cand'][1:].tolist()} != {kept}"
    for i in range(1, n):
        c = int(v["cand"][i])
        p = int(v["parent"][i])
        if not (0 <= p < i) or int(v["cand"][p]) != int(cands[c]["parent"]):
            return f"node {i}: parent {p} not a kept earlier node"
        if v["depth"][i] != v["depth"][p] + 1 or v["token"][i] != cands[c]["token"]:
            return f"node {i}: depth/token"
        if v["kind"][i] != cands[c]["kind"]:
            return f"node {i}: kind"
        if p > 0 and cands[c]["score"] > cands[int(v["cand"][p])]["score"]:
            return f"node {i}: child score above parent"
    # child lists: the kept children of each node in slot order
    for i in range(n):
        kids = v["child"][v["child_off"][i]:v["child_off"][i + 1]].tolist()
        want = sorted([j for j in range(1, n) if v["parent"][j] == i],
                      key=lambda j: int(cands[int(v["cand"][j])]["slot"]))
        if kids != want:
            return f"node {i}: child list {kids} != {want}"
        if len({int(v["token"][j]) for j in kids}) != len(kids):
            return f"node {i}: kept siblings share a token"
        has_probe = any(v["kind"][j] == orc.PROBE for j in kids)
        nt = int(v["tail_n"][i])
        if has_probe != (nt > 0):
            return f"node {i}: tail present {nt > 0}, probe kept {has_probe}"
        if nt:
            probe = [j for j in kids if v["kind"][j] == orc.PROBE][0]
            e = t.row(int(cands[int(v["cand"][probe])]["row"]))
            t0 = min(K - 1, e.n_sup) if kw["order"] == orc.PROBE_LAST else kw["m"]
            if v["tail_id"][i, :nt].tolist() != list(e.sup_id[t0:e.n_sup]):
                return f"node {i}: tail tokens"
            if abs(float(np.sum(v["tail_q"][i, :nt])) - 1.0) > 1e-12:
                return f"node {i}: tail q~ does not sum to 1"
            if int(v["token"][probe]) not in v["tail_id"][i, :nt].tolist():
                return f"node {i}: probe token outside its tail"
    return None


N_RANDOM = 10_000


def test_invariants_on_random_configs():
    rng = np.random.default_rng(20260)
    fails = []
    for k in range(N_RANDOM):
        kw = _random_config(rng)
        msg = check_invariants(kw, 1000 + k)
        if msg:
            fails.append((kw, msg))
    assert not fails, fails[:5]


def invariants_ok(n=300):
    rng = np.random.default_rng(99)
    for k in range(n):
        if check_invariants(_random_config(rng), 5000 + k):
            return False
    return True
