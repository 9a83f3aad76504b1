"""Drives the CPU oracle with synthetic rows (test infrastructure only).

Inputs for the oracle always come from the generator (synth) and the oracle's
own frontier; nothing here reads a result of the HIP path. `t_oracle` records the
seconds spent inside oracle calls (build layers, finish, verification), excluding
row generation, for the benchmark's CPU baseline.
"""
import time

import numpy as np

import synth
from oracle import oracle as orc


def oracle_cfg(w, **kw):
    c = dict(V=w.V, trunc=w.trunc, K=w.K, m=w.m, probe=w.probe, D=w.D, W=w.W, R=w.R, mode=w.mode,
             budget=w.budget, T=w.T, eps_m0=w.eps_m0, alpha=w.alpha, lam=w.lam, gamma=w.gamma,
             delta=w.delta, rho=w.rho, order=w.order)
    c.update(kw)
    return orc.make_cfg(**c)


class OracleStep:
    """One tree b at one step: built by the oracle from synthetic draft rows,
    with the target rows of its emitted nodes, and its verification."""

    def __init__(self, w, seed, b, step, root_key=None, cfg=None, verify=True):
        self.w = w
        self.cfg = cfg if cfg is not None else oracle_cfg(w)
        self.seed, self.b, self.step = seed, b, step
        self.t_oracle = 0.0
        p = w.params()
        tabs = w.tables()
        self.root_key = root_key if root_key is not None else synth.root_key(w.gen_seed, b)
        t = orc.Tree(self.cfg, seed, b, step)
        keys = {-1: self.root_key}
        front = np.array([-1], np.int32)
        self.layer_rows = []      # per layer: [n_par, V] draft rows as generated (bf16 bits or f32)
        self.layer_keys = []
        self.layer_front = []
        for layer in range(w.D):
            if front.size == 0:
                break
            ks = np.array([keys[int(c)] for c in front], np.uint64)
            rows = synth.rows_host(p, tabs, ks, np.full(ks.size, b, np.int32), synth.DRAFT)
            self.layer_rows.append(rows)
            self.layer_keys.append(ks)
            self.layer_front.append(front.copy())
            rows_f = synth.to_f32(rows)
            t0 = time.perf_counter()
            t.expand_layer(layer, rows_f)
            self.t_oracle += time.perf_counter() - t0
            front = t.frontier()
            cands = t.cands()
            for c in front:
                keys[int(c)] = synth.node_key(keys[int(cands[c]["parent"])], int(cands[c]["token"]))
        t0 = time.perf_counter()
        t.finish()
        self.t_oracle += time.perf_counter() - t0
        self.tree = t
        self.cands = t.cands()
        self.view = t.view()
        self.flags = t.flags()
        self.build_exempt = t.n_exempt()
        # keys of every emitted node (parents precede children)
        nk = np.zeros(self.view["n_nodes"], np.uint64)
        nk[0] = self.root_key
        for i in range(1, self.view["n_nodes"]):
            nk[i] = synth.node_key(int(nk[self.view["parent"][i]]), int(self.view["token"][i]))
        self.node_keys = nk
        self.target_rows = synth.rows_host(p, tabs, nk, np.full(nk.size, b, np.int32), synth.TARGET)
        if verify:
            target_f = synth.to_f32(self.target_rows)
            t0 = time.perf_counter()
            (self.out_tokens, self.out_nodes, self.per_node,
             self.verify_exempt) = orc.verify(self.cfg, self.view, target_f, seed, b, step)
            self.t_oracle += time.perf_counter() - t0

    @property
    def exempt(self):
        return self.build_exempt + getattr(self, "verify_exempt", 0)

    def replay(self):
        """The oracle alone on this step's stored inputs (the draft rows of every layer in
        frontier order, the target rows of the emitted nodes): every build layer, the
        finish and the verification, as in __init__. Returns the emitted tokens."""
        t = orc.Tree(self.cfg, self.seed, self.b, self.step)
        for layer, rows in enumerate(self.layer_rows):
            t.expand_layer(layer, synth.to_f32(rows))
        t.finish()
        view = t.view()
        toks, _, _, _ = orc.verify(self.cfg, view, synth.to_f32(self.target_rows), self.seed, self.b,
                                   self.step)
        return toks
