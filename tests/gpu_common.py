"""Helpers for the GPU parity tests: move generator rows and oracle trees into
the library's device layout, run the HIP path through the C ABI, read back."""
import numpy as np
import torch

import synth
from verify_row_top_amd import vrt


def lib_config(w, **kw):
    c = dict(B=w.B, V=w.V, dtype=w.dtype, trunc=w.trunc, K=w.K, m=w.m, probe=w.probe, D=w.D, W=w.W,
             R=w.R, mode=w.mode, budget=w.budget, T=w.T, eps_m0=w.eps_m0, alpha=w.alpha, lam=w.lam,
             gamma=w.gamma, delta=w.delta, rho=w.rho, order=w.order)
    c.update(kw)
    return vrt.make_config(**c)


def row_ld(w):
    """Row stride in elements: V rounded up to 16 bytes."""
    per = 8 if w.dtype == synth.BF16 else 4
    return (w.V + per - 1) // per * per


def to_device_rows(rows_list, w, n_rows, dev):
    """rows_list[b] is an [n_b, V] host array (bf16 bits or fp32); returns a
    [B, n_rows, ld] device tensor (int16 bits for bf16), rows past n_b zero."""
    ld = row_ld(w)
    if w.dtype == synth.BF16:
        host = np.zeros((len(rows_list), n_rows, ld), np.uint16)
    else:
        host = np.zeros((len(rows_list), n_rows, ld), np.float32)
    for b, r in enumerate(rows_list):
        if r is None:
            continue
        host[b, :r.shape[0], :w.V] = r
    t = torch.from_numpy(host.view(np.int16) if w.dtype == synth.BF16 else host)
    return t.to(dev), ld


class Lib:
    """Device buffers for one configuration."""

    def __init__(self, cfg, dev):
        self.cfg = cfg
        self.dev = dev
        self.tree = torch.zeros(vrt.tree_bytes(cfg), dtype=torch.uint8, device=dev)
        # the workspace needs no initialisation: start from garbage
        self.ws = torch.full((vrt.workspace_bytes(cfg),), 0xA5, dtype=torch.uint8, device=dev)
        self.views = vrt.tree_views(cfg, self.tree)
        L = vrt.tree_layout_of(cfg)
        self.N = L.N
        self.TC = L.TC
        self.FP = L.FP
        self.stats = torch.zeros((cfg.B, 8), dtype=torch.int32, device=dev)
        self.out_tokens = torch.zeros((cfg.B, cfg.D + 1), dtype=torch.int32, device=dev)
        self.out_nodes = torch.zeros((cfg.B, cfg.D), dtype=torch.int32, device=dev)
        self.out_len = torch.zeros(cfg.B, dtype=torch.int32, device=dev)
        self.node_out = torch.zeros((cfg.B, self.N, 4), dtype=torch.int32, device=dev)

    def write_view(self, b, view):
        """Write an oracle verification view into tree b's emitted-tree arrays."""
        n = view["n_nodes"]
        v = self.views
        v["n_nodes"][b] = n
        for k in ("token", "parent", "depth", "kind"):
            v["node_" + k][b, :n] = torch.from_numpy(view[k].astype(np.int32))
        v["node_cand"][b, :n] = torch.from_numpy(view["cand"].astype(np.int32))
        v["child_off"][b, :n + 1] = torch.from_numpy(view["child_off"].astype(np.int32))
        nch = view["child"].size
        if nch:
            v["child"][b, :nch] = torch.from_numpy(view["child"].astype(np.int32))
        v["tail_n"][b, :n] = torch.from_numpy(view["tail_n"].astype(np.int32))
        tc = view["tail_id"].shape[1]
        v["tail_id"][b, :n, :tc] = torch.from_numpy(view["tail_id"].astype(np.int32))
        v["tail_q"][b, :n, :tc] = torch.from_numpy(view["tail_q"].astype(np.float32))

    def verify(self, target, ld, seed, step, zero_stats=True):
        if zero_stats:
            self.stats.zero_()
        vrt.verify_tree(self.cfg, target, ld, target.stride(0), self.tree, seed, step, self.ws,
                        self.out_tokens, self.out_nodes, self.out_len, self.stats, self.node_out)
        torch.cuda.synchronize()

    def verify_dense(self, target, ld, seed, step, zero_stats=True):
        """Dense trees: the draft rows of every layer are self.layer_rows."""
        if zero_stats:
            self.stats.zero_()
        rows = self.layer_rows
        vrt.verify_dense(self.cfg, target, ld, target.stride(0), rows, rows[0].shape[-1], rows[0].stride(0),
                         self.tree, seed, step, self.ws, self.out_tokens, self.out_nodes, self.out_len,
                         self.stats, self.node_out)
        torch.cuda.synchronize()

    def verify_lazy(self, target, ld, seed, step, zero_stats=True):
        if zero_stats:
            self.stats.zero_()
        vrt.verify_lazy(self.cfg, target, ld, target.stride(0), self.tree, seed, step, self.ws,
                        self.out_tokens, self.out_nodes, self.out_len, self.stats, self.node_out)
        torch.cuda.synchronize()

    def build_layer(self, layer, rows, ld, seed, step):
        vrt.build_tree(self.cfg, layer, rows, ld, rows.stride(0), seed, step, self.tree, self.ws,
                       self.stats)

    def finish(self, seed=0, step=0):
        vrt.build_tree(self.cfg, vrt.FINISH, None, 0, 0, seed, step, self.tree, self.ws, self.stats)
        torch.cuda.synchronize()

    def host(self, name):
        return self.views[name].cpu().numpy()


def device_step(w, seed, step, dev, verify=True, keep_target=False, root_keys=None):
    """Every tree of workload w built and verified on the GPU, the way the benchmark
    runs it: the device generator plays the draft model along the GPU's own frontier,
    layer by layer, then the target model on the emitted trees (unless verify is
    False). root_keys: the trees' context keys (default: the generator's root keys; a
    decode passes the contexts extended by the tokens emitted so far). Returns the Lib."""
    cfg = lib_config(w)
    L = Lib(cfg, dev)
    B, D, K, N, FP = w.B, w.D, w.K, L.N, L.FP
    ld = row_ld(w)
    tdt = torch.int16 if w.dtype == synth.BF16 else torch.float32
    stream = torch.cuda.current_stream().cuda_stream
    p = w.params()
    zipf = torch.from_numpy(w.tables()).to(dev)
    rk = root_keys if root_keys is not None else [synth.root_key(w.gen_seed, b) for b in range(B)]
    root_keys = torch.tensor([k - (1 << 64) if k >= (1 << 63) else k for k in rk], dtype=torch.int64,
                             device=dev)
    tree_of = torch.arange(B, dtype=torch.int32, device=dev)
    dense = w.trunc == vrt.DENSE and w.probe  # the verification re-reads every layer's rows
    rows = torch.zeros((B, FP, ld), dtype=tdt, device=dev)
    L.layer_rows = [rows]
    keys_prev = root_keys.view(B, 1)
    synth.rows_dev(p, zipf, keys_prev.reshape(-1), tree_of, rows[:, 0], synth.DRAFT, stream)
    L.build_layer(0, rows, ld, seed, step)
    for layer in range(1, D):
        if dense:
            rows = torch.zeros((B, FP, ld), dtype=tdt, device=dev)
            L.layer_rows.append(rows)
        base = 0 if layer == 1 else K + (layer - 2) * FP * K  # the previous layer's candidates
        keys = torch.zeros((B, FP), dtype=torch.int64, device=dev)
        synth.frontier_keys_dev(B, K, base, keys_prev, L.views["front"], L.views["n_front"],
                                L.views["cand_token"], keys, stream)
        synth.rows_dev(p, zipf, keys.reshape(-1), tree_of.repeat_interleave(FP), rows.view(B * FP, ld),
                       synth.DRAFT, stream)
        L.build_layer(layer, rows, ld, seed, step)
        keys_prev = keys
    L.finish(seed, step)
    del rows
    if not verify:
        torch.cuda.synchronize()
        return L
    node_keys = torch.zeros((B, N), dtype=torch.int64, device=dev)
    synth.tree_keys_dev(B, N, root_keys, L.views["n_nodes"], L.views["node_token"],
                        L.views["node_parent"], node_keys, stream)
    target = torch.empty((B, N, ld), dtype=tdt, device=dev)
    synth.rows_dev(p, zipf, node_keys.reshape(-1), tree_of.repeat_interleave(N), target.view(B * N, ld),
                   synth.TARGET, stream)
    if dense:
        L.verify_dense(target, ld, seed, step, zero_stats=False)
    else:
        L.verify(target, ld, seed, step, zero_stats=False)
    if not dense:
        del L.layer_rows
    if keep_target:
        L.target, L.ld = target, ld
    del target
    return L


def oracle_steps(w, seed, step, trees, root_keys=None):
    """OracleStep of each tree b in `trees` (root_keys[b] its context key, if given), on a
    thread pool over this process's cores (the oracle's and generator's C calls release the
    interpreter lock). The libraries load in this thread first."""
    import concurrent.futures as cf
    import os

    from oracle import oracle as orc
    from oracle.drive import OracleStep
    synth.lib()
    orc.lib()
    trees = list(trees)
    rk = (lambda b: None) if root_keys is None else (lambda b: root_keys[b])
    with cf.ThreadPoolExecutor(max_workers=max(1, min(len(trees), len(os.sched_getaffinity(0))))) as ex:
        return list(ex.map(lambda b: OracleStep(w, seed, b, step, root_key=rk(b)), trees))
