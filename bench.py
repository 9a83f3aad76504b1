#!/usr/bin/env python3
"""Benchmark of one speculative step on one MI355X: draft-tree construction over
all D layers (support truncation, dual-identity expansion, beam, global top-R
prune) followed by probe-first verification, on seeded synthetic logits already
resident in HBM.

Prints ONE JSON line. `value` is verified draft trees per second for the whole
step; the roofline object is the verification call (one launch: every node's target
row streamed, each node decided, the walk fused into the last block of each tree),
whose algorithmic bytes are sum_b n_nodes[b] * V * 2. The input sets are consecutive
decode steps: step s builds from contexts extended by step s-1's emitted tokens and
draws with step counter s. The CPU baseline times the oracle (oracle/) in this
process on a bounded sample of the same workload, on every host core.
"""
import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD published peak


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--T", type=float, default=1.0)
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--cpu-trees", type=int, default=0,
                    help="trees in the oracle's timed sample (0: four per host core)")
    ap.add_argument("--sets", type=int, default=0,
                    help="decode steps made as input sets; the timed steps rotate over them (0: "
                         "the workload's decode length, as many as half the free HBM holds)")
    ap.add_argument("--t06-sets", type=int, default=8,
                    help="decode steps of the T=0.6 measurement (0: skip it)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replayed steps")
    ap.add_argument("--streams", type=int, default=0,
                    help="calls per step, each on its own stream and B/streams trees with tree_base "
                         "at its first tree (0: the workload's default)")
    ap.add_argument("--verify-only", action="store_true",
                    help="time only the verification call (for profiling it alone)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-MiB buffer 3 times (calibrates hardware byte counters)")
    ap.add_argument("--ablation", type=int, default=0, metavar="SETS",
                    help="only the depth-1 verification comparison (point-mass top-K, probe last "
                         "= RRSw, probe first = RheoVerification) over SETS input sets")
    ap.add_argument("--sweep", type=int, default=0, metavar="SETS",
                    help="only the support-size sweep (trunc 128/256/512/1024 and the dense "
                         "baseline) over SETS input sets")
    return ap.parse_args()


HERE = os.path.dirname(os.path.abspath(__file__))
# sources the verification kernels are compiled from; counters taken on other sources
# no longer describe the kernel
VERIFY_SOURCES = ["verify_row_top_amd/csrc/k_verify.hip", "verify_row_top_amd/csrc/vrt_dev.hpp"]
PMC_SUMMARY = "profiles/k_vnode_headline_pmc.md"


def sources_sha():
    import hashlib
    h = hashlib.sha256()
    for p in VERIFY_SOURCES:
        with open(os.path.join(HERE, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per verification call from the committed counter summary, or None when
    it is missing or was taken on other kernel sources."""
    import re
    try:
        with open(os.path.join(HERE, PMC_SUMMARY)) as f:
            text = f.read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("sources_sha") != sources_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_probe(mib):
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "copies": 3, "sources_sha": sources_sha()}), flush=True)


def cpu_baseline(w, seed, n_trees):
    """The oracle as it stands, in this process on every host core: the inputs of n_trees
    trees of the workload are made first (untimed; the generator along the oracle's own
    frontier), then the oracle builds and verifies them, one tree per task on a thread pool
    (its C calls release the interpreter lock), timed by the wall clock."""
    import concurrent.futures as cf

    import torch  # noqa: F401  (first: the helper libraries then share torch's HIP runtime)

    import synth
    from oracle import oracle as orc
    from oracle.drive import OracleStep
    synth.lib()  # loaded once, in this thread, before the pool starts
    orc.lib()
    cores = len(os.sched_getaffinity(0))
    n_trees = n_trees or min(64, 4 * cores)
    with cf.ThreadPoolExecutor(max_workers=cores) as ex:
        steps = list(ex.map(lambda b: OracleStep(w, seed, b, 0, verify=False), range(n_trees)))
    t0 = time.perf_counter()
    steps[0].replay()
    steps[1 % n_trees].replay()
    single = 2 / (time.perf_counter() - t0)
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=cores) as ex:
        list(ex.map(lambda s: s.replay(), steps))
    wall = time.perf_counter() - t0
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": n_trees / wall, "unit": "trees/s", "cores": cores, "kind": "oracle", "cpu": model,
            "sample": f"{n_trees} trees (b=0..{n_trees - 1}, seed {seed}, step 0) of the same workload: "
                      f"every build layer, the finish and the verification on rows made beforehand, one "
                      f"tree per task on {cores} threads of this process, wall time",
            "single_thread_value": single}


def read_ceiling(torch, dev, vrt, mib=1024, reps=10):
    """GB/s of the library's streaming-read probe over a buffer larger than the caches."""
    buf = torch.randint(0, 1 << 30, ((mib << 20) // 4,), dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    vrt.read_probe(buf, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        vrt.read_probe(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del buf
    return (mib << 20) / (ms * 1e-3) / 1e9


def make_inputs(w, cfg, dev, gen_seed, seed, step, tree, ws, stats, views, target=True, rk=None):
    """One input set: the generator plays the draft model along the GPU's own frontier,
    layer by layer (building the tree as it goes), then the target model on the emitted
    tree. rk: the trees' context keys (default: the generator's root keys). Returns
    (draft [B, rows, ld], target [B, N, ld] or None, n_nodes [B] on the host, expanded
    rows per layer)."""
    import torch

    import synth
    from verify_row_top_amd import vrt
    L = vrt.tree_layout_of(cfg)
    B, D, K, N, FP = w.B, w.D, w.K, L.N, L.FP
    esz = 2 if w.dtype == synth.BF16 else 4
    ld = (w.V + 16 // esz - 1) // (16 // esz) * (16 // esz)
    tdt = torch.int16 if w.dtype == synth.BF16 else torch.float32
    n_draft = 1 + (D - 1) * FP
    stream = torch.cuda.current_stream().cuda_stream
    ws_ = w.replace(gen_seed=gen_seed)
    p = ws_.params()
    zipf = torch.from_numpy(ws_.tables()).to(dev)
    if rk is None:
        rk = [synth.root_key(gen_seed, b) for b in range(B)]
    root_keys = torch.tensor([k - (1 << 64) if k >= (1 << 63) else k for k in rk],
                             dtype=torch.int64, device=dev)
    tree_of = torch.arange(B, dtype=torch.int32, device=dev)
    draft = torch.empty((B, n_draft, ld), dtype=tdt, device=dev)
    tmp = torch.empty((B, FP, ld), dtype=tdt, device=dev)
    keys_prev = root_keys.view(B, 1)
    synth.rows_dev(p, zipf, keys_prev.reshape(-1), tree_of, tmp[:, 0], synth.DRAFT, stream)
    draft[:, 0].copy_(tmp[:, 0])
    vrt.build_tree(cfg, 0, draft, ld, n_draft * ld, seed, step, tree, ws, stats)
    expanded = [torch.ones(B, dtype=torch.int32)]
    for layer in range(1, D):
        base = 0 if layer == 1 else K + (layer - 2) * FP * K  # the previous layer's candidates
        keys = torch.zeros((B, FP), dtype=torch.int64, device=dev)
        synth.frontier_keys_dev(B, K, base, keys_prev, views["front"], views["n_front"],
                                views["cand_token"], keys, stream)
        expanded.append(views["n_front"].cpu().clone())
        synth.rows_dev(p, zipf, keys.reshape(-1), tree_of.repeat_interleave(FP),
                       tmp.view(B * FP, ld), synth.DRAFT, stream)
        r0 = 1 + (layer - 1) * FP
        draft[:, r0:r0 + FP].copy_(tmp)
        vrt.build_tree(cfg, layer, draft[:, r0:], ld, n_draft * ld, seed, step, tree, ws, stats)
        keys_prev = keys
    vrt.build_tree(cfg, vrt.FINISH, None, 0, 0, seed, step, tree, ws, stats)
    tgt = None
    if target:
        node_keys = torch.zeros((B, N), dtype=torch.int64, device=dev)
        synth.tree_keys_dev(B, N, root_keys, views["n_nodes"], views["node_token"],
                            views["node_parent"], node_keys, stream)
        tgt = torch.empty((B, N, ld), dtype=tdt, device=dev)
        synth.rows_dev(p, zipf, node_keys.reshape(-1), tree_of.repeat_interleave(N),
                       tgt.view(B * N, ld), synth.TARGET, stream)
    torch.cuda.synchronize()
    return draft, tgt, views["n_nodes"].cpu().clone(), expanded


def sweep(args):
    """Support-size sweep (RheoSampling's support-size ablation) on the workload: for each
    support size and the dense baseline (support = the whole vocabulary), the draft-side
    time of one step (every build layer and the finish, HIP events on the launch stream),
    the verification time, the mean coverage of the expanded rows' supports, and the mean
    tokens per verified tree. Dense trees are verified by vrt_verify_dense, which
    regenerates the probe tails from the draft rows."""
    import torch

    import synth
    from synth import workloads
    from verify_row_top_amd import vrt
    dev = torch.device("cuda:0")
    w0 = workloads.get(args.workload, T=args.T)
    B, V, D = w0.B, w0.V, w0.D
    esz = 2 if w0.dtype == synth.BF16 else 4
    ld = (V + 16 // esz - 1) // (16 // esz) * (16 // esz)
    reps = max(1, args.steps)
    out = []
    for trunc in (128, 256, 512, 1024, vrt.DENSE):
        w = w0.replace(trunc=trunc)
        cfg = vrt.make_config(B=B, V=V, dtype=w.dtype, trunc=trunc, K=w.K, m=w.m, probe=w.probe, D=D,
                              W=w.W, R=w.R, mode=w.mode, budget=w.budget, T=w.T, eps_m0=w.eps_m0,
                              order=w.order)
        L = vrt.tree_layout_of(cfg)
        N, FP = L.N, L.FP
        n_draft = 1 + (D - 1) * FP
        tree = torch.zeros(vrt.tree_bytes(cfg), dtype=torch.uint8, device=dev)
        ws = torch.zeros(vrt.workspace_bytes(cfg), dtype=torch.uint8, device=dev)
        views = vrt.tree_views(cfg, tree)
        stats = torch.zeros((B, 8), dtype=torch.int32, device=dev)
        out_tokens = torch.zeros((B, D + 1), dtype=torch.int32, device=dev)
        out_nodes = torch.zeros((B, D), dtype=torch.int32, device=dev)
        out_len = torch.zeros(B, dtype=torch.int32, device=dev)
        cov = torch.zeros((B, n_draft), dtype=torch.float64, device=dev)
        dense = trunc == vrt.DENSE and w.probe
        times, vtimes, covs, lens = [], [], [], []
        for s in range(args.sweep):
            draft, target, _, expanded = make_inputs(w, cfg, dev, w.gen_seed + 7919 * s, args.seed, s,
                                                     tree, ws, stats, views)
            layers = [draft[:, 0 if l == 0 else 1 + (l - 1) * FP:] for l in range(D)]

            def verify():
                if dense:
                    vrt.verify_dense(cfg, target, ld, N * ld, layers, ld, n_draft * ld, tree, args.seed, s, ws,
                                     out_tokens, out_nodes, out_len, stats)
                else:
                    vrt.verify_tree(cfg, target, ld, N * ld, tree, args.seed, s, ws, out_tokens, out_nodes,
                                    out_len, stats)
            # coverage of the expanded rows (layer 0: the root; layer l: the first n_front rows)
            vrt.support_coverage(cfg, draft, ld, n_draft * ld, n_draft, cov)
            c = cov.cpu().numpy()
            for layer in range(D):
                r0 = 0 if layer == 0 else 1 + (layer - 1) * FP
                for b in range(B):
                    covs.extend(c[b, r0:r0 + int(expanded[layer][b])].tolist())
            verify()
            lens.append(out_len.float().mean().item())
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps + 2)]
            for k in range(reps + 2):
                evs[k][0].record()
                for layer in range(D):
                    vrt.build_tree(cfg, layer, layers[layer], ld, n_draft * ld, args.seed, s, tree, ws, stats)
                vrt.build_tree(cfg, vrt.FINISH, None, 0, 0, args.seed, s, tree, ws, stats)
                evs[k][1].record()
                verify()
                evs[k][2].record()
            torch.cuda.synchronize()
            times.append(sum(e[0].elapsed_time(e[1]) for e in evs[2:]) / reps)
            vtimes.append(sum(e[1].elapsed_time(e[2]) for e in evs[2:]) / reps)
            del draft, target, layers
        rec = {"trunc": "dense" if trunc == vrt.DENSE else trunc,
               "build_ms_per_step": sum(times) / len(times),
               "verify_ms_per_step": sum(vtimes) / len(vtimes),
               "coverage_mean": float(sum(covs) / len(covs)),
               "tokens_per_tree": (sum(lens) / len(lens)) if lens else None,
               "status_bits": int((stats.cpu()[:, 0] != 0).sum())}
        print(json.dumps(rec), flush=True)
        out.append(rec)
    print(json.dumps({"support_sweep": out, "workload": f"{w0.name}: B={B}, V={V}, D={D}, K={w0.K}, "
                      f"m={w0.m}, T={w0.T}", "sets": args.sweep, "reps_per_set": reps}), flush=True)


def ablation(args):
    """Depth-1 controlled comparison of the verification orders on the workload's rows: the
    share of trees whose first emitted token comes from the tree, for the point-mass top-K
    tree (probe off), RheoSampling's tree verified probe last (RRSw) and probe first."""
    import torch

    import synth
    from synth import workloads
    from verify_row_top_amd import vrt
    dev = torch.device("cuda:0")
    base = workloads.get(args.workload, T=args.T)
    w = base.replace(D=1, W=base.K, R=base.K)
    B, V, K = w.B, w.V, w.K
    esz = 2 if w.dtype == synth.BF16 else 4
    ld = (V + 16 // esz - 1) // (16 // esz) * (16 // esz)
    tdt = torch.int16 if w.dtype == synth.BF16 else torch.float32
    stream = torch.cuda.current_stream().cuda_stream
    rates = {}
    for name, kw in (("topk_vanilla", dict(probe=0)), ("rheo_probe_last_rrsw", dict(order=1)),
                     ("rheo_probe_first_ot", dict(order=0))):
        wv = w.replace(**kw)
        cfg = vrt.make_config(B=B, V=V, dtype=wv.dtype, trunc=wv.trunc, K=K, m=wv.m, probe=wv.probe,
                              D=1, W=K, R=K, T=wv.T, eps_m0=wv.eps_m0, order=wv.order)
        N = vrt.tree_layout_of(cfg).N
        tree = torch.zeros(vrt.tree_bytes(cfg), dtype=torch.uint8, device=dev)
        ws = torch.zeros(vrt.workspace_bytes(cfg), dtype=torch.uint8, device=dev)
        views = vrt.tree_views(cfg, tree)
        stats = torch.zeros((B, 8), dtype=torch.int32, device=dev)
        out_tokens = torch.zeros((B, 2), dtype=torch.int32, device=dev)
        out_nodes = torch.zeros((B, 1), dtype=torch.int32, device=dev)
        out_len = torch.zeros(B, dtype=torch.int32, device=dev)
        hits = total = 0
        for s in range(args.ablation):
            ws_ = wv.replace(gen_seed=w.gen_seed + 104729 * s)
            p = ws_.params()
            zipf = torch.from_numpy(ws_.tables()).to(dev)
            rk = [synth.root_key(ws_.gen_seed, b) for b in range(B)]
            root_keys = torch.tensor([k - (1 << 64) if k >= (1 << 63) else k for k in rk],
                                     dtype=torch.int64, device=dev)
            tree_of = torch.arange(B, dtype=torch.int32, device=dev)
            draft = torch.empty((B, 1, ld), dtype=tdt, device=dev)
            synth.rows_dev(p, zipf, root_keys, tree_of, draft[:, 0], synth.DRAFT, stream)
            vrt.build_tree(cfg, 0, draft, ld, ld, args.seed, s, tree, ws, stats)
            vrt.build_tree(cfg, vrt.FINISH, None, 0, 0, args.seed, s, tree, ws, stats)
            node_keys = torch.zeros((B, N), dtype=torch.int64, device=dev)
            synth.tree_keys_dev(B, N, root_keys, views["n_nodes"], views["node_token"],
                                views["node_parent"], node_keys, stream)
            target = torch.empty((B, N, ld), dtype=tdt, device=dev)
            synth.rows_dev(p, zipf, node_keys.reshape(-1), tree_of.repeat_interleave(N),
                           target.view(B * N, ld), synth.TARGET, stream)
            vrt.verify_tree(cfg, target, ld, N * ld, tree, args.seed, s, ws, out_tokens, out_nodes,
                            out_len, stats)
            hits += int((out_len >= 2).sum().item())
            total += B
        rates[name] = hits / total
    print(json.dumps({"ablation_depth1": rates, "workload": f"{w.name} rows, D=1, K={K}, m={w.m}, "
                      f"T={w.T}", "trees": total}), flush=True)


def decode_inputs(w, cfg, dev, n_sets, seed, tree, ws, stats, views, out):
    """n_sets consecutive decode steps of the workload as input sets: set s is made along
    the GPU's own frontier from contexts extended by every token set s-1 emitted, with
    step counter s, then verified once (untimed) to learn those tokens. Returns a list of
    dicts (draft, target, n_nodes, step, near-threshold draws of the step, tokens)."""
    import torch

    import synth
    from verify_row_top_amd import vrt
    out_tokens, out_nodes, out_len = out
    N = vrt.tree_layout_of(cfg).N
    rk = [synth.root_key(w.gen_seed, b) for b in range(w.B)]
    sets = []
    for s in range(n_sets):
        draft, target, n_nodes, _ = make_inputs(w, cfg, dev, w.gen_seed, seed, s, tree, ws, stats, views,
                                                rk=rk)
        ld = target.shape[-1]
        stats.zero_()
        vrt.verify_tree(cfg, target, ld, N * ld, tree, seed, s, ws, out_tokens, out_nodes, out_len, stats)
        torch.cuda.synchronize()
        toks, lens = out_tokens.cpu().numpy(), out_len.cpu().numpy()
        st = stats.cpu().numpy()
        emitted = [toks[b, :lens[b]].tolist() for b in range(w.B)]
        sets.append({"draft": draft, "target": target, "n_nodes": n_nodes, "step": s,
                     "near": int(st[:, 3].sum()), "bad": int((st[:, 0] != 0).sum()),
                     "tokens": float(lens.sum())})
        rk = synth.decode_keys(rk, emitted)
    print(f"bench: {n_sets} decode steps of {w.name} (T={w.T}) made", file=sys.stderr, flush=True)
    return sets


def call_sizes(B, S):
    """Trees per call when a batch of B trees is issued as S calls, and each call's first
    tree (its tree_base): the first B % S calls take one tree more."""
    sizes = [B // S + (1 if p < B % S else 0) for p in range(S)]
    return sizes, [sum(sizes[:p]) for p in range(S)]


def default_streams(w):
    """Calls per step: two for beam-and-prune batches of at least 16 trees, one otherwise.
    Measured on one box: headline 0.296 against 0.348 ms per step, fp32 headline 0.491
    against 0.583; at B = 8 two calls take 0.212 against 0.180 ms (rows of 64 KB leave
    little stream to overlap, and the launches double), and SMART 0.395 against 0.193 ms
    (its short kernels wait on the host's launches, which a second call multiplies)."""
    from synth import workloads
    return 2 if w.mode != workloads.SMART and w.B >= 16 and w.B % 2 == 0 else 1


def measure(w, args, n_sets, lazy=True):
    """Build + verify steps of workload w over n_sets decode steps: warm-up, then timed
    steps rotating over the sets. Returns the measurements as a dict."""
    import torch

    import synth
    from verify_row_top_amd import vrt
    dev = torch.device("cuda:0")
    cfg = vrt.make_config(B=w.B, V=w.V, dtype=w.dtype, trunc=w.trunc, K=w.K, m=w.m, probe=w.probe,
                          D=w.D, W=w.W, R=w.R, mode=w.mode, budget=w.budget, T=w.T, eps_m0=w.eps_m0,
                          alpha=w.alpha, lam=w.lam, gamma=w.gamma, delta=w.delta, rho=w.rho,
                          order=w.order)
    L = vrt.tree_layout_of(cfg)
    B, V, D, N, FP = w.B, w.V, w.D, L.N, L.FP
    esz = 2 if w.dtype == synth.BF16 else 4
    per = 16 // esz
    ld = (V + per - 1) // per * per
    n_draft = 1 + (D - 1) * FP
    tree = torch.zeros(vrt.tree_bytes(cfg), dtype=torch.uint8, device=dev)
    ws = torch.zeros(vrt.workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    views = vrt.tree_views(cfg, tree)
    stats = torch.zeros((B, 8), dtype=torch.int32, device=dev)
    out_tokens = torch.zeros((B, D + 1), dtype=torch.int32, device=dev)
    out_nodes = torch.zeros((B, D), dtype=torch.int32, device=dev)
    out_len = torch.zeros(B, dtype=torch.int32, device=dev)
    seed = args.seed
    if n_sets <= 0:  # the whole decode, if half the free memory holds its rows
        per_set = B * (n_draft + N) * ld * esz
        n_sets = max(3, min(w.steps, int(0.5 * torch.cuda.mem_get_info()[0] // per_set)))
    sets = decode_inputs(w, cfg, dev, n_sets, seed, tree, ws, stats, views, (out_tokens, out_nodes, out_len))

    def layer_rows(draft, layer):
        r0 = 0 if layer == 0 else 1 + (layer - 1) * FP
        return draft[:, r0:]

    def build(st):
        for layer in range(D):
            vrt.build_tree(cfg, layer, layer_rows(st["draft"], layer), ld, n_draft * ld, seed, st["step"],
                           tree, ws, stats)
        vrt.build_tree(cfg, vrt.FINISH, None, 0, 0, seed, st["step"], tree, ws, stats)

    def verify(st):
        vrt.verify_tree(cfg, st["target"], ld, N * ld, tree, seed, st["step"], ws, out_tokens, out_nodes,
                        out_len, stats)

    # ---- timed: whole steps (every build layer, finish, the verification call)
    def one_step(k, evs=None):
        st = sets[k % len(sets)]
        if evs:
            evs[0].record()
        if not args.verify_only:
            build(st)
        if evs:
            evs[1].record()
        verify(st)
        if evs:
            evs[2].record()

    if args.verify_only:  # the tree of set 0 stays in place; every step verifies set 0's rows
        sets = sets[:1]
        build(sets[0])
    for k in range(args.warmup):
        one_step(k)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    k0 = args.warmup  # the timed steps continue the decode after the warm-up steps
    t0 = time.perf_counter()
    for k in range(args.steps):
        one_step(k0 + k, evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    used = [sets[(k0 + k) % len(sets)] for k in range(args.steps)]
    build_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    vt = sorted(e[1].elapsed_time(e[2]) for e in evs)
    verify_ms = sum(vt) / len(vt)
    q = lambda f: vt[min(len(vt) - 1, int(f * len(vt)))]
    ms_per_step = wall * 1e3 / args.steps
    verify_bytes = sum(int(st["n_nodes"].sum()) for st in used) * V * esz / args.steps
    tokens = sum(st["tokens"] for st in used)
    one_call_ms = ms_per_step

    # the step issued as S calls, each on its own stream and B/S trees (tree_base at its
    # first tree): one call's dependent phases (the rows' post-load work, the layer
    # ranking, launch gaps) overlap the other calls' row streams. The calls give the one
    # call's trees and tokens bit for bit; set 0's step is checked.
    S = default_streams(w) if getattr(args, "streams", 0) == 0 else args.streams
    split = None
    if 1 < S <= B and not args.verify_only:
        sizes, starts = call_sizes(B, S)
        pcfg = [vrt.make_config(B=sizes[p], V=w.V, dtype=w.dtype, trunc=w.trunc, K=w.K, m=w.m, probe=w.probe,
                                D=w.D, W=w.W, R=w.R, mode=w.mode, budget=w.budget, T=w.T, eps_m0=w.eps_m0,
                                alpha=w.alpha, lam=w.lam, gamma=w.gamma, delta=w.delta, rho=w.rho,
                                order=w.order, tree_base=starts[p]) for p in range(S)]
        ptree = [torch.zeros(vrt.tree_bytes(c), dtype=torch.uint8, device=dev) for c in pcfg]
        pws = [torch.zeros(vrt.workspace_bytes(c), dtype=torch.uint8, device=dev) for c in pcfg]
        pstreams = [torch.cuda.Stream() for _ in range(S)]  # default priority

        def split_step(st):
            # launches issued layer by layer across the calls (one call after the other
            # measured 0.300-0.304 against 0.297 ms per headline step)
            sls = [slice(starts[p], starts[p] + sizes[p]) for p in range(S)]
            for layer in range(D):
                for p in range(S):
                    vrt.build_tree(pcfg[p], layer, layer_rows(st["draft"], layer)[sls[p]], ld, n_draft * ld, seed,
                                   st["step"], ptree[p], pws[p], stats[sls[p]], stream=pstreams[p])
            for p in range(S):
                sl = sls[p]
                vrt.build_tree(pcfg[p], vrt.FINISH, None, 0, 0, seed, st["step"], ptree[p], pws[p], stats[sl],
                               stream=pstreams[p])
                vrt.verify_tree(pcfg[p], st["target"][sl], ld, N * ld, ptree[p], seed, st["step"], pws[p],
                                out_tokens[sl], out_nodes[sl], out_len[sl], stats[sl], stream=pstreams[p])

        build(sets[0])
        verify(sets[0])
        torch.cuda.synchronize()
        ref = (out_tokens.clone(), out_len.clone())
        out_tokens.fill_(-1)
        out_len.fill_(-1)
        torch.cuda.synchronize()
        split_step(sets[0])
        torch.cuda.synchronize()
        same = bool(torch.equal(ref[0], out_tokens)) and bool(torch.equal(ref[1], out_len))
        for k in range(args.warmup):
            split_step(sets[k % len(sets)])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            split_step(sets[(k0 + k) % len(sets)])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_per_step = wall * 1e3 / args.steps
        split = {"calls": S, "trees_per_call": sizes, "same_tokens_as_one_call": same,
                 "one_call_ms_per_step": one_call_ms, "one_call_trees_per_s": B / (one_call_ms * 1e-3)}
    r = {"cfg": cfg, "tree": tree, "sets": sets, "B": B, "esz": esz, "ld": ld, "streams": split,
         "ms_per_step": ms_per_step, "value": B / (ms_per_step * 1e-3) if not args.verify_only
         else B / (verify_ms * 1e-3),
         "build_ms": build_ms if not args.verify_only else None, "verify_ms": verify_ms,
         "verify_ms_p10_p50_p90": [q(0.1), q(0.5), q(0.9)], "verify_bytes": verify_bytes,
         "verify_gbs": verify_bytes / (verify_ms * 1e-3) / 1e9,
         "near_threshold_draws": sum(st["near"] for st in used),
         "status_bits": sum(st["bad"] for st in used),
         "verified_tokens_per_s": tokens / (wall if not args.verify_only else verify_ms * 1e-3 * args.steps),
         "mean_tokens_per_tree": tokens / (len(used) * B),
         "mean_nodes_per_tree": sum(float(st["n_nodes"].float().mean()) for st in used) / len(used)}
    if w.mode == 0 and not args.verify_only:
        r["build_gbps"] = B * n_draft * V * esz / (build_ms * 1e-3) / 1e9

    # the same whole steps launched from HIP graphs: the step of each of the first (up to
    # 16) sets captured once, with its launches' arguments fixed, then replays rotating over
    # them; the GPU does the eager step's work without the host's per-launch cost. Each
    # set's replay must emit the eager step's tokens.
    if lazy and not args.verify_only and not args.no_graph:
        gsets = sets[:min(len(sets), 16)]
        ref = []
        for st in gsets:
            build(st)
            verify(st)
            torch.cuda.synchronize()
            ref.append((out_tokens.clone(), out_len.clone()))
        graphs = []
        for st in gsets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                build(st)
                verify(st)
            graphs.append(g)
        torch.cuda.synchronize()
        same = True
        for g, (rt, rl) in zip(graphs, ref):
            out_tokens.fill_(-1)
            out_len.fill_(-1)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            same &= bool(torch.equal(rt, out_tokens)) and bool(torch.equal(rl, out_len))
        for k in range(args.warmup):
            graphs[k % len(graphs)].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            graphs[k % len(graphs)].replay()
        torch.cuda.synchronize()
        gwall = time.perf_counter() - t0
        r["graph_step"] = {"ms_per_step": gwall * 1e3 / args.steps, "trees_per_s": B * args.steps / gwall,
                           "sets": len(graphs), "same_tokens_as_eager": same}
        del graphs

    # the verification call on its own, for the roofline: every set's tree built into a blob
    # of its own (untimed), then the sets verified back to back between two HIP events on
    # the launch stream, so the average is the call's own duration (the in-step timing
    # above also holds the dispatch after the build's last kernel)
    if not args.verify_only:
        blobs = []
        for st in sets:
            tb = torch.zeros_like(tree)
            for layer in range(D):
                vrt.build_tree(cfg, layer, layer_rows(st["draft"], layer), ld, n_draft * ld, seed, st["step"],
                               tb, ws, stats)
            vrt.build_tree(cfg, vrt.FINISH, None, 0, 0, seed, st["step"], tb, ws, stats)
            blobs.append(tb)
        for st, tb in zip(sets[:3], blobs[:3]):  # warm-up
            vrt.verify_tree(cfg, st["target"], ld, N * ld, tb, seed, st["step"], ws, out_tokens, out_nodes,
                            out_len, stats)
        torch.cuda.synchronize()
        reps = max(1, -(-args.steps // len(sets)))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            for st, tb in zip(sets, blobs):
                vrt.verify_tree(cfg, st["target"], ld, N * ld, tb, seed, st["step"], ws, out_tokens, out_nodes,
                                out_len, stats)
        e1.record()
        torch.cuda.synchronize()
        calls = reps * len(sets)
        r["call_ms"] = e0.elapsed_time(e1) / calls
        r["call_bytes"] = sum(int(st["n_nodes"].sum()) for st in sets) * V * esz / len(sets)
        r["call_gbs"] = r["call_bytes"] / (r["call_ms"] * 1e-3) / 1e9
        r["calls"] = calls
        del blobs
    if not lazy:
        return r

    # lazy verification (only the rows of the nodes the walk visits), timed on its own:
    # each rep rebuilds a set's tree (untimed), then verifies it lazily between two events
    lz_ms, lz_rows, lz_near, lazy_ok = [], 0, 0, True
    for k in range(min(args.steps, 2 * len(sets)) + 3):
        st = sets[k % len(sets)]
        build(st)
        verify(st)
        ref = out_tokens.clone()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        vrt.verify_lazy(cfg, st["target"], ld, N * ld, tree, seed, st["step"], ws, out_tokens, out_nodes,
                        out_len, stats)
        e1.record()
        torch.cuda.synchronize()
        lazy_ok &= bool(torch.equal(ref, out_tokens))
        if k >= 3:
            lz_ms.append(e0.elapsed_time(e1))
            lz_rows += int(out_len.sum().item())
            lz_near += int(stats[:, 3].sum().item())  # the visited nodes' near-threshold draws
    lazy_ms = sum(lz_ms) / len(lz_ms)
    r["lazy_verify"] = {"ms": lazy_ms, "trees_per_s": B / (lazy_ms * 1e-3),
                        "rows_read_per_tree": lz_rows / (len(lz_ms) * B),
                        "rows_per_tree_full": r["mean_nodes_per_tree"],
                        "step_trees_per_s": (B / ((build_ms + lazy_ms) * 1e-3)) if not args.verify_only
                        else None,
                        "same_tokens_as_full": lazy_ok, "near_threshold_draws": lz_near,
                        "calls": len(lz_ms)}

    # the step after the prune, timed on its own: attention mask + position ids of the
    # target forward over the emitted trees, and the KV entries kept after verification
    W32 = (N + 31) // 32
    mask = torch.empty((B, N, W32), dtype=torch.int32, device=dev)
    pos = torch.empty((B, N), dtype=torch.int32, device=dev)
    keep = torch.empty((B, D + 1), dtype=torch.int32, device=dev)
    keep_n = torch.empty(B, dtype=torch.int32, device=dev)
    aux = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    for _ in range(3):
        vrt.tree_mask(cfg, tree, mask, pos)
        vrt.accepted_kv(cfg, out_nodes, out_len, keep, keep_n)
    aux[0].record()
    for _ in range(20):
        vrt.tree_mask(cfg, tree, mask, pos)
    aux[1].record()
    for _ in range(20):
        vrt.accepted_kv(cfg, out_nodes, out_len, keep, keep_n)
    aux[2].record()
    torch.cuda.synchronize()
    r["tree_mask_us"] = aux[0].elapsed_time(aux[1]) / 20 * 1e3
    r["accepted_kv_us"] = aux[1].elapsed_time(aux[2]) / 20 * 1e3
    return r


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.ablation:
        ablation(args)
        return
    if args.sweep:
        sweep(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported (trees are "
              f"independent: shard the batch, one process per GPU)", file=sys.stderr)
        sys.exit(2)
    from synth import workloads
    w = workloads.get(args.workload, T=args.T)
    cpu = None if args.no_cpu else cpu_baseline(w, args.seed, args.cpu_trees)
    if cpu is not None:
        print(f"bench: oracle baseline {cpu['value']:.2f} trees/s on {cpu['cores']} cores", file=sys.stderr,
              flush=True)

    import torch

    from verify_row_top_amd import vrt
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    r = measure(w, args, args.sets)
    B, V, D = w.B, w.V, w.D
    esz = r["esz"]
    vgbs = r["verify_gbs"]
    result = {
        "metric": "verified draft trees/sec and HBM GB/s (% peak) at B=32, V=128256, R=60",
        "value": r["value"],
        "unit": "trees/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if esz == 2 else "fp32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={B}, V={V} {'bf16' if esz == 2 else 'fp32'} logits, "
                               f"R={w.R}, D={D}, K=W={w.width}, m={w.m}, T={w.T}, trunc={w.trunc}, "
                               f"{len(r['sets'])} consecutive decode steps",
                   "B": B, "V": V, "R": w.R, "D": D, "K": w.K, "m": w.m, "T": w.T,
                   "decode_steps": len(r["sets"]),
                   "calls_per_step": r["streams"]["calls"] if r["streams"] else 1},
        "roofline": {"bound": "hbm", "kernel": "k_vnode<bf16, walk fused> (vrt_verify_tree: the whole "
                     "verification call, one launch)" if esz == 2 else
                     "k_vnode<fp32, walk fused> (vrt_verify_tree: the whole verification call, one launch)",
                     "achieved": r.get("call_gbs", vgbs), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": r.get("call_gbs", vgbs) / HBM_PEAK_GBS,
                     # the counters were taken on the headline workload only
                     "traffic": measured_traffic() if w == workloads.get("headline") else None,
                     "algorithmic_bytes_per_launch": r.get("call_bytes", r["verify_bytes"]),
                     "avg_launch_ms": r.get("call_ms", r["verify_ms"]),
                     "timed": f"{r.get('calls', args.steps)} calls back to back over the {len(r['sets'])} "
                              f"decode steps' trees, between two HIP events on the launch stream"},
        "verify_ms": r["verify_ms"],
        "verify_call_gbs": vgbs,
        "verify_ms_p10_p50_p90": r["verify_ms_p10_p50_p90"],
        "read_ceiling_gbs": read_ceiling(torch, dev, vrt),
        "verify_trees_per_s": B / (r["verify_ms"] * 1e-3),
        "build_ms": r["build_ms"],
        "build_gbps": r.get("build_gbps"),
        "verified_tokens_per_s": r["verified_tokens_per_s"],
        "mean_tokens_per_tree": r["mean_tokens_per_tree"],
        "near_threshold_draws": r["near_threshold_draws"],
        "status_bits": r["status_bits"],
        "streams": r.get("streams"),
        "lazy_verify": r.get("lazy_verify"),
        "graph_step": r.get("graph_step"),
        "tree_mask_us": r.get("tree_mask_us"),
        "accepted_kv_us": r.get("accepted_kv_us"),
    }
    del r
    if args.t06_sets and w.T != 0.6 and not args.verify_only:
        r6 = measure(w.replace(T=0.6), args, args.t06_sets, lazy=False)
        result["T06"] = {k: r6[k] for k in ("value", "ms_per_step", "build_ms", "verify_ms", "verify_gbs",
                                            "near_threshold_draws", "status_bits", "mean_tokens_per_tree")}
        result["T06"]["frac"] = r6["verify_gbs"] / HBM_PEAK_GBS
        result["T06"]["decode_steps"] = len(r6["sets"])
        del r6
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
