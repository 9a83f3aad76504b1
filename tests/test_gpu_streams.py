"""The library keeps no state between calls but the caller's buffers: two batches built
and verified on two streams at once, their launches interleaved, give exactly what the
same calls give one after the other on one stream."""
import pytest
import torch

from synth import workloads
from tests.gpu_common import Lib, lib_config, row_ld, to_device_rows
from oracle.drive import OracleStep

pytestmark = pytest.mark.gpu


def _inputs(w, seed, step, L, dev):
    steps = [OracleStep(w, seed, b, step, verify=False) for b in range(w.B)]
    layers = []
    for layer in range(w.D):
        rows_list = [s.layer_rows[layer] if layer < len(s.layer_rows) else None for s in steps]
        rows, _ = to_device_rows(rows_list, w, L.FP, dev)
        layers.append(rows)
    target, _ = to_device_rows([s.target_rows for s in steps], w, L.N, dev)
    return layers, target


def _run(L, layers, target, ld, seed, step, stream):
    import verify_row_top_amd.vrt as vrt
    with torch.cuda.stream(stream):
        for layer, rows in enumerate(layers):
            vrt.build_tree(L.cfg, layer, rows, ld, rows.stride(0), seed, step, L.tree, L.ws, L.stats, stream=stream)
        vrt.build_tree(L.cfg, vrt.FINISH, None, 0, 0, seed, step, L.tree, L.ws, L.stats, stream=stream)
        vrt.verify_tree(L.cfg, target, ld, target.stride(0), L.tree, seed, step, L.ws, L.out_tokens, L.out_nodes,
                        L.out_len, L.stats, L.node_out, stream=stream)


def test_two_streams_match_one(gpu):
    import verify_row_top_amd.vrt as vrt
    w = workloads.get("headline").replace(B=4, V=20000)
    ld = row_ld(w)
    runs = [(11, 0), (12, 5)]
    libs = [Lib(lib_config(w), gpu) for _ in runs]
    data = [_inputs(w, seed, step, L, gpu) for (seed, step), L in zip(runs, libs)]
    s0 = torch.cuda.current_stream()
    for L, (layers, target), (seed, step) in zip(libs, data, runs):  # one after the other
        _run(L, layers, target, ld, seed, step, s0)
    torch.cuda.synchronize()
    ref = [(L.out_tokens.clone(), L.out_len.clone(), L.node_out.clone(), L.tree.clone()) for L in libs]
    for L in libs:
        L.tree.zero_()
        L.out_tokens.zero_()
        L.node_out.zero_()
        L.stats.zero_()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    torch.cuda.synchronize()
    # interleave the two batches' launches layer by layer
    for layer in range(w.D):
        for L, (layers, target), (seed, step), st in zip(libs, data, runs, streams):
            rows = layers[layer]
            vrt.build_tree(L.cfg, layer, rows, ld, rows.stride(0), seed, step, L.tree, L.ws, L.stats, stream=st)
    for L, (layers, target), (seed, step), st in zip(libs, data, runs, streams):
        vrt.build_tree(L.cfg, vrt.FINISH, None, 0, 0, seed, step, L.tree, L.ws, L.stats, stream=st)
        vrt.verify_tree(L.cfg, target, ld, target.stride(0), L.tree, seed, step, L.ws, L.out_tokens, L.out_nodes,
                        L.out_len, L.stats, L.node_out, stream=st)
    torch.cuda.synchronize()
    for L, (tok, ln, no, tree) in zip(libs, ref):
        assert torch.equal(L.out_tokens, tok)
        assert torch.equal(L.out_len, ln)
        assert torch.equal(L.node_out, no)
        assert torch.equal(L.tree, tree)


TREE_FIELDS = ("n_nodes", "node_token", "node_parent", "node_depth", "node_kind", "node_cand", "child_off",
               "child", "tail_n", "tail_id", "tail_q", "cand_token", "cand_parent", "cand_score", "cand_kind")


@pytest.mark.parametrize("name,w", [
    ("headline_rows_B6", workloads.get("headline").replace(B=6, V=20000)),
    ("smart_B6", workloads.get("smart").replace(B=6, V=12000, D=4, budget=40)),
], ids=lambda x: x if isinstance(x, str) else None)
def test_batch_split_over_streams_matches_one_call(gpu, name, w):
    """A batch issued as two calls of half the trees each, on two streams, with tree_base
    set to each call's first tree, gives the one call's trees, decisions and tokens bit for
    bit; without tree_base the second half draws as the first half's trees would."""
    import verify_row_top_amd.vrt as vrt
    seed, step = 21, 2
    ld = row_ld(w)
    full = Lib(lib_config(w), gpu)
    layers, target = _inputs(w, seed, step, full, gpu)
    print(f"batch split: {name} B={w.B} V={w.V}", flush=True)
    _run(full, layers, target, ld, seed, step, torch.cuda.current_stream())
    torch.cuda.synchronize()
    h = w.B // 2
    halves = [Lib(lib_config(w.replace(B=h), tree_base=base), gpu) for base in (0, h)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    torch.cuda.synchronize()
    for layer in range(w.D):
        for k, (L, st) in enumerate(zip(halves, streams)):
            rows = layers[layer][k * h:(k + 1) * h]
            vrt.build_tree(L.cfg, layer, rows, ld, rows.stride(0), seed, step, L.tree, L.ws, L.stats, stream=st)
    for k, (L, st) in enumerate(zip(halves, streams)):
        tg = target[k * h:(k + 1) * h]
        vrt.build_tree(L.cfg, vrt.FINISH, None, 0, 0, seed, step, L.tree, L.ws, L.stats, stream=st)
        vrt.verify_tree(L.cfg, tg, ld, tg.stride(0), L.tree, seed, step, L.ws, L.out_tokens, L.out_nodes,
                        L.out_len, L.stats, L.node_out, stream=st)
    torch.cuda.synchronize()
    for k, L in enumerate(halves):
        sl = slice(k * h, (k + 1) * h)
        assert torch.equal(L.out_tokens, full.out_tokens[sl])
        assert torch.equal(L.out_len, full.out_len[sl])
        assert torch.equal(L.out_nodes, full.out_nodes[sl])
        assert torch.equal(L.node_out, full.node_out[sl])
        assert torch.equal(L.stats, full.stats[sl])
        for f in TREE_FIELDS:
            assert torch.equal(L.views[f], full.views[f][sl]), f
    # the second half again with tree_base 0: its draws are those of trees 0 .. h-1
    L = Lib(lib_config(w.replace(B=h)), gpu)
    for layer in range(w.D):
        rows = layers[layer][h:]
        vrt.build_tree(L.cfg, layer, rows, ld, rows.stride(0), seed, step, L.tree, L.ws, L.stats)
    vrt.build_tree(L.cfg, vrt.FINISH, None, 0, 0, seed, step, L.tree, L.ws, L.stats)
    tg = target[h:]
    vrt.verify_tree(L.cfg, tg, ld, tg.stride(0), L.tree, seed, step, L.ws, L.out_tokens, L.out_nodes, L.out_len,
                    L.stats, L.node_out)
    torch.cuda.synchronize()
    assert not (torch.equal(L.node_out, full.node_out[h:]) and
                torch.equal(L.views["cand_token"], full.views["cand_token"][h:]))
