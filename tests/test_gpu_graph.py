"""A whole step captured in a HIP graph and replayed: every build layer, the finish and
the one-launch verification, with the kernels' arguments (the split rows' join epoch, the
fused walk's tag, SMART's cost table) fixed at capture. Each replay must give the oracle's
tree and tokens again: the words those launches hand between their blocks (row_sync, the
verification's per-tree counters) are set back to 0 by their last user, so a replay with
the same arguments starts afresh. Eager work runs between replays, and every replay is
checked."""
import numpy as np
import pytest
import torch

import synth
from oracle.drive import OracleStep
from tests.gpu_common import Lib, lib_config, to_device_rows
from tests.test_gpu_build import _small, _smart_small, compare_tree
from verify_row_top_amd import vrt

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,w", [
    ("split_fp32_V70000", _small(dtype=synth.F32, V=70000, R=30, D=4, B=3)),
    ("smart_small", _smart_small(B=3)),
    # 5 trees of 128 frontier slots: 640 slots per layer, more than the compact grid's 512
    # blocks, so the ranking kernel also reads the grid's stored prefix sums
    ("smart_compact_merged", _smart_small(B=5, budget=128, D=4)),
    ("headline_rows", _small(V=128256, R=60, D=4, K=10, B=2)),
    # 270 rows per layer on 256 CUs: the extra rows in quarters, joined on row words that
    # carry the same tag in every replay
    ("rows_beyond_cus", _small(B=27, K=10, W=10, V=57000, R=30, D=3)),
], ids=lambda x: x if isinstance(x, str) else None)
def test_captured_step_replays_match_oracle(gpu, name, w):
    seed, step = 9, 4
    steps = [OracleStep(w, seed, b, step) for b in range(w.B)]
    L = Lib(lib_config(w), gpu)
    layers = []
    for layer in range(w.D):
        rows_list = [s.layer_rows[layer] if layer < len(s.layer_rows) else None for s in steps]
        rows, ld = to_device_rows(rows_list, w, L.FP, gpu)
        layers.append(rows)
    target, _ = to_device_rows([s.target_rows for s in steps], w, L.N, gpu)

    def run():
        L.stats.zero_()
        for layer in range(w.D):
            vrt.build_tree(L.cfg, layer, layers[layer], ld, layers[layer].stride(0), seed, step, L.tree,
                           L.ws, L.stats)
        vrt.build_tree(L.cfg, vrt.FINISH, None, 0, 0, seed, step, L.tree, L.ws, L.stats)
        vrt.verify_tree(L.cfg, target, ld, target.stride(0), L.tree, seed, step, L.ws, L.out_tokens,
                        L.out_nodes, L.out_len, L.stats, L.node_out)

    print(f"graph replay: {name} B={w.B} V={w.V}", flush=True)
    run()  # eager once (lazy initialisation outside the capture)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work in between: scribble over the outputs and the tree's emitted arrays
        L.out_tokens.fill_(-9)
        L.views["node_token"].fill_(-9)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert (L.stats.cpu().numpy()[:, 0] == 0).all()
        for b, s in enumerate(steps):
            if s.exempt:
                continue
            compare_tree(w, s, L, b)
            Lt = len(s.out_tokens)
            assert L.out_len[b].item() == Lt, (rep, b)
            np.testing.assert_array_equal(L.out_tokens[b, :Lt].cpu().numpy(), s.out_tokens)
