"""vrt_verify_tree_static (the verification on the library's static per-GPU workspace, for
callers that cannot allocate) against vrt_verify_tree with a workspace of its own: the same
outputs, bit for bit, on two calls in a row, the second with a smaller batch; a
configuration whose workspace exceeds the static array is refused before any launch."""
import numpy as np
import pytest
import torch

import synth
from oracle.drive import OracleStep
from tests.gpu_common import Lib, lib_config, to_device_rows
from tests.test_gpu_build import _small, gpu_build
from verify_row_top_amd import vrt

pytestmark = pytest.mark.gpu


def _check_against_workspace_call(w, seed, step, dev):
    steps = [OracleStep(w, seed, b, step, verify=False) for b in range(w.B)]
    L = gpu_build(w, steps, seed, step, dev)
    target, ld = to_device_rows([s.target_rows for s in steps], w, L.N, dev)
    L.verify(target, ld, seed, step)
    ref = [x.clone() for x in (L.out_tokens, L.out_nodes, L.out_len, L.stats, L.node_out)]
    for x in (L.out_tokens, L.out_nodes, L.out_len, L.node_out):
        x.fill_(-7)
    L.stats.zero_()
    vrt.verify_tree_static(L.cfg, target, ld, target.stride(0), L.tree, seed, step, L.out_tokens, L.out_nodes,
                           L.out_len, L.stats, L.node_out)
    torch.cuda.synchronize()
    for got, want, name in zip((L.out_tokens, L.out_nodes, L.out_len, L.stats, L.node_out), ref,
                               ("out_tokens", "out_nodes", "out_len", "stats", "node_out")):
        assert torch.equal(got, want), name
    # decisions in the static array itself (node_out NULL) give the same tokens
    L.out_tokens.fill_(-7)
    vrt.verify_tree_static(L.cfg, target, ld, target.stride(0), L.tree, seed, step, L.out_tokens, L.out_nodes,
                           L.out_len, L.stats)
    torch.cuda.synchronize()
    assert torch.equal(L.out_tokens, ref[0])


def test_static_workspace_call_equals_the_workspace_call(gpu):
    print("static-workspace verification: B=8, then B=3", flush=True)
    _check_against_workspace_call(_small(B=8, V=7000, R=40, D=5), 3, 1, gpu)
    _check_against_workspace_call(_small(B=3, V=3000, R=20, D=4, dtype=synth.F32), 4, 2, gpu)


def test_static_workspace_refuses_oversized_configs(gpu):
    cfg = vrt.make_config(B=4096, V=1000, dtype=vrt.F32, K=4, D=2, R=1000)
    assert vrt.workspace_bytes(cfg) > 4 << 20
    t = torch.zeros(16, dtype=torch.int32, device=gpu)
    with pytest.raises(vrt.VrtError) as e:
        vrt.verify_tree_static(cfg, t, 1000, 1000, t, 1, 0, t, t, t, t)
    assert e.value.code == vrt.ENOMEM and "static" in str(e.value)
