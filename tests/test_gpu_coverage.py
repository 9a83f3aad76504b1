"""GPU parity of vrt_support_coverage (the coverage column of RheoSampling's
support-size ablation) against the oracle's support mass, row by row: generator rows
of the workloads (peaked and flat, bf16 and fp32, full vocabulary), every support
size of the ablation and the dense case, and edge rows (ties, -inf, NaN, short rows).
Within 1e-6 absolute (the kernel's exponentials are good to about 1e-7 relative)."""
import numpy as np
import pytest
import torch

import synth
from oracle import oracle as orc
from synth import workloads
from tests.gpu_common import lib_config, row_ld, to_device_rows
from verify_row_top_amd import vrt

pytestmark = pytest.mark.gpu

TRUNCS = (1, 4, 128, 256, 512, 1024, vrt.DENSE)


def _rows(w, n, seed):
    keys = np.array([synth.root_key(seed + i, 0) for i in range(n)], np.uint64)
    return synth.rows_host(w.params(), w.tables(), keys, np.zeros(n, np.int32), synth.DRAFT)


def _gpu_coverage(w, rows, trunc, dev):
    cfg = lib_config(w, B=1, trunc=trunc)
    d, ld = to_device_rows([rows], w, rows.shape[0], dev)
    out = torch.full((1, rows.shape[0]), -1.0, dtype=torch.float64, device=dev)
    vrt.support_coverage(cfg, d, ld, d.stride(0), rows.shape[0], out)
    torch.cuda.synchronize()
    return out[0].cpu().numpy()


@pytest.mark.parametrize("name,w", [
    ("headline_bf16", workloads.get("headline")),
    ("flat_bf16", workloads.get("headline").replace(zipf=(0.8,))),
    ("fp32_V70001", workloads.get("headline").replace(dtype=synth.F32, V=70001)),
    ("short_rows_V900", workloads.get("headline").replace(V=900)),
])
def test_coverage_matches_oracle(gpu, name, w):
    rows = _rows(w, 12, 31)
    f = synth.to_f32(rows)
    for trunc in TRUNCS:
        print(f"coverage parity: {name} V={w.V} trunc={trunc}", flush=True)
        got = _gpu_coverage(w, rows, trunc, gpu)
        ref = np.array([orc.support_mass(r, trunc if trunc != vrt.DENSE else w.V) for r in f])
        np.testing.assert_allclose(got, ref, atol=1e-6, rtol=0, err_msg=f"trunc={trunc}")


def _bf16_bits(x):
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x, np.float32))
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16], ids=["fp32", "bf16"])
def test_coverage_edge_rows(gpu, dtype):
    w = workloads.get("headline").replace(V=3000, dtype=dtype)
    rows = np.zeros((5, w.V), np.float32)          # row 0: all ties
    rows[1] = -np.inf                              # row 1: no finite logit
    rows[2] = -np.inf
    rows[2, 17] = 3.0                              # row 2: one finite logit
    rows[3] = np.linspace(0, -30, w.V, dtype=np.float32)
    rows[4] = 1.0
    rows[4, 5] = np.nan                            # row 4: NaN
    if dtype == synth.BF16:
        rows = _bf16_bits(rows)
    f = synth.to_f32(rows) if dtype == synth.BF16 else rows
    for trunc in (128, 1024, vrt.DENSE):
        got = _gpu_coverage(w, rows, trunc, gpu)
        share = 1.0 if trunc == vrt.DENSE else trunc / w.V
        assert abs(got[0] - share) < 1e-6
        assert got[1] == 0.0
        assert got[2] == 1.0 or abs(got[2] - 1.0) < 1e-12
        ref = orc.support_mass(f[3], trunc if trunc != vrt.DENSE else w.V)
        assert abs(got[3] - ref) < 1e-6
        assert np.isnan(got[4])


def test_coverage_argument_errors(gpu):
    w = workloads.get("headline").replace(V=3000)
    cfg = lib_config(w, B=1)
    d = torch.zeros((1, 2, row_ld(w)), dtype=torch.int16, device=gpu)
    out = torch.zeros((1, 2), dtype=torch.float64, device=gpu)
    with pytest.raises(vrt.VrtError):
        vrt.support_coverage(cfg, d, row_ld(w), d.stride(0), 0, out)
    with pytest.raises(vrt.VrtError):
        vrt.support_coverage(cfg, d, w.V - 1, d.stride(0), 2, out)
