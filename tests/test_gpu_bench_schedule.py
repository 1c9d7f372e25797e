"""The two-stream step schedule of bench.py computes exactly what the one-stream
schedule computes (every cast and GEMM output, bit for bit), over repeated steps
so that a missing wait between steps would show."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import bench  # noqa: E402
import fine_grained_block_amd as fgb  # noqa: E402
from fine_grained_block_amd import workloads as wl  # noqa: E402

pytestmark = pytest.mark.gpu


def _outputs(bufs):
    return {k: v.clone() for k, v in bufs.items()}


@pytest.mark.parametrize("ue8m0,two_stage", [(False, False), (True, False), (True, True)])
def test_linear_overlap_matches_serial(ue8m0, two_stage):
    dev = torch.device("cuda:0")
    M, K, N = 640, 1024, 896
    d = {"M": M, "K": K, "N": N,
         "x": wl.normal_bf16((M, K), 0.02, 5, 0), "w": wl.normal_bf16((K, N), 0.02, 5, 1),
         "dy": wl.normal_bf16((M, N), 1e-3, 5, 2)}
    res = {}
    for overlap in (False, True):
        bufs = {}
        kernels = bench.linear_step(fgb, torch, dev, d, ue8m0=ue8m0, bufs=bufs, two_stage=two_stage)
        for b in bufs.values():
            b.zero_()
        step = bench.make_runner(torch, dev, kernels, overlap)
        for _ in range(4):
            step()
        torch.cuda.synchronize()
        res[overlap] = _outputs(bufs)
    for k in res[False]:
        a, b = res[False][k], res[True][k]
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), k


def test_moe_overlap_matches_serial():
    dev = torch.device("cuda:0")
    d = wl.moe_grouped(tokens=256, experts=8, topk=2, d_model=256, d_ff2=512, d_ff=256)
    res = {}
    for overlap in (False, True):
        bufs = {}
        kernels = bench.moe_step(fgb, torch, dev, d, bufs=bufs)
        step = bench.make_runner(torch, dev, kernels, overlap)
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        res[overlap] = _outputs(bufs)
    for k in res[False]:
        a, b = res[False][k], res[True][k]
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), k
