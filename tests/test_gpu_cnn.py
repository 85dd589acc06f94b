"""GPU parity: conv networks (implicit-GEMM conv / transposed conv) against the float64 oracle."""
import pytest
import torch

import workloads as wk
from helpers import compare_workload, ensure_built
from oracle import crown_bounds

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lbp():
    ensure_built()
    import linear_bound_propagation_amd as m
    return m


def _run(lbp, wl):
    net, x, C = lbp.prepare(wl)
    out = lbp.crown(net, x, float(wl.eps), C, wl.intermediate, wl.region_start)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("method", ["ibp", "crown", "crown+ibp"])
@pytest.mark.parametrize("convs,fcs,in_shape,batch,eps,seed", [
    # odd spatial sizes: stride-2 parity classes of different sizes; C_in = 3
    (((8, 1), (16, 2), (8, 1)), (20, 10), (3, 9, 9), 3, 0.02, 11),
    # channel counts that are not multiples of the tiles, two stride-2 layers
    (((5, 2), (33, 1), (70, 2)), (37, 6), (2, 10, 7), 2, 0.01, 12),
    # the configuration's layer sequence at a reduced width
    (((16, 1), (16, 2), (32, 1), (32, 2)), (64, 10), (3, 16, 16), 2, 0.004, 13),
])
def test_cnn_small(lbp, method, convs, fcs, in_shape, batch, eps, seed):
    print(f"cnn {convs} {fcs} {in_shape} batch {batch} {method}", flush=True)
    wl = wk.cnn(batch, eps, seed, convs=convs, fcs=fcs, in_shape=in_shape, intermediate=method)
    ref = crown_bounds(wl)
    out = _run(lbp, wl)
    compare_workload(wl, out, ref)


def test_config3_full_size_sampled_inputs(lbp):
    wl = wk.config(3)
    print(wl.name, flush=True)
    out = _run(lbp, wl)
    idx = [0, 13, 31]
    ref = crown_bounds(wl, batch_idx=idx)
    compare_workload(wl, out, ref, batch_idx=idx)
    assert bool((out["lb"] <= out["ub"]).all())
