"""GPU parity: residual networks (ADD, 1x1 stride-2 projections, GAP, hybrid IBP/CROWN)."""
import numpy as np
import pytest
import torch

import workloads as wk
from helpers import assert_close, compare_workload, ensure_built, nhwc
from oracle import Oracle, backward, crown_bounds, ibp
from oracle.bounds import _identity_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lbp():
    ensure_built()
    import linear_bound_propagation_amd as m
    return m


def _run(lbp, wl, ws=None):
    net, x, C = lbp.prepare(wl)
    out = lbp.crown(net, x, float(wl.eps), C, wl.intermediate, wl.region_start, ws=ws)
    torch.cuda.synchronize()
    return net, out


@pytest.mark.parametrize("method", ["hybrid", "crown", "ibp", "hybrid+ibp", "crown+ibp"])
def test_resnet_small(lbp, method):
    wl = wk.resnet(2, 0.01, 31, widths=(4, 6, 8), blocks=(1, 2, 2), n_out=5, in_shape=(3, 8, 8))
    wl.intermediate = method
    print(f"resnet small {method}", flush=True)
    ref = crown_bounds(wl)
    _, out = _run(lbp, wl)
    compare_workload(wl, out, ref)


def test_resnet_odd_sizes_hybrid(lbp):
    wl = wk.resnet(3, 0.005, 32, widths=(5, 7, 9), blocks=(1, 1, 2), n_out=4, in_shape=(2, 7, 9))
    print("resnet odd sizes hybrid", flush=True)
    ref = crown_bounds(wl)
    _, out = _run(lbp, wl)
    compare_workload(wl, out, ref)


def test_config5_full_size(lbp):
    wl = wk.config(5, batch=2)
    print(wl.name, "region starts at node", wl.region_start, flush=True)
    net, out = _run(lbp, wl)
    # chunked workspace (one input at a time) gives bitwise the same bounds
    ws1 = net.workspace(net.workspace_size(1, wl.m, "hybrid", wl.region_start))
    _, out1 = _run(lbp, wl, ws=ws1)
    for key in ("lb", "ub"):
        assert torch.equal(out[key], out1[key]), key
    assert bool((out["lb"] <= out["ub"]).all())
    # IBP bounds of every node up to the region (channels-last) against the oracle
    onet = Oracle(wl.nodes)
    lo, hi = ibp(onet, wl.x0, wl.eps)
    for k in range(1, wl.region_start + 1):
        if wl.nodes[k].op in ("conv", "add", "relu"):
            assert_close(out["lo"][k], nhwc(lo[k], wl.nodes[k].shape), f"ibp lo[{k}]")
            assert_close(out["hi"][k], nhwc(hi[k], wl.nodes[k].shape), f"ibp hi[{k}]")
    # first CROWN layer of the region: sampled rows, back-substituted to the IBP box of the region input
    v = wl.region_start
    relus = [k for k, n in enumerate(wl.nodes) if n.op == "relu" and k > v]
    z = next(wl.nodes[r].inputs[0] for r in relus if wl.nodes[wl.nodes[r].inputs[0]].op == "add")
    shape = wl.nodes[z].shape
    n = int(np.prod(shape))
    rng = np.random.default_rng(0)
    sample = np.sort(rng.choice(n, 48, replace=False))
    for b in range(wl.batch):
        dc, dr = (lo[v][b] + hi[v][b]) / 2, (hi[v][b] - lo[v][b]) / 2
        eye = _identity_rows(shape, 1.0).reshape(n, -1)[sample].reshape((len(sample),) + shape)
        lz = backward(onet, lo, hi, b, z, eye, v, dc, dr)
        uz = -backward(onet, lo, hi, b, z, -eye, v, dc, dr)
        # the library stores node z channels-last: index (y*W + x)*C + c of NCHW index c*H*W + y*W + x
        C_, H, W = shape
        cc, rem = np.divmod(sample, H * W)
        yy, xx = np.divmod(rem, W)
        idx = (yy * W + xx) * C_ + cc
        assert_close(out["lo"][z][b][idx], lz, f"crown lo[{z}] sampled")
        assert_close(out["hi"][z][b][idx], uz, f"crown hi[{z}] sampled")
