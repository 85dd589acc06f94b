"""GPU parity of IBP through Linear layers for small batches (at most 16 inputs), where
the library streams each weight matrix once with the batch on the MFMA columns and
splits long rows over several slices; against the float64 oracle.  With packed weight
copies (vb_pack_linear: the same numbers in 16 x 16 blocks in the lanes' read order)
every bound is bitwise the same as with the row-major weights."""
import numpy as np
import pytest
import torch

import workloads as wk
from helpers import assert_close, ensure_built
from oracle import Oracle, ibp as oracle_ibp, spec_bounds_ibp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lbp():
    ensure_built()
    import linear_bound_propagation_amd as m
    return m


def _check(lbp, wl, packed=False):
    net, x, C = lbp.prepare(wl)
    ws = net.workspace(net.workspace_size(wl.batch, wl.m, "ibp"))
    lo, hi, slo, shi = lbp.ibp(net, x, float(wl.eps), C=C, ws=ws)
    torch.cuda.synchronize()
    if packed:
        held = net.pack_linear()
        assert held > 0, "no Linear node with an input size that is a multiple of 16"
        plo, phi, pslo, pshi = lbp.ibp(net, x, float(wl.eps), C=C, ws=ws)
        torch.cuda.synchronize()
        for k in range(1, len(wl.nodes)):
            assert torch.equal(plo[k], lo[k]) and torch.equal(phi[k], hi[k]), f"packed node {k}"
        assert torch.equal(pslo, slo) and torch.equal(pshi, shi)
    on = Oracle(wl.nodes)
    rlo, rhi = oracle_ibp(on, wl.x0, wl.eps)
    for k, nd in enumerate(wl.nodes):
        if k == 0:
            continue
        assert_close(lo[k], rlo[k], f"lo[{k}] ({nd.op})")
        assert_close(hi[k], rhi[k], f"hi[{k}] ({nd.op})")
    rs_lo, rs_hi = spec_bounds_ibp(on, rlo, rhi, wl.C)
    assert_close(slo, rs_lo, "spec lo")
    assert_close(shi, rs_hi, "spec hi")


@pytest.mark.parametrize("widths,batch,eps,seed", [
    ([36, 1000, 77], 1, 0.05, 11),        # one input; ragged rows
    ([8200, 300, 20], 16, 0.01, 12),      # 16 inputs; 8200-long rows in 8 slices, last one short
    ([64, 4100, 12], 7, 0.02, 13),        # second layer over a box, 4 slices
    ([40, 36, 37, 9], 17, 0.05, 14),      # 17 inputs and a 37-long row: the general GEMM path
])
def test_narrow_ibp_ragged(lbp, widths, batch, eps, seed):
    print(f"narrow IBP {widths} batch {batch}", flush=True)
    _check(lbp, wk.tiny_mlp(widths, eps, seed, batch=batch))


@pytest.mark.parametrize("widths,batch,eps,seed", [
    ([48, 1000, 80, 9], 5, 0.05, 15),     # packed first layer with a ragged last 16-row block
    ([8192, 300, 32, 6], 16, 0.01, 16),   # packed 8192-long rows in slices; the 300-wide layer row-major
    ([64, 4096, 20], 3, 0.02, 17),        # packed second layer over a box, in slices
])
def test_narrow_ibp_packed_weights(lbp, widths, batch, eps, seed):
    print(f"narrow IBP packed {widths} batch {batch}", flush=True)
    _check(lbp, wk.tiny_mlp(widths, eps, seed, batch=batch), packed=True)


def test_wide_layer_full(lbp):
    """The 4096-262144-100 network (4.3 GB of first-layer weights), 8 inputs, every bound,
    with row-major and with packed weights."""
    wl = wk.wide()
    print(wl.name, flush=True)
    _check(lbp, wl, packed=True)
