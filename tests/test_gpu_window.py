"""GPU parity of footprint-window back-substitution through residual blocks.

Identity rows (intermediate bounds) over a node of a residual stage keep their
Lambda on a window of each node they reach (the union of the convolution branch
and the skip), and each branch is concretised on its own reach at the domain.
These residual networks have stages wide enough that the windows are smaller
than the images, so the library takes that path (checked through its own
choice); every node's bounds and the spec bounds are compared with the float64
oracle in every mode, and the results are bitwise deterministic and the same
when the batch is processed in chunks.
"""
import ctypes

import numpy as np
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


NETS = {
    # 8-channel stages (scalar GEMM path), last stage 8 x 8
    "narrow": lambda: wk.resnet(2, 0.01, 81, widths=(4, 8), blocks=(1, 2), n_out=5, in_shape=(3, 16, 16)),
    # 32 / 64 channels (vector GEMM path with per-tile tap skipping), last stage 8 x 8
    "wide": lambda: wk.resnet(1, 0.004, 82, widths=(32, 64), blocks=(1, 2), n_out=10, in_shape=(3, 16, 16)),
    # one stage of two blocks on 12 x 12 (odd window clipping at the borders)
    "one_stage": lambda: wk.resnet(2, 0.01, 83, widths=(8,), blocks=(2,), n_out=4, in_shape=(2, 12, 12)),
}


def _paths(lbp, net, wl, stop):
    f = lbp.lib().vb_testing_identity_path
    f.restype = ctypes.c_int32
    f.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32]
    out = {}
    for k, nd in enumerate(wl.nodes):
        if nd.op != "relu":
            continue
        z = nd.inputs[0]
        if z > stop:
            out[z] = f(ctypes.cast(net.gp, ctypes.c_void_p), z, stop)
    return out


@pytest.mark.parametrize("mode", ["hybrid", "crown", "hybrid+ibp", "crown+ibp"])
@pytest.mark.parametrize("name", list(NETS))
def test_window_rows_through_residual_blocks(lbp, name, mode):
    wl = NETS[name]()
    wl.intermediate = mode
    net, x, C = lbp.prepare(wl)
    stop = wl.region_start if mode.startswith("hybrid") else 0
    paths = _paths(lbp, net, wl, stop)
    print(f"{name} {mode}: identity paths per ReLU input {paths}", flush=True)
    # (hybrid on the one-stage net: the region's first block adds the domain node itself
    # as its skip, which the window path does not take; those rows stay dense)
    if not (name == "one_stage" and mode.startswith("hybrid")):
        assert 2 in paths.values(), "no layer takes the window path"
    ref = crown_bounds(wl)
    out = lbp.crown(net, x, float(wl.eps), C, wl.intermediate, wl.region_start)
    torch.cuda.synchronize()
    compare_workload(wl, out, ref)


@pytest.mark.parametrize("name", ["narrow", "wide"])
def test_window_rows_deterministic_and_chunked(lbp, name):
    wl = NETS[name]()
    if wl.batch < 2:
        wl = wk.resnet(2, 0.004, 82, widths=(32, 64), blocks=(1, 2), n_out=10, in_shape=(3, 16, 16))
    net, x, C = lbp.prepare(wl)
    a = lbp.crown(net, x, float(wl.eps), C, "hybrid", wl.region_start)
    b = lbp.crown(net, x, float(wl.eps), C, "hybrid", wl.region_start)
    ws1 = net.workspace(net.workspace_size(1, wl.m, "hybrid", wl.region_start))
    c = lbp.crown(net, x, float(wl.eps), C, "hybrid", wl.region_start, ws=ws1)
    torch.cuda.synchronize()
    for key in ("lb", "ub"):
        assert torch.equal(a[key], b[key]), key
        assert torch.equal(a[key], c[key]), key
    for k in range(1, len(wl.nodes)):
        assert torch.equal(a["lo"][k], b["lo"][k]) and torch.equal(a["hi"][k], b["hi"][k]), k
        assert torch.equal(a["lo"][k], c["lo"][k]) and torch.equal(a["hi"][k], c["hi"][k]), k
