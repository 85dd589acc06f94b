"""GPU parity at full size against the float64 oracle's own bounds end to end.

The oracle takes minutes per input at these sizes, so its results were written
once by tests/golden/make_full_size.py (which calls only the oracle and the
seeded workload generators) into tests/golden/full_size_*.npz: the spec bounds
by CROWN and IBP of the stored inputs, and a seeded sample of 2048 neurons of
every CROWN-refined layer with the oracle's bounds.  Here the GPU runs the whole
pipeline on the same inputs and every stored value is compared.

* The residual workload (hybrid: IBP up to the last stage, CROWN inside it), inputs
  0 and 1.  Its back-substitution through the 256 -> 256 3x3 convolutions at 8 x 8
  (32768 identity rows per input: 32768 x 2 x 64 / 256 = 16384 tiles of 256 rows)
  takes the 256 x 256-tile GEMM, asserted through the library's own tile choice.
* The CNN workload with CROWN intermediate bounds (footprint rows through the conv
  chain), input 0.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import workloads as wk
from helpers import assert_close, ensure_built

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def fingerprint(wl):
    """The generator's checksum of the seeded parameters and inputs."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("_make_full_size", os.path.join(GOLDEN, "make_full_size.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.fingerprint(wl)


@pytest.fixture(scope="module")
def lbp():
    ensure_built()
    import linear_bound_propagation_amd as m
    return m


def _nhwc_index(idx, shape):
    C, H, W = shape
    c, rem = np.divmod(idx, H * W)
    y, x = np.divmod(rem, W)
    return (y * W + x) * C + c


def _check(lbp, name, cfg, method=None):
    g = np.load(os.path.join(GOLDEN, f"full_size_{name}.npz"))
    inputs = g["inputs"].tolist()
    wl = wk.config(cfg, batch=max(inputs) + 1)
    if method:
        wl.intermediate = method
    assert str(g["intermediate"]) == wl.intermediate
    assert np.allclose(fingerprint(wl), g["fingerprint"], rtol=1e-12, atol=0), "seeded workload changed"
    print(f"{wl.name} ({wl.intermediate}): inputs {inputs}", flush=True)
    net, x, C = lbp.prepare(wl)
    out = lbp.crown(net, x, float(wl.eps), C, wl.intermediate, wl.region_start)
    torch.cuda.synchronize()
    worst = 0.0
    for key in ("lb", "ub", "ibp_lb", "ibp_ub"):
        worst = max(worst, assert_close(out[key][inputs], g[key], key))
    for z in g["layers"].tolist():
        shape = wl.nodes[z].shape
        idx = g[f"idx_{z}"]
        col = _nhwc_index(idx, shape) if len(shape) == 3 else idx
        col = torch.as_tensor(col, device=x.device)
        for j, b in enumerate(inputs):
            worst = max(worst, assert_close(out["lo"][z][b][col], g[f"lo_{z}"][j], f"lo[{z}] input {b}"))
            worst = max(worst, assert_close(out["hi"][z][b][col], g[f"hi_{z}"][j], f"hi[{z}] input {b}"))
    print(f"  {len(g['layers'])} refined layers, worst |d| / allowed = {worst:.3g}", flush=True)
    return wl, out


def test_residual_workload_end_to_end(lbp):
    f = lbp.lib().vb_testing_conv_tile_n
    f.restype = ctypes.c_int32
    f.argtypes = [ctypes.c_int32] * 6
    assert f(1, 2 * 32768, 8, 8, 256, 256) == 256
    wl, out = _check(lbp, "resnet_hybrid", 5)
    assert bool((out["lb"] <= out["ub"]).all())


def test_cnn_crown_intermediates_end_to_end(lbp):
    _check(lbp, "cnn_crown", 3, "crown")
