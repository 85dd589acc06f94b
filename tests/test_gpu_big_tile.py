"""GPU parity of the 256 x 256-tile transposed-convolution GEMM (the variant the
launcher picks for back-substitution through convolutions with >= 256 input
channels when the grid has >= 512 such tiles), against the float64 oracle, for
each epilogue it has: relaxation into the ReLU below, concretisation over a box
domain, and the stored product (returned linear bounds).

The chain: 16 x 4 x 4 input -> conv 3x3 16->256 -> ReLU -> conv 3x3 256->32 ->
ReLU -> flatten -> linear.  Rows: 2048 margin-like rows e_i - e_j per input
(random pairs) over the 32 x 4 x 4 output of the second conv, both signs, two inputs: 8192 rows x 16
output pixels = 131072 GEMM rows = 512 tiles of 256, N = 256 (the first conv's
output channels), so the back-substitution through the second conv takes the
256 x 256 tile (asserted through the library's own tile choice).
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads as wk
from helpers import assert_close, ensure_built, nhwc
from oracle import backward, concretize
from test_gpu_entry_points import _f64, _fp32_bounds, _to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lbp():
    ensure_built()
    import linear_bound_propagation_amd as m
    return m


M_ROWS = 2048


@pytest.fixture(scope="module")
def chain(lbp):
    wl = wk.cnn(2, 0.02, 61, convs=((256, 1), (32, 1)), fcs=(10,), in_shape=(16, 4, 4), intermediate="ibp")
    on, lo, hi = _fp32_bounds(wl)
    net, x, _ = lbp.prepare(wl)
    dlo, dhi = _to_device(lbp, net, wl, lo, hi)
    start = 3                                       # the second conv
    shape = wl.nodes[start].shape
    # rows shaped like margin specifications: e_i - e_j for random pairs of neurons
    rng = np.random.default_rng(62)
    n = int(np.prod(shape))
    C = np.zeros((wl.batch, M_ROWS, n), dtype=np.float32)
    for b in range(wl.batch):
        i = rng.integers(0, n, M_ROWS)
        j = (i + rng.integers(1, n, M_ROWS)) % n
        C[b, np.arange(M_ROWS), i] = 1.0
        C[b, np.arange(M_ROWS), j] = -1.0
    C = C.reshape((wl.batch, M_ROWS) + tuple(shape))
    Cd = torch.as_tensor(nhwc(C.reshape((-1,) + tuple(shape)), shape).reshape(wl.batch, M_ROWS, -1),
                         device=x.device).contiguous()
    ws = net.workspace(2 << 30)
    return wl, on, lo, hi, net, x, dlo, dhi, start, C, Cd, ws


def test_this_shape_takes_the_256_tile(lbp):
    f = lbp.lib().vb_testing_conv_tile_n
    f.restype = ctypes.c_int32
    f.argtypes = [ctypes.c_int32] * 6
    rows = 2 * 2 * M_ROWS        # two inputs, both signs
    for mode in (0, 1, 2):       # store, relax, concretise
        assert f(mode, rows, 4, 4, 256, 32) == 256


def _domain(wl, lo, hi, b, stop):
    if stop == 0:
        c = _f64(wl.x0[b])
        return c, torch.full_like(c, float(np.float32(wl.eps)))
    return (lo[stop][b] + hi[stop][b]) / 2, (hi[stop][b] - lo[stop][b]) / 2


@pytest.mark.parametrize("stop", [0, 2])
def test_relax_and_concretise_epilogues(lbp, chain, stop):
    """stop = 0: the second conv's product is relaxed into the ReLU below (256-tile
    relaxation epilogue); stop = 2: it is concretised over that ReLU's box (256-tile
    concretisation epilogue)."""
    wl, on, lo, hi, net, x, dlo, dhi, start, C, Cd, ws = chain
    print(f"256-tile chain: rows over node {start} to node {stop}", flush=True)
    lb, ub = lbp.crown_backward(net, start, stop, dlo, dhi, x, float(wl.eps), ws, C=Cd)
    torch.cuda.synchronize()
    for b in range(wl.batch):
        c, r = _domain(wl, lo, hi, b, stop)
        rows = _f64(C[b])
        assert_close(lb[b], backward(on, lo, hi, b, start, rows, stop, c, r), f"lb input {b}")
        assert_close(ub[b], -backward(on, lo, hi, b, start, -rows, stop, c, r), f"ub input {b}")


def test_store_epilogue_returns_the_linear_bounds(lbp, chain):
    """stop = 2 with the linear bounds returned: the product is stored (256-tile store
    epilogue) and equals the oracle's Lambda over the ReLU node."""
    wl, on, lo, hi, net, x, dlo, dhi, start, C, Cd, ws = chain
    stop = 2
    print(f"256-tile chain: linear bounds over node {stop}", flush=True)
    lb, ub, A, bias = lbp.crown_backward(net, start, stop, dlo, dhi, x, float(wl.eps), ws, C=Cd, linear=True)
    torch.cuda.synchronize()
    shape = wl.nodes[stop].shape
    for b in range(wl.batch):
        c, r = _domain(wl, lo, hi, b, stop)
        for sgn, sl in ((1.0, slice(0, M_ROWS)), (-1.0, slice(M_ROWS, 2 * M_ROWS))):
            keep = {}
            val = backward(on, lo, hi, b, start, sgn * _f64(C[b]), stop, c, r, keep=keep)
            Lam = keep["domain"]
            beta = val - concretize(Lam, torch.zeros(M_ROWS, dtype=torch.float64), c, r)
            assert_close(A[b, sl], nhwc(Lam, shape), f"A input {b} sign {sgn}")
            assert_close(bias[b, sl], beta, f"bias input {b} sign {sgn}")
