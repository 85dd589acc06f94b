"""GPU parity: conv networks (implicit-GEMM conv / transposed conv) against the float64 oracle."""
import pytest
import torch

import workloads as wk
from helpers import assert_close, compare_workload, ensure_built
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
    # seven 3x3 convs: footprint windows up to 13 x 13 over the first conv's
    # output (more than 128 pixels: one window per workgroup onto the domain)
    (((8, 1),) * 7, (10, 5), (3, 16, 16), 1, 0.01, 14),
])
def test_cnn_small(lbp, method, convs, fcs, in_shape, batch, eps, seed):
    print(f"cnn {convs} {fcs} {in_shape} batch {batch} {method}", flush=True)
    wl = wk.cnn(batch, eps, seed, convs=convs, fcs=fcs, in_shape=in_shape, intermediate=method)
    ref = crown_bounds(wl)
    out = _run(lbp, wl)
    compare_workload(wl, out, ref)


@pytest.mark.parametrize("mode", ["hybrid", "hybrid+ibp"])
def test_cnn_hybrid_region_inside_conv_chain(lbp, mode):
    """The CROWN region starts at the first ReLU of a CNN (its IBP box is the domain):
    the identity rows of the third conv walk conv -> ReLU -> conv on footprint windows
    (the library's chain walker, checked through its own choice) and are concretised
    over that ReLU's box; every node's bounds and the spec bounds against the oracle."""
    import ctypes
    wl = wk.cnn(2, 0.03, 71, convs=((8, 1), (8, 2), (16, 1), (16, 1)), fcs=(10,), in_shape=(3, 12, 12),
                intermediate=mode)
    wl.region_start = 2
    net, x, C = lbp.prepare(wl)
    f = lbp.lib().vb_testing_identity_path
    f.restype = ctypes.c_int32
    f.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32]
    assert f(ctypes.cast(net.gp, ctypes.c_void_p), 5, 2) == 1, "the third conv's rows do not take the chain walker"
    ref = crown_bounds(wl)
    out = lbp.crown(net, x, float(wl.eps), C, wl.intermediate, wl.region_start)
    torch.cuda.synchronize()
    compare_workload(wl, out, ref)


def test_config3_full_size_sampled_inputs(lbp):
    wl = wk.config(3)
    print(wl.name, flush=True)
    out = _run(lbp, wl)
    idx = [0, 13, 31]
    ref = crown_bounds(wl, batch_idx=idx)
    compare_workload(wl, out, ref, batch_idx=idx)
    assert bool((out["lb"] <= out["ub"]).all())


def test_config3_crown_intermediates_sampled_rows(lbp):
    """The CNN of the measured configuration with CROWN intermediate bounds (each
    conv-output neuron's rows on its footprint window): for 40 sampled neurons of
    every CROWN-refined layer, the oracle's back-substitution over the same (GPU,
    fp32) bounds of the earlier layers gives the same bounds."""
    import numpy as np
    from helpers import nhwc
    from oracle import Oracle, backward
    wl = wk.config(3, batch=2)
    wl.intermediate = "crown"
    out = _run(lbp, wl)
    on = Oracle(wl.nodes)
    lo = [None] + [torch.as_tensor(np.zeros((wl.batch,) + tuple(nd.shape))) for nd in wl.nodes[1:]]
    hi = [None] + [torch.as_tensor(np.zeros((wl.batch,) + tuple(nd.shape))) for nd in wl.nodes[1:]]
    for k, nd in enumerate(wl.nodes):
        if k == 0 or nd.op == "flatten":
            continue
        g_lo = out["lo"][k].double().cpu().numpy()
        g_hi = out["hi"][k].double().cpu().numpy()
        if len(nd.shape) == 3:
            c, h, w = nd.shape
            g_lo = g_lo.reshape(wl.batch, h, w, c).transpose(0, 3, 1, 2)
            g_hi = g_hi.reshape(wl.batch, h, w, c).transpose(0, 3, 1, 2)
        lo[k] = torch.as_tensor(g_lo.reshape((wl.batch,) + tuple(nd.shape)).copy())
        hi[k] = torch.as_tensor(g_hi.reshape((wl.batch,) + tuple(nd.shape)).copy())
    rng = np.random.default_rng(3)
    relu_in = [nd.inputs[0] for nd in wl.nodes if nd.op == "relu"]
    b = 1
    c0 = torch.as_tensor(wl.x0[b].astype(np.float64))
    r0 = torch.full_like(c0, float(np.float32(wl.eps)))
    for z in relu_in[1:]:
        nd = wl.nodes[z]
        if nd.op != "conv":
            continue
        n = nd.size
        idx = rng.choice(n, 40, replace=False)
        rows = torch.zeros((80, n), dtype=torch.float64)
        rows[np.arange(40), idx] = 1.0
        rows[40 + np.arange(40), idx] = -1.0
        ref = backward(on, lo, hi, b, z, rows.reshape((80,) + tuple(nd.shape)), 0, c0, r0)
        c, h, w = nd.shape
        # sampled neuron (c, y, x) in NCHW order -> its channels-last position
        cc, yy, xx = np.unravel_index(idx, (c, h, w))
        pos = (yy * w + xx) * c + cc
        print(f"node {z}: {nd.shape}", flush=True)
        assert_close(out["lo"][z][b][pos], ref[:40], f"lo[{z}] sampled")
        assert_close(out["hi"][z][b][pos], -ref[40:], f"hi[{z}] sampled")


def _first_conv_net(seed, in_shape, c_out, k, stride, pad, batch=2, eps=0.02, intermediate="crown"):
    """conv(k, stride, pad) + ReLU, conv 3x3 + ReLU, flatten, FC, FC."""
    import numpy as np
    rng_w = np.random.default_rng([seed, 0])
    rng_x = np.random.default_rng([seed, 1])
    nb = wk.NetBuilder(rng_w, "he")
    x = nb.input(in_shape)
    x = nb.relu(nb.conv(x, c_out, k, stride, pad))
    x = nb.relu(nb.conv(x, 8, 3, 1, 1))
    x = nb.flatten(x)
    x = nb.relu(nb.linear(x, 16))
    x = nb.linear(x, 7)
    x0 = rng_x.random((batch,) + tuple(in_shape)).astype(np.float32)
    labels, C = wk.margin_specs(nb.nodes, x0)
    return wk.Workload("first_conv", seed, nb.nodes, x0, np.float32(eps), labels, C, intermediate)


@pytest.mark.parametrize("in_shape,c_out,k,stride,pad", [
    ((3, 11, 9), 8, 3, 2, 1),     # stride 2, odd sizes: taps of both parities
    ((1, 12, 12), 12, 3, 1, 2),   # one input channel, padding wider than the halo
    ((4, 9, 10), 16, 3, 2, 0),    # four input channels, no padding
    ((2, 7, 7), 4, 3, 1, 1),      # two input channels
    # shapes the direct matrix-core kernel takes (Co a multiple of 16 up to
    # 64): every (input channels, tap-table width, stride) instance
    ((1, 12, 12), 16, 3, 1, 2),   # 1 channel, 9 columns, stride 1
    ((1, 15, 15), 16, 3, 2, 1),   # 1 channel, stride 2
    ((2, 20, 20), 32, 3, 1, 1),   # 18 columns; bands of 12 rows, ragged last band
    ((2, 10, 10), 16, 2, 2, 0),   # 2x2 kernel: 8 columns, stride 2
    ((3, 6, 6), 16, 2, 1, 0),     # 3 channels, 12 columns
    ((3, 13, 17), 48, 3, 2, 1),   # 27 columns, stride 2, odd sizes
    ((3, 5, 150), 16, 3, 1, 1),   # wide image: one-row bands, ragged M-blocks
    ((4, 8, 8), 64, 3, 1, 1),     # 36 columns (three column blocks), 64 channels
    ((4, 8, 8), 32, 2, 2, 0),     # 4 channels, 16 columns, stride 2
])
def test_first_conv_to_domain(lbp, in_shape, c_out, k, stride, pad):
    """The transposed first conv and the concretisation over the input box in one
    kernel (few input channels): every bound of the network against the oracle."""
    wl = _first_conv_net(31, in_shape, c_out, k, stride, pad)
    print(f"first conv {in_shape} -> {c_out} k{k} s{stride} p{pad}", flush=True)
    ref = crown_bounds(wl)
    out = _run(lbp, wl)
    compare_workload(wl, out, ref)
