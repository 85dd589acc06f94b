"""GPU soundness: bounds from the HIP library hold on 1e5 sampled points per instance.

The sampled network values are computed by a plain float64 torch forward pass
on the GPU (test infrastructure; the library is not involved), for points drawn
uniformly in the L-inf ball plus random ball corners.  A bound passes if every
sampled value lies within it up to the parity tolerance 1e-5 + 1e-4 |bound|.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads as wk
from helpers import ensure_built

pytestmark = pytest.mark.gpu
N_SAMPLES = 100_000


@pytest.fixture(scope="module")
def lbp():
    ensure_built()
    import linear_bound_propagation_amd as m
    return m


def _forward(nodes, x, dtype=torch.float64):
    """Values of every node for a batch x [n][*input shape] (NCHW), on x's device."""
    dev = x.device
    vals = []
    for nd in nodes:
        if nd.op == "input":
            v = x
        elif nd.op == "linear":
            v = vals[nd.inputs[0]] @ torch.as_tensor(nd.weight, dtype=dtype, device=dev).T + \
                torch.as_tensor(nd.bias, dtype=dtype, device=dev)
        elif nd.op == "conv":
            v = F.conv2d(vals[nd.inputs[0]], torch.as_tensor(nd.weight, dtype=dtype, device=dev),
                         torch.as_tensor(nd.bias, dtype=dtype, device=dev), stride=nd.stride, padding=nd.pad)
        elif nd.op == "relu":
            v = vals[nd.inputs[0]].clamp(min=0)
        elif nd.op == "add":
            v = vals[nd.inputs[0]] + vals[nd.inputs[1]]
        elif nd.op == "gap":
            v = vals[nd.inputs[0]].mean(dim=(2, 3))
        elif nd.op == "flatten":
            v = vals[nd.inputs[0]].reshape(x.shape[0], -1)
        vals.append(v)
    return vals


def _check(wl, b, bounds, node_bounds=None, chunk=10_000, dtype=torch.float64, seed=0):
    """Sample N_SAMPLES points around input b; check spec bounds (list of (lb, ub) [m])
    and optionally node bounds {k: (lo [size], hi [size])} (channels-last flattening)."""
    g = torch.Generator(device="cuda").manual_seed(seed + 7919 * b)
    x0 = torch.as_tensor(wl.x0[b], dtype=dtype, device="cuda")
    eps = float(wl.eps)
    C = torch.as_tensor(wl.C[b], dtype=dtype, device="cuda")
    worst = -float("inf")
    for start in range(0, N_SAMPLES, chunk):
        n = min(chunk, N_SAMPLES - start)
        u = torch.rand((n,) + x0.shape, generator=g, device="cuda", dtype=dtype) * 2 - 1
        n_corner = n // 5
        u[:n_corner] = torch.sign(u[:n_corner])
        x = x0 + eps * u
        vals = _forward(wl.nodes, x, dtype)
        spec = vals[-1] @ C.T
        for lb, ub in bounds:
            lb = lb.to(dtype)
            ub = ub.to(dtype)
            tl = 1e-5 + 1e-4 * lb.abs()
            tu = 1e-5 + 1e-4 * ub.abs()
            assert bool((spec >= lb - tl).all()), f"input {b}: spec value below its lower bound"
            assert bool((spec <= ub + tu).all()), f"input {b}: spec value above its upper bound"
            worst = max(worst, float((lb - spec.min(0).values).max()), float((spec.max(0).values - ub).max()))
        for k, (lo, hi) in (node_bounds or {}).items():
            v = vals[k]
            if v.dim() == 4:
                v = v.permute(0, 2, 3, 1)
            v = v.reshape(n, -1)
            lo = lo.to(dtype)
            hi = hi.to(dtype)
            assert bool((v >= lo - (1e-5 + 1e-4 * lo.abs())).all()), f"input {b}: node {k} below its lower bound"
            assert bool((v <= hi + (1e-5 + 1e-4 * hi.abs())).all()), f"input {b}: node {k} above its upper bound"
    return worst


def _crown(lbp, wl):
    net, x, C = lbp.prepare(wl)
    # the whole-batch workspace of the residual workload exceeds the device: a
    # smaller one makes the library process the batch in chunks (same results)
    need = net.workspace_size(wl.batch, wl.m, wl.intermediate, wl.region_start or 0)
    ws = net.workspace(min(need, int(torch.cuda.mem_get_info()[0] * 0.8)))
    out = lbp.crown(net, x, float(wl.eps), C, wl.intermediate, wl.region_start, ws=ws)
    torch.cuda.synchronize()
    return out


# every instance of every workload; the convolutional networks are sampled with a
# float32 forward pass (float64 convolutions are slow), whose rounding the
# tolerance of the check covers
@pytest.mark.parametrize("cfg,dtype", [(1, torch.float64), (2, torch.float64), (3, torch.float32)])
def test_sound_crown_and_ibp(lbp, cfg, dtype):
    wl = wk.config(cfg)
    print(wl.name, flush=True)
    out = _crown(lbp, wl)
    relu_inputs = [wl.nodes[k].inputs[0] for k, n in enumerate(wl.nodes) if n.op == "relu"]
    for b in range(wl.batch):
        nb = {z: (out["lo"][z][b], out["hi"][z][b]) for z in relu_inputs}
        w = _check(wl, b, [(out["lb"][b], out["ub"][b]), (out["ibp_lb"][b], out["ibp_ub"][b])], nb, dtype=dtype)
        print(f"  input {b}: sound; smallest gap between a sampled value and a bound: {-w:.4g}", flush=True)


def test_sound_alpha_crown_iterates(lbp):
    wl = wk.config(4)
    print(wl.name, flush=True)
    net, x, C = lbp.prepare(wl)
    out = lbp.crown(net, x, float(wl.eps), C, "ibp")
    lay = lbp.alpha_layout(net, out["lo"], out["hi"])   # the compact alpha state the benchmark uses
    best, lb_steps, _ = lbp.alpha_crown(net, x, float(wl.eps), C, out["lo"], out["hi"], wl.alpha_steps, wl.alpha_lr,
                                        layout=lay)
    torch.cuda.synchronize()
    for b in range(wl.batch):
        bounds = [(lb_steps[t][b], torch.full_like(best[b], float("inf"))) for t in range(lb_steps.shape[0])]
        bounds.append((best[b], out["ub"][b]))
        _check(wl, b, bounds, dtype=torch.float32)


@pytest.fixture(scope="module")
def residual_out(lbp):
    wl = wk.config(5)
    print(wl.name, flush=True)
    out = _crown(lbp, wl)
    return wl, {k: out[k].cpu() for k in ("lb", "ub", "ibp_lb", "ibp_ub")}


@pytest.mark.parametrize("part", range(4))
def test_sound_residual(lbp, residual_out, part):
    """All 32 inputs of the residual workload, eight per test."""
    wl, out = residual_out
    for b in range(8 * part, 8 * part + 8):
        bd = [(out["lb"][b].cuda(), out["ub"][b].cuda()), (out["ibp_lb"][b].cuda(), out["ibp_ub"][b].cuda())]
        w = _check(wl, b, bd, dtype=torch.float32)
        print(f"  input {b}: sound; smallest gap {-w:.4g}", flush=True)


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_sound_at_crown_attaining_vertices(lbp, cfg):
    """Row r's CROWN bound is the minimum over the input box of its linear bound
    Lambda_r x + beta_r, reached at the vertex x0 - eps sign(Lambda_r).  The linear
    bounds come from the library (vb_crown_backward returning Lambda over the input);
    at each of those 2m vertices per input, the network's value (float64 forward)
    must respect every spec bound and every intermediate bound."""
    wl = wk.config(cfg)
    print(wl.name, flush=True)
    net, x, C = lbp.prepare(wl)
    out = lbp.crown(net, x, float(wl.eps), C, wl.intermediate, wl.region_start)
    L = len(wl.nodes) - 1
    ws = net.workspace(net.workspace_size(wl.batch, wl.m, wl.intermediate, 0))
    _, _, A, _ = lbp.crown_backward(net, L, 0, out["lo"], out["hi"], x, float(wl.eps), ws, C=C, linear=True)
    torch.cuda.synchronize()
    relu_inputs = [wl.nodes[k].inputs[0] for k, n in enumerate(wl.nodes) if n.op == "relu"]
    in_shape = tuple(wl.nodes[0].shape)
    eps = float(np.float32(wl.eps))
    worst = float("inf")
    for b in range(wl.batch):
        x0 = torch.as_tensor(wl.x0[b], dtype=torch.float64, device="cuda")
        # Lambda rows are over the channels-last input; the vertices go back to (c, h, w)
        sg = torch.sign(A[b].double())
        if len(in_shape) == 3:
            c, h, w = in_shape
            sg = sg.reshape(-1, h, w, c).permute(0, 3, 1, 2)
        else:
            sg = sg.reshape((-1,) + in_shape)
        xv = x0 - eps * sg
        vals = _forward(wl.nodes, xv)
        spec = vals[-1] @ torch.as_tensor(wl.C[b], dtype=torch.float64, device="cuda").T
        lb = out["lb"][b].double()
        ub = out["ub"][b].double()
        assert bool((spec >= lb - (1e-5 + 1e-4 * lb.abs())).all()), f"input {b}: a vertex value below its lower bound"
        assert bool((spec <= ub + (1e-5 + 1e-4 * ub.abs())).all()), f"input {b}: a vertex value above its upper bound"
        m = wl.m
        own = torch.cat([spec[torch.arange(m), torch.arange(m)] - lb, ub - spec[m + torch.arange(m), torch.arange(m)]])
        worst = min(worst, float(own.min()))
        for z in relu_inputs:
            v = vals[z]
            if v.dim() == 4:
                v = v.permute(0, 2, 3, 1)
            v = v.reshape(v.shape[0], -1)
            lo, hi = out["lo"][z][b].double(), out["hi"][z][b].double()
            assert bool((v >= lo - (1e-5 + 1e-4 * lo.abs())).all()), f"input {b}: node {z} below its bound at a vertex"
            assert bool((v <= hi + (1e-5 + 1e-4 * hi.abs())).all()), f"input {b}: node {z} above its bound at a vertex"
    print(f"  smallest gap between a row's value at its own vertex and its bound: {worst:.4g}", flush=True)
