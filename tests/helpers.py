"""Shared test helpers: library loading, tolerance checks, layout conversion."""
import os

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "linear_bound_propagation_amd", "libvbprop.so")

# parity bar: |gpu - oracle| <= ATOL + RTOL * |oracle|, elementwise
ATOL = 1e-5
RTOL = 1e-4


def ensure_built():
    if not os.path.exists(LIB):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_vbprop_build", os.path.join(ROOT, "linear_bound_propagation_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()


def nhwc(t, shape):
    """Oracle tensor [B][*shape] (float64, NCHW) -> numpy [B][size] in the library's layout."""
    a = t.detach().cpu().numpy() if isinstance(t, torch.Tensor) else np.asarray(t)
    if len(shape) == 3:
        a = a.transpose(0, 2, 3, 1)
    return a.reshape(a.shape[0], -1)


def assert_close(gpu, ref, what, atol=ATOL, rtol=RTOL):
    g = gpu.detach().double().cpu().numpy() if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = ref.detach().cpu().numpy() if isinstance(ref, torch.Tensor) else np.asarray(ref, np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    err = np.abs(g - r)
    bound = atol + rtol * np.abs(r)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} outside tolerance; worst at {i}: "
                             f"gpu {g[i]!r} oracle {r[i]!r} (|d| = {err[i]:.3g}, allowed {bound[i]:.3g})")
    return float((err / bound).max()) if err.size else 0.0


def near_ties(lo, hi, relu_inputs, tau=1e-5):
    """Neurons whose adaptive lower-slope decision u >= -l is within tau*(u-l) of flipping."""
    n = 0
    for z in relu_inputs:
        l, u = lo[z], hi[z]
        unst = (l < 0) & (u > 0)
        n += int((unst & ((u + l).abs() <= tau * (u - l))).sum())
    return n


def gpu_decisions(wl, out, relu_inputs):
    """The library's adaptive lower-slope choice (a = 1 iff u >= -l, compared in float32
    on the bounds it returned) for every neuron of each ReLU input, as [B][*shape]
    boolean tensors in the oracle's layout."""
    import torch
    dec = {}
    for z in relu_inputs:
        lo = out["lo"][z].detach().cpu()
        hi = out["hi"][z].detach().cpu()
        a = hi >= -lo
        shape = tuple(wl.nodes[z].shape)
        if len(shape) == 3:
            c, h, w = shape
            a = a.reshape(-1, h, w, c).permute(0, 3, 1, 2)
        dec[z] = a.reshape((-1,) + shape).clone()
    return dec


def aligned_reference(wl, out, ref, idx, relu_inputs, tau=1e-6):
    """Decision-aligned parity at the adaptive-slope tie: count the neurons where the
    oracle sits within tau*(u-l) of the tie u = -l and chose differently from the
    library; if there are any, recompute the oracle taking the library's choice at
    exactly those near-tie neurons (both choices are sound).  Returns (reference,
    number of aligned neurons)."""
    import torch
    from oracle import crown_bounds
    dec = gpu_decisions(wl, out, relu_inputs)
    flips = 0
    for z in relu_inputs:
        l, u = ref["lo"][z][idx], ref["hi"][z][idx]
        unst = (l < 0) & (u > 0)
        tie = unst & ((u + l).abs() <= tau * (u - l))
        flips += int((tie & ((u >= -l) != dec[z][idx])).sum())
    if flips == 0:
        return ref, 0
    return crown_bounds(wl, batch_idx=idx, decide=dec), flips


def compare_workload(wl, out, ref, batch_idx=None, check_nodes=True, keys=("lb", "ub", "ibp_lb", "ibp_ub")):
    """Elementwise parity of a vb_crown result with the oracle's crown_bounds result
    (decision-aligned at adaptive-slope ties, see aligned_reference)."""
    idx = list(range(wl.batch)) if batch_idx is None else list(batch_idx)
    relu_inputs = [wl.nodes[k].inputs[0] for k, n in enumerate(wl.nodes) if n.op == "relu"]
    ties = near_ties({z: ref["lo"][z][idx] for z in relu_inputs},
                     {z: ref["hi"][z][idx] for z in relu_inputs}, relu_inputs)
    ref, aligned = aligned_reference(wl, out, ref, idx, relu_inputs)
    print(f"{wl.name} ({wl.intermediate}): near-tie neurons in the oracle: {ties}; "
          f"decisions aligned to the library's: {aligned}", flush=True)
    worst = 0.0
    for key in keys:
        worst = max(worst, assert_close(out[key][idx], ref[key][idx], key))
    if check_nodes:
        for k, nd in enumerate(wl.nodes):
            if k == 0 or nd.op not in ("linear", "conv", "add"):
                continue
            worst = max(worst, assert_close(out["lo"][k][idx], nhwc(ref["lo"][k][idx], nd.shape), f"lo[{k}]"))
            worst = max(worst, assert_close(out["hi"][k][idx], nhwc(ref["hi"][k][idx], nd.shape), f"hi[{k}]"))
    print(f"  worst |d| / allowed = {worst:.3g}", flush=True)
    return worst
