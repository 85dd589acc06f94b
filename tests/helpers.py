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
