"""GPU parity: IBP and CROWN on MLPs through the C ABI against the float64 oracle."""
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


def _run(lbp, wl, method=None):
    net, x, C = lbp.prepare(wl)
    out = lbp.crown(net, x, float(wl.eps), C, method or wl.intermediate, wl.region_start)
    torch.cuda.synchronize()
    return net, out


def _compare(wl, out, ref, batch_idx=None, check_nodes=True):
    compare_workload(wl, out, ref, batch_idx, check_nodes)


@pytest.mark.parametrize("widths,batch,eps,seed", [
    ([50, 130, 97, 200, 11], 5, 0.05, 1),      # ragged: no dimension a multiple of the tiles
    ([37, 64, 128, 33, 7], 3, 0.1, 2),
    ([300, 257, 129, 10], 9, 0.02, 3),
])
def test_mlp_small_ragged(lbp, widths, batch, eps, seed):
    print(f"mlp {widths} batch {batch} eps {eps}", flush=True)
    wl = wk.tiny_mlp(widths, eps, seed, batch=batch)
    for method in ("crown", "ibp"):
        wl.intermediate = method
        ref = crown_bounds(wl)
        _, out = _run(lbp, wl)
        _compare(wl, out, ref)


@pytest.mark.parametrize("widths,batch,eps,seed", [
    ([50, 130, 97, 200, 11], 5, 0.05, 1),
    ([300, 257, 129, 10], 9, 0.02, 3),
])
def test_mlp_crown_intersected_with_ibp(lbp, widths, batch, eps, seed):
    wl = wk.tiny_mlp(widths, eps, seed, batch=batch)
    wl.intermediate = "crown+ibp"
    ref = crown_bounds(wl)
    _, out = _run(lbp, wl)
    _compare(wl, out, ref)


def test_config1_full(lbp):
    wl = wk.config(1)
    print(wl.name, flush=True)
    ref = crown_bounds(wl)
    _, out = _run(lbp, wl)
    _compare(wl, out, ref)
    # sound and ordered
    assert bool((out["lb"] <= out["ub"]).all())


def test_config2_full_size_sampled_inputs(lbp):
    wl = wk.config(2)
    print(wl.name, flush=True)
    _, out = _run(lbp, wl)
    idx = [0, 37, 63]
    ref = crown_bounds(wl, batch_idx=idx)
    _compare(wl, out, ref, batch_idx=idx)


def test_determinism_bitwise(lbp):
    wl = wk.tiny_mlp([300, 257, 129, 10], 0.02, 3, batch=9)
    net, x, C = lbp.prepare(wl)
    a = lbp.crown(net, x, float(wl.eps), C, "crown")
    b = lbp.crown(net, x, float(wl.eps), C, "crown")
    torch.cuda.synchronize()
    for key in ("lb", "ub", "ibp_lb", "ibp_ub"):
        assert torch.equal(a[key], b[key]), key
    for k in range(1, len(wl.nodes)):
        assert torch.equal(a["lo"][k], b["lo"][k]) and torch.equal(a["hi"][k], b["hi"][k])


def test_chunked_workspace_matches_whole_batch(lbp):
    wl = wk.tiny_mlp([120, 90, 80, 6], 0.05, 4, batch=7)
    net, x, C = lbp.prepare(wl)
    full = lbp.crown(net, x, float(wl.eps), C, "crown")
    per_b = net.workspace_size(1, C.shape[1], "crown")
    ws = net.workspace(per_b * 2)           # room for about two batch elements at a time
    part = lbp.crown(net, x, float(wl.eps), C, "crown", ws=ws)
    torch.cuda.synchronize()
    for key in ("lb", "ub"):
        assert torch.equal(full[key], part[key]), key


@pytest.mark.parametrize("mode", ["crown+unstable", "crown+ibp+unstable"])
@pytest.mark.parametrize("which", ["tiny", "config1"])
def test_unstable_only_rows(lbp, which, mode):
    """Rows only for the IBP-unstable neurons of each Linear layer: every node's
    bounds and the spec bounds against the oracle's unstable-only mode; and with the
    IBP intersection the spec bounds are bitwise those of all rows (stable neurons
    keep their class, so every relaxation is the same)."""
    wl = wk.config(1) if which == "config1" else wk.tiny_mlp([40, 64, 48, 48, 7], 0.07, 61, batch=3)
    wl.intermediate = mode
    print(f"{wl.name} {mode}", flush=True)
    ref = crown_bounds(wl)
    _, out = _run(lbp, wl)
    _compare(wl, out, ref)
    if "ibp" in mode.split("+")[1:]:
        _, full = _run(lbp, wl, "crown+ibp")
        assert torch.equal(out["lb"], full["lb"]) and torch.equal(out["ub"], full["ub"])


def test_unstable_only_rows_config2_equal_to_all_rows(lbp):
    wl = wk.config(2, batch=8)
    _, out = _run(lbp, wl, "crown+ibp+unstable")
    _, full = _run(lbp, wl, "crown+ibp")
    assert torch.equal(out["lb"], full["lb"]) and torch.equal(out["ub"], full["ub"])
