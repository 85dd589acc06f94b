"""Bitwise determinism of every back-substitution path: two identical calls give
identical bits (no float atomics; every sum runs in a fixed order).  Covers the
convolution gather GEMM with its stride-2 parity classes, footprint rows on the
conv chain walker (over the input and over an inner ReLU's box), footprint
windows through residual blocks (including the two branches concretised in one
GEMM), unstable-only identity rows, and alpha-CROWN with compact and dense state."""
import pytest
import torch

import workloads as wk
from helpers import ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lbp():
    ensure_built()
    import linear_bound_propagation_amd as m
    return m


def _hybrid_cnn():
    wl = wk.cnn(2, 0.03, 71, convs=((8, 1), (8, 2), (16, 1), (16, 1)), fcs=(10,), in_shape=(3, 12, 12),
                intermediate="hybrid")
    wl.region_start = 2
    return wl


CASES = {
    "cnn_gather_ibp": lambda: wk.cnn(3, 0.02, 11, convs=((8, 1), (16, 2), (8, 1)), fcs=(20, 10), in_shape=(3, 9, 9)),
    "cnn_footprint_chain_crown": lambda: wk.cnn(2, 0.01, 14, convs=((8, 1),) * 7, fcs=(10, 5), in_shape=(3, 16, 16),
                                                intermediate="crown"),
    "cnn_chain_over_inner_box": _hybrid_cnn,
    "resnet_windows_two_branches": lambda: wk.resnet(2, 0.004, 82, widths=(32, 64), blocks=(1, 2), n_out=10,
                                                     in_shape=(3, 16, 16)),
    "mlp_unstable_rows": lambda: wk.tiny_mlp([40, 64, 48, 48, 7], 0.07, 61, batch=3),
}
MODES = {"cnn_gather_ibp": "ibp", "cnn_footprint_chain_crown": "crown", "cnn_chain_over_inner_box": "hybrid",
         "resnet_windows_two_branches": "hybrid", "mlp_unstable_rows": "crown+ibp+unstable"}


@pytest.mark.parametrize("name", list(CASES))
def test_crown_bitwise_repeatable(lbp, name):
    wl = CASES[name]()
    mode = MODES[name]
    print(f"{name}: {mode}", flush=True)
    net, x, C = lbp.prepare(wl)
    a = lbp.crown(net, x, float(wl.eps), C, mode, wl.region_start)
    b = lbp.crown(net, x, float(wl.eps), C, mode, wl.region_start)
    torch.cuda.synchronize()
    for key in ("lb", "ub", "ibp_lb", "ibp_ub"):
        assert torch.equal(a[key], b[key]), key
    for k in range(1, len(wl.nodes)):
        if a["lo"][k] is not None:
            assert torch.equal(a["lo"][k], b["lo"][k]) and torch.equal(a["hi"][k], b["hi"][k]), k


@pytest.mark.parametrize("compact", [True, False])
def test_alpha_crown_bitwise_repeatable(lbp, compact):
    wl = wk.cnn(2, 0.02, 31, convs=((8, 1), (16, 2), (16, 1)), fcs=(24, 10), in_shape=(3, 10, 10))
    net, x, C = lbp.prepare(wl)
    out = lbp.crown(net, x, float(wl.eps), C, "ibp")
    runs = []
    for _ in range(2):
        lay = lbp.alpha_layout(net, out["lo"], out["hi"]) if compact else None
        best, lb_steps, state = lbp.alpha_crown(net, x, float(wl.eps), C, out["lo"], out["hi"], 5, 0.1, layout=lay)
        torch.cuda.synchronize()
        slopes = {}
        for k, t in enumerate(state[0]):
            if t is None:
                continue
            if lay is None:
                slopes[k] = t.clone()
            else:
                # compact rows are as wide as the largest count over the batch: an input
                # with fewer unstable neurons leaves the tail of its rows unused
                for b in range(wl.batch):
                    cnt = int((lay.index[k][b] >= 0).sum())
                    slopes[(k, b)] = t[b, :, :cnt].clone()
        runs.append((best.clone(), lb_steps.clone(), slopes))
    (b1, s1, a1), (b2, s2, a2) = runs
    assert torch.equal(b1, b2) and torch.equal(s1, s2)
    assert a1.keys() == a2.keys() and all(torch.equal(a1[k], a2[k]) for k in a1)
