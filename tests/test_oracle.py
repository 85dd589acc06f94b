"""Pins of the float64 oracle against brute force, closed forms and hand-derived values.

None of these compares the oracle with itself: each expected value comes from
enumeration of box vertices, dense sampling of the network, an independent
dense rewrite of a conv/GAP/residual network, a closed form, finite
differences, or numbers worked out by hand (tests/golden/hand_crown.json).
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import workloads as wk
from workloads import Node, NetBuilder
from oracle import (Oracle, ibp, crown_bounds, intermediate_bounds, spec_bounds_crown,
                    spec_bounds_ibp, relaxation, adam_ascent_step)
from oracle.alpha import alpha_crown, alpha_gradient, alpha_init, compact_columns, evaluate

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _net_from_layers(layers, n_in):
    nodes = [Node("input", (), (n_in,))]
    for i, L in enumerate(layers):
        W = np.asarray(L["W"], dtype=np.float32)
        b = np.asarray(L["b"], dtype=np.float32)
        nodes.append(Node("linear", (len(nodes) - 1,), (W.shape[0],), W, b))
        if i < len(layers) - 1:
            nodes.append(Node("relu", (len(nodes) - 1,), (W.shape[0],)))
    return nodes


def _wl(nodes, x0, eps, C, mode="crown", region_start=None):
    x0 = np.asarray(x0, dtype=np.float32)
    C = np.asarray(C, dtype=np.float32)
    return wk.Workload("t", 0, nodes, x0, np.float32(eps), np.zeros(x0.shape[0], np.int64), C,
                       mode, region_start)


def _vertices(x0, eps):
    n = x0.size
    for signs in itertools.product((-1.0, 1.0), repeat=n):
        yield x0.reshape(-1).astype(np.float64) + eps * np.asarray(signs)


def _spec_values(nodes, C, xs, in_shape):
    out = wk.forward(nodes, xs.reshape((xs.shape[0],) + tuple(in_shape)))[-1]
    return out @ C.astype(np.float64).T


# ---------------------------------------------------------------------------
# hand-derived golden values


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "hand_crown.json")))["cases"],
                         ids=lambda c: c["name"])
def test_hand_derived_examples(case):
    nodes = _net_from_layers(case["layers"], len(case["x0"]))
    x0 = [case["x0"]]
    C = [case["C"]]
    for mode, key in (("crown", "crown_crown"), ("ibp", "crown_ibp")):
        res = crown_bounds(_wl(nodes, x0, case["eps"], C, mode))
        assert res["ibp_lb"][0, 0].item() == pytest.approx(case["ibp"][0], abs=1e-12)
        assert res["ibp_ub"][0, 0].item() == pytest.approx(case["ibp"][1], abs=1e-12)
        assert res["lb"][0, 0].item() == pytest.approx(case[key][0], abs=1e-12)
        assert res["ub"][0, 0].item() == pytest.approx(case[key][1], abs=1e-12)
        if mode == "crown" and "intermediate_crown" in case:
            z = 3   # second linear node
            assert res["lo"][z][0].tolist() == pytest.approx(case["intermediate_crown"]["lo"], abs=1e-12)
            assert res["hi"][z][0].tolist() == pytest.approx(case["intermediate_crown"]["hi"], abs=1e-12)


# ---------------------------------------------------------------------------
# closed forms


def test_single_relu_closed_form():
    # z = x on [x0-eps, x0+eps]; y = relu(z)
    nodes = [Node("input", (), (1,)),
             Node("linear", (0,), (1,), np.array([[1.0]], np.float32), np.array([0.0], np.float32)),
             Node("relu", (1,), (1,)),
             Node("linear", (2,), (1,), np.array([[1.0]], np.float32), np.array([0.0], np.float32))]
    # z in [-1, 3]: s = t = 3/4, a = 1 -> lb = -1, ub = 3 (IBP lb = 0: CROWN >= IBP is not invariant)
    r = crown_bounds(_wl(nodes, [[1.0]], 2.0, [[[1.0]]]))
    assert (r["lb"].item(), r["ub"].item()) == (pytest.approx(-1.0), pytest.approx(3.0))
    assert (r["ibp_lb"].item(), r["ibp_ub"].item()) == (pytest.approx(0.0), pytest.approx(3.0))
    # z in [-3, 1]: a = 0, s = 1/4, t = 3/4 -> lb = 0, ub = max(z/4 + 3/4) = 1
    r = crown_bounds(_wl(nodes, [[-1.0]], 2.0, [[[1.0]]]))
    assert (r["lb"].item(), r["ub"].item()) == (pytest.approx(0.0), pytest.approx(1.0))
    # inactive and active neurons
    r = crown_bounds(_wl(nodes, [[-3.0]], 1.0, [[[1.0]]]))
    assert (r["lb"].item(), r["ub"].item()) == (0.0, 0.0)
    r = crown_bounds(_wl(nodes, [[3.0]], 1.0, [[[1.0]]]))
    assert (r["lb"].item(), r["ub"].item()) == (pytest.approx(2.0), pytest.approx(4.0))


def test_tie_decision_alignment_closed_form():
    """At the adaptive-slope tie u = -l both lower slopes are sound: with z on [-1, 1]
    the lower bound of relu(z) is min(a z) = -1 for a = 1 (the oracle's own choice) and
    0 for a = 0.  `decide` takes another implementation's choice there, and only at
    near-ties: on [-1, 3] the slope stays 1 whatever `decide` says."""
    import torch
    nodes = [Node("input", (), (1,)),
             Node("linear", (0,), (1,), np.array([[1.0]], np.float32), np.array([0.0], np.float32)),
             Node("relu", (1,), (1,)),
             Node("linear", (2,), (1,), np.array([[1.0]], np.float32), np.array([0.0], np.float32))]
    wl = _wl(nodes, [[0.0]], 1.0, [[[1.0]]])
    assert crown_bounds(wl)["lb"].item() == pytest.approx(-1.0)
    assert crown_bounds(wl, decide={1: torch.tensor([[True]])})["lb"].item() == pytest.approx(-1.0)
    assert crown_bounds(wl, decide={1: torch.tensor([[False]])})["lb"].item() == pytest.approx(0.0)
    wl = _wl(nodes, [[1.0]], 2.0, [[[1.0]]])
    assert crown_bounds(wl, decide={1: torch.tensor([[False]])})["lb"].item() == pytest.approx(-1.0)


def test_relaxation_cases():
    l = torch.tensor([-2.0, 0.0, 1.0, -1.0, -3.0, 0.0, -2.0], dtype=torch.float64)
    u = torch.tensor([-1.0, 2.0, 2.0, 3.0, 1.0, 0.0, 2.0], dtype=torch.float64)
    a, s, t, unst = relaxation(l, u)
    assert a.tolist() == [0, 1, 1, 1, 0, 0, 1]
    assert s.tolist() == pytest.approx([0, 1, 1, 0.75, 0.25, 0, 0.5])
    assert t.tolist() == pytest.approx([0, 0, 0, 0.75, 0.75, 0, 1.0])
    assert unst.tolist() == [False, False, False, True, True, False, True]
    # the upper line passes through (l, 0) and (u, u); the lower line is under relu
    for i in range(len(l)):
        if unst[i]:
            assert s[i] * l[i] + t[i] == pytest.approx(0.0)
            assert s[i] * u[i] + t[i] == pytest.approx(u[i].item())


# ---------------------------------------------------------------------------
# brute force


@pytest.mark.parametrize("seed", range(4))
def test_single_affine_layer_is_exact(seed):
    rng = np.random.default_rng(seed)
    n, m = 9, 4
    W = rng.standard_normal((m, n)).astype(np.float32)
    b = rng.standard_normal(m).astype(np.float32)
    nodes = [Node("input", (), (n,)), Node("linear", (0,), (m,), W, b)]
    x0 = rng.random((1, n)).astype(np.float32)
    C = rng.standard_normal((1, 3, m)).astype(np.float32)
    eps = np.float32(0.3)
    res = crown_bounds(_wl(nodes, x0, eps, C))
    vals = _spec_values(nodes, C[0], np.stack(list(_vertices(x0[0], float(eps)))), (n,))
    for key_lb, key_ub in (("ibp_lb", "ibp_ub"), ("lb", "ub")):
        assert np.allclose(res[key_lb][0].numpy(), vals.min(0), atol=1e-12, rtol=1e-12)
        assert np.allclose(res[key_ub][0].numpy(), vals.max(0), atol=1e-12, rtol=1e-12)
    # node bounds of the affine layer itself are the vertex extremes too
    z = wk.forward(nodes, np.stack(list(_vertices(x0[0], float(eps)))))[1]
    assert np.allclose(res["ibp_lo"][1][0].numpy(), z.min(0), atol=1e-12)
    assert np.allclose(res["ibp_hi"][1][0].numpy(), z.max(0), atol=1e-12)


def test_eps_zero_gives_the_forward_value():
    for wl in (wk.tiny_mlp([6, 7, 5, 4], 0.0, 1, batch=2),
               wk.cnn(2, 0.0, 77, convs=((4, 1), (5, 2)), fcs=(6, 3), in_shape=(2, 6, 6), intermediate="crown"),
               wk.resnet(1, 0.0, 78, widths=(3, 4), blocks=(1, 1), n_out=3, in_shape=(2, 6, 6))):
        f = wk.forward(wl.nodes, wl.x0)[-1]
        ref = np.einsum("bmn,bn->bm", wl.C.astype(np.float64), f)
        res = crown_bounds(wl)
        for k in ("lb", "ub", "ibp_lb", "ibp_ub"):
            assert np.allclose(res[k].numpy(), ref, atol=1e-10), k


@pytest.mark.parametrize("seed", range(3))
def test_all_stable_crown_is_exact(seed):
    # tiny eps: every ReLU is stable, the net is affine on the box, so the true
    # extremes are attained at box vertices and CROWN must reach them.
    wl = wk.tiny_mlp([8, 10, 9, 5], 1e-4, seed)
    res = crown_bounds(wl)
    net = Oracle(wl.nodes)
    for r in net.relu_nodes():
        z = wl.nodes[r].inputs[0]
        assert bool(((res["lo"][z] >= 0) | (res["hi"][z] <= 0)).all())
    vals = _spec_values(wl.nodes, wl.C[0], np.stack(list(_vertices(wl.x0[0], float(wl.eps)))), (8,))
    assert np.allclose(res["lb"][0].numpy(), vals.min(0), atol=1e-10)
    assert np.allclose(res["ub"][0].numpy(), vals.max(0), atol=1e-10)


def _sample_ball(x0, eps, n, rng):
    d = x0.size
    pts = x0.reshape(1, -1).astype(np.float64) + eps * rng.uniform(-1, 1, (n, d))
    corners = x0.reshape(1, -1).astype(np.float64) + eps * rng.choice([-1.0, 1.0], (n // 10, d))
    return np.concatenate([pts, corners])


def _check_sound(wl, res, n=100000, seed=0):
    rng = np.random.default_rng(seed)
    in_shape = wl.nodes[0].shape
    for b in range(wl.batch):
        xs = _sample_ball(wl.x0[b], float(wl.eps), n, rng)
        vals = wk.forward(wl.nodes, xs.reshape((-1,) + tuple(in_shape)))
        spec = vals[-1] @ wl.C[b].astype(np.float64).T
        for lbk, ubk in (("lb", "ub"), ("ibp_lb", "ibp_ub")):
            lb = res[lbk][b].numpy()
            ub = res[ubk][b].numpy()
            assert (spec >= lb - 1e-9 * (1 + abs(lb))).all(), lbk
            assert (spec <= ub + 1e-9 * (1 + abs(ub))).all(), ubk
            assert (lb <= ub + 1e-12).all()
        for k, nd in enumerate(wl.nodes):
            if nd.op in ("linear", "conv", "add"):
                v = vals[k].reshape(vals[k].shape[0], -1)
                lo = res["lo"][k][b].reshape(-1).numpy()
                hi = res["hi"][k][b].reshape(-1).numpy()
                assert (v >= lo - 1e-9 * (1 + abs(lo))).all()
                assert (v <= hi + 1e-9 * (1 + abs(hi))).all()


@pytest.mark.parametrize("mode", ["crown", "ibp", "crown+ibp"])
def test_soundness_mlp_sampling(mode):
    for seed, widths, eps in ((0, [4, 8, 8, 3], 0.3), (1, [6, 12, 10, 7, 4], 0.15), (2, [3, 5, 5, 5, 2], 0.5)):
        wl = wk.tiny_mlp(widths, eps, seed, batch=2)
        wl.intermediate = mode
        _check_sound(wl, crown_bounds(wl), n=20000, seed=seed)


def test_soundness_cnn_and_resnet_sampling():
    wl = wk.cnn(2, 0.05, 91, convs=((3, 1), (4, 2)), fcs=(6, 4), in_shape=(2, 4, 4), intermediate="crown")
    _check_sound(wl, crown_bounds(wl), n=20000)
    wl.intermediate = "ibp"
    _check_sound(wl, crown_bounds(wl), n=20000)
    wl = wk.resnet(2, 0.05, 92, widths=(2, 3), blocks=(1, 2), n_out=3, in_shape=(2, 4, 4))
    _check_sound(wl, crown_bounds(wl), n=20000)


def test_intersection_mode_is_sound_and_inside_both():
    """CROWN intermediates intersected with IBP: sound on samples; every node's box lies
    inside its IBP box and inside the pure-CROWN box at the first refined layer (whose
    relaxations come from IBP bounds in both modes); strictly tighter than pure CROWN
    somewhere.  (The exact values of this mode are pinned by exact rational
    arithmetic in test_oracle_exact.py.)"""
    for seed, widths, eps in ((3, [5, 9, 9, 8, 3], 0.3), (4, [6, 12, 10, 7, 4], 0.2)):
        wl = wk.tiny_mlp(widths, eps, seed, batch=2)
        net = Oracle(wl.nodes)
        lo_i, hi_i = intermediate_bounds(net, wl.x0, wl.eps, "ibp")
        lo_c, hi_c = intermediate_bounds(net, wl.x0, wl.eps, "crown")
        lo_x, hi_x = intermediate_bounds(net, wl.x0, wl.eps, "crown+ibp")
        zs = [nd.inputs[0] for nd in wl.nodes if nd.op == "relu"]
        for z in zs:
            assert bool((lo_x[z] >= lo_i[z] - 1e-12).all() and (hi_x[z] <= hi_i[z] + 1e-12).all())
        first = zs[1]          # zs[0] is one affine step from the input: IBP = CROWN there
        assert bool((lo_x[first] >= lo_c[first] - 1e-12).all() and (hi_x[first] <= hi_c[first] + 1e-12).all())
        # the intersection is strictly tighter than pure CROWN somewhere in these nets
        assert any(bool((hi_x[z] < hi_c[z] - 1e-9).any() or (lo_x[z] > lo_c[z] + 1e-9).any()) for z in zs)
        wl.intermediate = "crown+ibp"
        _check_sound(wl, crown_bounds(wl), n=20000, seed=seed)
    wl = wk.cnn(2, 0.05, 93, convs=((3, 1), (4, 2)), fcs=(6, 4), in_shape=(2, 4, 4), intermediate="crown+ibp")
    _check_sound(wl, crown_bounds(wl), n=20000)


def test_ibp_monotone_in_eps():
    wl = wk.tiny_mlp([10, 12, 12, 4], 0.05, 5, batch=3)
    net = Oracle(wl.nodes)
    lo1, hi1 = ibp(net, wl.x0, 0.05)
    lo2, hi2 = ibp(net, wl.x0, 0.1)
    for a, b in zip(lo1, lo2):
        assert bool((b <= a + 1e-15).all())
    for a, b in zip(hi1, hi2):
        assert bool((b >= a - 1e-15).all())


# ---------------------------------------------------------------------------
# structural equivalences (independent dense rewrites)


def _toeplitz(w, stride, pad, in_shape):
    """Dense matrix of a cross-correlation with zero padding, from the definition."""
    ci, h, wd = in_shape
    co, _, kh, kw = w.shape
    ho = (h + 2 * pad - kh) // stride + 1
    wo = (wd + 2 * pad - kw) // stride + 1
    M = np.zeros((co * ho * wo, ci * h * wd))
    for o in range(co):
        for y in range(ho):
            for x in range(wo):
                row = (o * ho + y) * wo + x
                for i in range(ci):
                    for ky in range(kh):
                        for kx in range(kw):
                            iy, ix = y * stride + ky - pad, x * stride + kx - pad
                            if 0 <= iy < h and 0 <= ix < wd:
                                M[row, (i * h + iy) * wd + ix] += w[o, i, ky, kx]
    return M, (co, ho, wo)


def _densify(nodes):
    """Same network with every conv / GAP replaced by a Linear on flattened
    (C, H, W)-order tensors and every flatten removed (it is the identity there).
    Returns the dense node list and the map old index -> new index."""
    alias = {}
    for k, nd in enumerate(nodes):
        if nd.op == "flatten":
            alias[k] = alias.get(nd.inputs[0], nd.inputs[0])
    keep = [k for k, nd in enumerate(nodes) if nd.op != "flatten"]
    newidx = {k: i for i, k in enumerate(keep)}
    res = []
    for k in keep:
        nd = nodes[k]
        ins = tuple(newidx[alias.get(i, i)] for i in nd.inputs)
        if nd.op == "conv":
            M, shp = _toeplitz(nd.weight.astype(np.float64), nd.stride, nd.pad, nodes[nd.inputs[0]].shape)
            bias = np.repeat(nd.bias.astype(np.float64), shp[1] * shp[2])
            res.append(Node("linear", ins, (M.shape[0],), M, bias))
        elif nd.op == "gap":
            c, h, w = nodes[nd.inputs[0]].shape
            M = np.zeros((c, c * h * w))
            for i in range(c):
                M[i, i * h * w:(i + 1) * h * w] = 1.0 / (h * w)
            res.append(Node("linear", ins, (c,), M, np.zeros(c)))
        else:
            res.append(Node(nd.op, ins, (nd.size,), nd.weight, nd.bias))
    return res, newidx


def _compare_dense(wl, modes=("crown", "ibp")):
    dense, newidx = _densify(wl.nodes)
    x0d = wl.x0.reshape(wl.batch, -1)
    for mode in modes:
        wl.intermediate = mode
        ref = crown_bounds(wl)
        rs = newidx[wl.region_start] if wl.region_start is not None else None
        wd = wk.Workload("d", 0, dense, x0d, wl.eps, wl.labels, wl.C, mode, rs)
        got = crown_bounds(wd)
        for key in ("lb", "ub", "ibp_lb", "ibp_ub"):
            assert np.allclose(ref[key].numpy(), got[key].numpy(), atol=1e-10, rtol=1e-10), (mode, key)
        for k, i in newidx.items():
            a = ref["lo"][k].reshape(wl.batch, -1).numpy()
            b = got["lo"][i].reshape(wl.batch, -1).numpy()
            assert np.allclose(a, b, atol=1e-10, rtol=1e-10), (mode, k)


def test_conv_equals_toeplitz_linear():
    wl = wk.cnn(2, 0.05, 93, convs=((3, 1), (4, 2), (3, 2)), fcs=(5, 4), in_shape=(2, 6, 6))
    _compare_dense(wl)


def test_gap_and_residual_equal_dense_rewrite():
    wl = wk.resnet(2, 0.03, 94, widths=(2, 3), blocks=(2, 1), n_out=3, in_shape=(2, 4, 4))
    _compare_dense(wl, modes=("crown", "ibp", "hybrid"))


def test_residual_zero_branch_is_the_skip():
    full = wk.resnet(2, 0.02, 95, widths=(3, 4), blocks=(2, 1), n_out=4, in_shape=(2, 6, 6),
                     zero_branch_block=1)
    # block 1 (conv_a, relu, conv_b, add, relu) is nodes 8..12 and reads node 7;
    # without it, node 13 onwards reads node 7 directly
    nodes = full.nodes
    assert [nodes[k].op for k in range(8, 13)] == ["conv", "relu", "conv", "add", "relu"]
    assert float(np.abs(nodes[8].weight).max()) == 0.0 and nodes[11].inputs == (10, 7)
    drop = set(range(8, 13))
    keep = [k for k in range(len(nodes)) if k not in drop]
    newidx = {k: i for i, k in enumerate(keep)}
    remap = lambda i: newidx[7] if i == 12 else newidx[i]
    short = [Node(nodes[k].op, tuple(remap(i) for i in nodes[k].inputs), nodes[k].shape,
                  nodes[k].weight, nodes[k].bias, nodes[k].stride, nodes[k].pad) for k in keep]
    # Pure CROWN intermediate bounds (not intersected with IBP) do not know that a
    # ReLU output is >= 0, so relu(x + 0) gets relaxed again there; the identity
    # holds when the block's bounds come from IBP (IBP mode, or hybrid mode with
    # the block before the CROWN region).
    for mode in ("ibp", "hybrid"):
        full.intermediate = mode
        a = crown_bounds(full)
        rs = None if full.region_start is None else remap(full.region_start)
        b = crown_bounds(wk.Workload("s", 0, short, full.x0, full.eps, full.labels, full.C, mode, rs))
        for key in ("lb", "ub", "ibp_lb", "ibp_ub"):
            assert np.allclose(a[key].numpy(), b[key].numpy(), atol=1e-12), (mode, key)


# ---------------------------------------------------------------------------
# alpha-CROWN


def _alpha_wl():
    wl = wk.tiny_mlp([5, 9, 8, 4], 0.25, 11, batch=2)
    wl.alpha_steps = 6
    return wl


def test_alpha_init_reproduces_crown():
    wl = _alpha_wl()
    lo, hi = intermediate_bounds(Oracle(wl.nodes), wl.x0, wl.eps, "crown")
    ref_lb, _ = spec_bounds_crown(Oracle(wl.nodes), lo, hi, wl.x0, wl.eps, wl.C)
    net = Oracle(wl.nodes)
    for b in range(wl.batch):
        al = alpha_init(net, lo, hi, b, wl.m)
        assert torch.equal(evaluate(wl, lo, hi, b, al), ref_lb[b])


def test_alpha_gradient_matches_finite_differences():
    wl = _alpha_wl()
    net = Oracle(wl.nodes)
    lo, hi = intermediate_bounds(net, wl.x0, wl.eps, "crown")
    rng = np.random.default_rng(3)
    for b in range(wl.batch):
        al = {k: torch.as_tensor(rng.uniform(0.1, 0.9, v.shape)) for k, v in alpha_init(net, lo, hi, b, wl.m).items()}
        _, g = alpha_gradient(wl, lo, hi, b, al)
        checked = 0
        for k, v in al.items():
            z = wl.nodes[k].inputs[0]
            unstable = ((lo[z][b] < 0) & (hi[z][b] > 0)).expand_as(v)
            for idx in zip(*np.nonzero(unstable.numpy())):
                h = 1e-6
                ap = {kk: vv.clone() for kk, vv in al.items()}
                am = {kk: vv.clone() for kk, vv in al.items()}
                ap[k][idx] += h
                am[k][idx] -= h
                fd = (evaluate(wl, lo, hi, b, ap).sum() - evaluate(wl, lo, hi, b, am).sum()) / (2 * h)
                assert g[k][idx].item() == pytest.approx(fd.item(), abs=1e-7, rel=1e-6)
                checked += 1
            # stable neurons get no gradient
            assert bool((g[k][~unstable] == 0).all())
        assert checked > 0


def test_adam_first_step_moves_by_lr_times_sign():
    # bias correction makes the first step lr * g / (|g| + eps') with eps' = eps / sqrt(1-b2)... ~ lr * sign(g)
    x = torch.tensor([0.5, 0.5, 0.5, 0.5], dtype=torch.float64)
    g = torch.tensor([2.0, -3.0, 1e-3, 0.0], dtype=torch.float64)
    x1, m, v = adam_ascent_step(x, g, torch.zeros(4, dtype=torch.float64), torch.zeros(4, dtype=torch.float64), 1, 0.1)
    assert x1.tolist() == pytest.approx([0.6, 0.4, 0.6, 0.5], abs=1e-6)
    # clipping to [0, 1]
    x2, _, _ = adam_ascent_step(torch.tensor([0.95, 0.05], dtype=torch.float64), torch.tensor([1.0, -1.0], dtype=torch.float64),
                                torch.zeros(2, dtype=torch.float64), torch.zeros(2, dtype=torch.float64), 1, 0.1)
    assert x2.tolist() == [1.0, 0.0]


def test_alpha_crown_improves_and_stays_sound():
    wl = _alpha_wl()
    net = Oracle(wl.nodes)
    lo, hi = intermediate_bounds(net, wl.x0, wl.eps, "crown")
    ref_lb, _ = spec_bounds_crown(net, lo, hi, wl.x0, wl.eps, wl.C)
    res = alpha_crown(wl, lo, hi)
    assert torch.equal(res["lb_steps"][0], ref_lb)
    assert bool((res["best"] >= ref_lb).all())
    assert bool((res["best"] > ref_lb + 1e-6).any())
    rng = np.random.default_rng(0)
    for b in range(wl.batch):
        xs = _sample_ball(wl.x0[b], float(wl.eps), 50000, rng)
        spec = wk.forward(wl.nodes, xs)[-1] @ wl.C[b].astype(np.float64).T
        for t in range(res["lb_steps"].shape[0]):
            assert (spec >= res["lb_steps"][t, b].numpy() - 1e-9).all()
        for v in res["alpha"][b].values():
            assert bool(((v >= 0) & (v <= 1)).all())


def test_compact_columns_hand_example():
    # input 0: only neuron 0 is unstable (l = 0 is active, u = -1 and u = 0 are inactive);
    # input 1: neurons 1 and 3
    lo = [[-1.0, 0.0, -2.0, 1.0, -5.0], [0.5, -0.1, -3.0, -1.0, -2.0]]
    hi = [[1.0, 1.0, -1.0, 2.0, 0.0], [1.0, 0.2, 0.0, 2.0, -1.0]]
    col, width = compact_columns(lo, hi)
    assert col.tolist() == [[0, -1, -1, -1, -1], [-1, 0, -1, 1, -1]]
    assert width == 2
    col, width = compact_columns([[1.0, 2.0]], [[3.0, 4.0]])
    assert col.tolist() == [[-1, -1]] and width == 0


def test_compact_columns_are_a_dense_ordered_numbering():
    rng = np.random.default_rng(5)
    vals = np.array([-2.0, -1.0, 0.0, 1.0, 2.0])
    lo = rng.choice(vals, size=(6, 40))
    hi = lo + rng.choice(vals[2:], size=(6, 40))   # hi >= lo, ties at zero included
    col, width = compact_columns(lo, hi)
    counts = []
    for b in range(lo.shape[0]):
        unstable = [j for j in range(lo.shape[1]) if lo[b, j] < 0 < hi[b, j]]
        assert [int(col[b, j]) for j in unstable] == list(range(len(unstable)))
        assert all(col[b, j] == -1 for j in range(lo.shape[1]) if j not in unstable)
        counts.append(len(unstable))
    assert width == max(counts)


def test_slopes_of_stable_neurons_do_not_matter():
    """What compact alpha storage relies on: a slope only enters the bound through an
    unstable neuron, so changing it anywhere else leaves the bound bit-identical."""
    wl = _alpha_wl()
    net = Oracle(wl.nodes)
    lo, hi = intermediate_bounds(net, wl.x0, wl.eps, "crown")
    rng = np.random.default_rng(3)
    for b in range(wl.batch):
        al = {k: torch.as_tensor(rng.uniform(0.1, 0.9, v.shape)) for k, v in alpha_init(net, lo, hi, b, wl.m).items()}
        ref = evaluate(wl, lo, hi, b, al)
        moved = {}
        n_stable = 0
        for k, v in al.items():
            z = wl.nodes[k].inputs[0]
            stable = ~((lo[z][b] < 0) & (hi[z][b] > 0))
            n_stable += int(stable.sum())
            moved[k] = torch.where(stable.unsqueeze(0).expand_as(v), torch.as_tensor(rng.uniform(0, 1, v.shape)), v)
        assert n_stable > 0
        assert torch.equal(evaluate(wl, lo, hi, b, moved), ref)
