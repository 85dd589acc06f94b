"""Pins of the float64 oracle against exact rational arithmetic and closed forms.

* An independent exact implementation (tests/rational_oracle.py, Python
  Fractions and loops) on 20 random tiny networks (MLP, CNN, residual) in every
  intermediate-bound mode: every node's bounds and the IBP / CROWN spec bounds
  agree with the float64 oracle to 1e-12 relative.
* alpha-CROWN evaluation at random slopes agrees with the exact value.
* The hybrid mode's domain is the IBP box of region_start: on a net whose
  region is one affine layer the spec bound is the exact minimum over the
  vertices of that box, which is built by brute force layer by layer (the
  extremes of one affine map over a box are attained at its vertices).  Other
  boxes (before the ReLU, the CROWN box, the input domain) give other values.
* Multi-step Adam with a constant gradient: the bias-corrected moments are the
  gradient and its square at every step, so each ascent step is
  lr * g / (|g| + eps_hat); through alpha-CROWN on a one-neuron network whose
  bound is linear in its slope, the iterates follow that closed form.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as wk
from workloads import Node
from oracle import Oracle, crown_bounds, intermediate_bounds, adam_ascent_step
from oracle.alpha import alpha_crown, alpha_init, evaluate

import rational_oracle as rq

MODES = ["ibp", "crown", "hybrid", "crown+ibp", "hybrid+ibp", "crown+unstable", "crown+ibp+unstable",
         "hybrid+ibp+unstable"]


def _nets():
    out = []
    for seed, (widths, eps) in enumerate([([3, 5, 4, 3], 0.3), ([4, 6, 6, 5, 3], 0.2), ([2, 4, 4, 2], 0.5),
                                          ([5, 4, 6, 4, 3], 0.15), ([3, 6, 5, 4], 0.25), ([4, 3, 5, 3, 2], 0.4),
                                          ([6, 5, 5, 3], 0.2), ([3, 4, 4, 4, 3], 0.35)]):
        wl = wk.tiny_mlp(widths, eps, 300 + seed, batch=1)
        wl.region_start = 2            # the first ReLU output
        out.append(wl)
    for seed, (convs, in_shape, eps) in enumerate([(((2, 1), (2, 2)), (1, 4, 4), 0.1),
                                                   (((2, 2), (3, 1)), (2, 4, 4), 0.08),
                                                   (((3, 1), (2, 1)), (1, 3, 3), 0.15),
                                                   (((2, 1), (2, 2)), (2, 5, 5), 0.05),
                                                   (((1, 1), (2, 2)), (1, 5, 4), 0.2),
                                                   (((2, 2), (2, 1)), (1, 6, 6), 0.1)]):
        wl = wk.cnn(1, eps, 400 + seed, convs=convs, fcs=(4, 3), in_shape=in_shape, intermediate="crown")
        wl.region_start = 2
        out.append(wl)
    # (seeds chosen so that the exact arithmetic stays small: rational bounds grow in
    # length with every relaxation they pass through)
    for seed, widths, blocks, in_shape, eps in [(501, (2, 3), (1, 1), (1, 4, 4), 0.05),
                                                (507, (2, 2), (1, 1), (1, 4, 4), 0.1),
                                                (500, (1, 2), (1, 1), (2, 4, 4), 0.08),
                                                (517, (2,), (2,), (1, 4, 4), 0.05),
                                                (501, (2, 2), (1, 1), (1, 3, 3), 0.1),
                                                (500, (2,), (1,), (2, 5, 5), 0.04)]:
        out.append(wk.resnet(1, eps, seed, widths=widths, blocks=blocks, n_out=3, in_shape=in_shape))
    return out


NETS = _nets()


def _close(f64, exact_vals, what):
    a = np.asarray(f64, dtype=np.float64).reshape(-1)
    assert a.size == len(exact_vals), what
    worst = 0.0
    for v, q in zip(a.tolist(), exact_vals):
        d = abs(Fraction(v) - q)
        tol = Fraction(1, 10 ** 12) * max(Fraction(1), abs(q))
        assert d <= tol, f"{what}: float64 {v!r} vs exact {float(q)!r}"
        worst = max(worst, float(d / tol))
    return worst


def test_nets_have_unstable_neurons():
    # the pins below would be weak on nets whose every ReLU is stable
    for wl in NETS:
        lo, hi = intermediate_bounds(Oracle(wl.nodes), wl.x0, wl.eps, "ibp")
        zs = [wl.nodes[k].inputs[0] for k, n in enumerate(wl.nodes) if n.op == "relu"]
        assert sum(int(((lo[z] < 0) & (hi[z] > 0)).sum()) for z in zs) >= 2, wl.name


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("i", range(len(NETS)))
def test_float64_oracle_equals_exact_arithmetic(i, mode):
    wl = NETS[i]
    wl.intermediate = mode
    ref = crown_bounds(wl)
    ex = rq.bounds(wl, 0, mode)
    for key in ("ibp_lb", "ibp_ub", "lb", "ub"):
        _close(ref[key][0], ex[key], f"{wl.name} {mode} {key}")
    for k, nd in enumerate(wl.nodes):
        if k == 0:
            continue
        _close(ref["lo"][k][0], ex["lo"][k], f"{wl.name} {mode} lo[{k}]")
        _close(ref["hi"][k][0], ex["hi"][k], f"{wl.name} {mode} hi[{k}]")


@pytest.mark.parametrize("i", [0, 1, 3, 8, 9, 11])
def test_alpha_evaluation_equals_exact_arithmetic(i):
    wl = NETS[i]
    net = Oracle(wl.nodes)
    lo, hi = intermediate_bounds(net, wl.x0, wl.eps, "crown")
    ex = rq.bounds(wl, 0, "crown")
    rng = np.random.default_rng(i)
    al = {k: torch.as_tensor(rng.uniform(0, 1, v.shape)) for k, v in alpha_init(net, lo, hi, 0, wl.m).items()}
    got = evaluate(wl, lo, hi, 0, al)
    want = rq.alpha_lower_bounds(wl, ex["lo"], ex["hi"], 0, {k: v.reshape(v.shape[0], -1).numpy()
                                                             for k, v in al.items()})
    _close(got, want, f"{wl.name} alpha")


# ---------------------------------------------------------------------------
# hybrid: the domain is the IBP box of region_start


def _vertices(lo, hi):
    return np.array(list(itertools.product(*zip(lo, hi))), dtype=np.float64)


def _affine_range(W, b, lo, hi):
    """Exact extremes of W y + b over the box [lo, hi] (brute force over vertices)."""
    v = _vertices(lo, hi) @ W.T.astype(np.float64) + b.astype(np.float64)
    return v.min(0), v.max(0)


def test_hybrid_domain_is_the_ibp_box_of_region_start():
    rng = np.random.default_rng(17)
    n0, n1, n2, n3 = 3, 4, 4, 3
    W1, W2, W3 = (rng.standard_normal((a, b)).astype(np.float32) for a, b in ((n1, n0), (n2, n1), (n3, n2)))
    b1, b2, b3 = (rng.standard_normal(n).astype(np.float32) * np.float32(0.3) for n in (n1, n2, n3))
    nodes = [Node("input", (), (n0,)), Node("linear", (0,), (n1,), W1, b1), Node("relu", (1,), (n1,)),
             Node("linear", (2,), (n2,), W2, b2), Node("relu", (3,), (n2,)), Node("linear", (4,), (n3,), W3, b3)]
    x0 = np.array([[0.2, -0.1, 0.4]], dtype=np.float32)
    eps = np.float32(0.5)
    C = np.array([[[1, -1, 0], [1, 0, -1]]], dtype=np.float32)
    e = float(eps)
    xl, xh = x0[0].astype(np.float64) - e, x0[0].astype(np.float64) + e
    # IBP box of node 4 by brute force, one affine layer at a time
    z1l, z1h = _affine_range(W1, b1, xl, xh)
    r1l, r1h = np.maximum(z1l, 0), np.maximum(z1h, 0)
    z2l, z2h = _affine_range(W2, b2, r1l, r1h)
    r2l, r2h = np.maximum(z2l, 0), np.maximum(z2h, 0)
    spec = lambda lo, hi: _affine_range(C[0].astype(np.float64) @ W3, C[0].astype(np.float64) @ b3, lo, hi)
    want_lb, want_ub = spec(r2l, r2h)
    wl = wk.Workload("hybrid_pin", 0, nodes, x0, eps, np.zeros(1, np.int64), C, "hybrid", region_start=4)
    got = crown_bounds(wl)
    assert got["lb"][0].numpy() == pytest.approx(want_lb, abs=1e-12)
    assert got["ub"][0].numpy() == pytest.approx(want_ub, abs=1e-12)
    # this net tells the IBP box of region_start apart from the other readings
    assert (z2l < 0).any()
    pre_relu = spec(z2l, z2h)[0]
    wl_c = wk.Workload("hybrid_pin", 0, nodes, x0, eps, np.zeros(1, np.int64), C, "crown")
    full_crown = crown_bounds(wl_c)
    crown_box = spec(np.maximum(full_crown["lo"][3][0].numpy(), 0), np.maximum(full_crown["hi"][3][0].numpy(), 0))[0]
    for other in (pre_relu, crown_box, full_crown["lb"][0].numpy()):
        assert np.abs(other - want_lb).max() > 1e-6


# ---------------------------------------------------------------------------
# multi-step Adam


def test_adam_constant_gradient_closed_form():
    lr, eps_hat = 0.1, 1e-8
    g = torch.tensor([0.8, -2.5, 1e-3], dtype=torch.float64)
    x = torch.tensor([0.2, 0.9, 0.5], dtype=torch.float64)
    m = torch.zeros(3, dtype=torch.float64)
    v = torch.zeros(3, dtype=torch.float64)
    for t in range(1, 4):
        x_prev = x
        x, m, v = adam_ascent_step(x, g, m, v, t, lr)
        step = lr * g / (g.abs() + eps_hat)
        assert (x - x_prev).tolist() == pytest.approx(step.tolist(), abs=1e-13), t


def test_alpha_crown_iterates_follow_the_adam_closed_form():
    """One unstable neuron z = 2x - 0.8 on x in [0, 1] feeding y = relu(z) + 0.3: the
    lower bound is alpha * l_z + 0.3 = -0.8 alpha + 0.3, a constant gradient -0.8, so
    alpha_t = max(0, 1 - t * lr * 0.8 / (0.8 + 1e-8)) and lb_t = -0.8 alpha_t + 0.3."""
    nodes = [Node("input", (), (1,)), Node("linear", (0,), (1,), np.array([[2.0]], np.float32),
                                           np.array([-0.8], np.float32)),
             Node("relu", (1,), (1,)), Node("linear", (2,), (1,), np.array([[1.0]], np.float32),
                                            np.array([0.3], np.float32))]
    wl = wk.Workload("adam_pin", 0, nodes, np.array([[0.5]], np.float32), np.float32(0.5), np.zeros(1, np.int64),
                     np.array([[[1.0]]], np.float32), "ibp", alpha_steps=12, alpha_lr=0.1)
    net = Oracle(nodes)
    lo, hi = intermediate_bounds(net, wl.x0, wl.eps, "ibp")
    l_z = float(lo[1][0, 0])
    assert l_z == pytest.approx(-0.8, abs=1e-7) and float(hi[1][0, 0]) > -l_z   # adaptive slope 1
    res = alpha_crown(wl, lo, hi)
    b3 = float(np.float32(0.3))
    delta = 0.1 * abs(l_z) / (abs(l_z) + 1e-8)
    for t in range(13):
        a_t = max(0.0, 1.0 - t * delta)
        assert res["lb_steps"][t, 0, 0].item() == pytest.approx(l_z * a_t + b3, abs=1e-12), t
    assert res["alpha"][0][2].item() == 0.0
    assert res["best"][0, 0].item() == pytest.approx(b3, abs=1e-12)


# ---------------------------------------------------------------------------
# unstable-only rows


def test_unstable_only_nets_mix_stable_and_unstable_neurons():
    # the +unstable modes differ from the full ones only where IBP already settles a
    # neuron of a refined layer: some nets must have both kinds there
    mixed = 0
    for wl in NETS:
        net = Oracle(wl.nodes)
        lo, hi = intermediate_bounds(net, wl.x0, wl.eps, "ibp")
        for r in net.relu_nodes():
            z = wl.nodes[r].inputs[0]
            if z <= 0 or _one_step(net, z):
                continue
            u = ((lo[z] < 0) & (hi[z] > 0)).reshape(-1)
            mixed += int(bool(u.any()) and not bool(u.all()))
    assert mixed >= 3


def _one_step(net, z):
    from oracle.bounds import _one_affine_step
    return _one_affine_step(net, z, 0)


@pytest.mark.parametrize("i", range(len(NETS)))
def test_unstable_only_with_intersection_keeps_every_relaxation(i):
    """With the IBP intersection, a neuron IBP already settles keeps its class under
    CROWN, so every ReLU relaxation is the same with rows for all neurons or for the
    unstable ones only: the spec bounds agree to the last bit, and so do the bounds
    of every neuron IBP leaves unstable."""
    wl = NETS[i]
    wl.intermediate = "crown+ibp"
    full = crown_bounds(wl)
    wl.intermediate = "crown+ibp+unstable"
    part = crown_bounds(wl)
    assert torch.equal(full["lb"], part["lb"]) and torch.equal(full["ub"], part["ub"])
    net = Oracle(wl.nodes)
    lo0, hi0 = intermediate_bounds(net, wl.x0, wl.eps, "ibp")
    for r in net.relu_nodes():
        z = wl.nodes[r].inputs[0]
        u = (lo0[z] < 0) & (hi0[z] > 0)
        assert torch.equal(full["lo"][z][u], part["lo"][z][u]) and torch.equal(full["hi"][z][u], part["hi"][z][u])


# ---------------------------------------------------------------------------
# alpha-CROWN on the identity rows of intermediate layers


@pytest.mark.parametrize("i", [0, 1, 3, 5])
def test_alpha_rows_evaluation_equals_exact_arithmetic(i):
    """The per-row slope evaluation that alpha_rows optimises (identity rows over an
    intermediate node, each row with its own slopes for every ReLU below it) equals
    the exact back-substitution with the same slopes."""
    from oracle.bounds import _domain, _identity_rows, backward
    wl = NETS[i]
    net = Oracle(wl.nodes)
    lo, hi = intermediate_bounds(net, wl.x0, wl.eps, "crown")
    ex = rq.bounds(wl, 0, "crown")
    rng = np.random.default_rng(50 + i)
    checked = 0
    for r in net.relu_nodes():
        z = wl.nodes[r].inputs[0]
        if z <= 0 or _one_step(net, z):
            continue
        shape = net.shape[z]
        n = int(np.prod(shape))
        rows = torch.cat([_identity_rows(shape, 1.0).reshape(n, -1), _identity_rows(shape, -1.0).reshape(n, -1)])
        al = {k: torch.as_tensor(rng.uniform(0, 1, (2 * n,) + net.shape[wl.nodes[k].inputs[0]]))
              for k in net.relu_nodes() if k < z}
        dc, dr = _domain(net, lo, hi, wl.x0, wl.eps, 0, 0)
        got = backward(net, lo, hi, 0, z, rows.reshape((2 * n,) + tuple(shape)), 0, dc, dr, alpha=al)
        want = rq.row_lower_bounds(wl, ex["lo"], ex["hi"], 0, z, rows.numpy(),
                                   {k: v.reshape(2 * n, -1).numpy() for k, v in al.items()})
        _close(got, want, f"{wl.name} alpha rows over node {z}")
        checked += 1
    assert checked >= 1


def test_alpha_rows_are_independent():
    """Each row's slopes follow the gradient of its own bound: optimising two rows
    together gives each the trajectory it has alone."""
    from oracle.alpha import alpha_rows
    from oracle.bounds import _identity_rows
    wl = NETS[1]
    net = Oracle(wl.nodes)
    lo, hi = intermediate_bounds(net, wl.x0, wl.eps, "ibp")
    z = [wl.nodes[r].inputs[0] for r in net.relu_nodes()][-1]
    shape = net.shape[z]
    n = int(np.prod(shape))
    rows = torch.cat([_identity_rows(shape, 1.0).reshape(n, -1), _identity_rows(shape, -1.0).reshape(n, -1)])
    both, _ = alpha_rows(wl, lo, hi, 0, z, rows, 6, 0.1)
    for j in (0, n + 1):
        alone, _ = alpha_rows(wl, lo, hi, 0, z, rows[j:j + 1], 6, 0.1)
        assert torch.allclose(both[:, j], alone[:, 0], rtol=1e-12, atol=1e-12)


def test_alpha_intermediate_bounds_tighter_than_crown_and_below_the_exact_range():
    """alpha-CROWN intermediate bounds start from CROWN (its first iterate) and keep
    the best iterate, so they are at least as tight as CROWN's; and they stay sound:
    inside the exact range of each neuron over the input box, found by linear
    programming per activation pattern on 2-input networks."""
    from oracle.alpha import alpha_intermediate_bounds
    from test_oracle_bab import exact_min
    checked = 0
    for seed in range(4):
        wl = wk.tiny_mlp([2, 5, 5, 4, 2], 0.3, 900 + seed, batch=1)
        net = Oracle(wl.nodes)
        lo_c, hi_c = intermediate_bounds(net, wl.x0, wl.eps, "crown")
        lo_a, hi_a = alpha_intermediate_bounds(wl, 8, 0.1)
        for r in net.relu_nodes():
            z = wl.nodes[r].inputs[0]
            assert bool((lo_a[z] >= lo_c[z] - 1e-12).all()) and bool((hi_a[z] <= hi_c[z] + 1e-12).all())
            if _one_step(net, z):
                continue  # (IBP there: exact)
            # exact range of z_j over the box: the network cut after node z
            cut = wk.Workload(wl.name, wl.cfg, wl.nodes[:z + 1], wl.x0, wl.eps, wl.labels, wl.C, "ibp")
            for j in range(net.shape[z][0]):
                e = np.zeros(net.shape[z][0])
                e[j] = 1.0
                lo_ex = exact_min(cut, 0, e)
                hi_ex = -exact_min(cut, 0, -e)
                assert lo_a[z][0, j].item() <= lo_ex + 1e-9 and hi_a[z][0, j].item() >= hi_ex - 1e-9
                checked += 1
    assert checked > 10
