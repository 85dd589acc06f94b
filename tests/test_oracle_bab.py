"""Pins of the beta-CROWN / branch-and-bound oracle (oracle/bab.py).

* With no split and beta = 0 the sub-domain bound is the CROWN bound; with splits
  and beta = 0 it is CROWN over the clamped bounds (computed independently by
  the plain back-substitution).
* The gradient of the bound with respect to beta (and alpha) matches central
  finite differences.
* Exact minima by linear programming: on tiny 2-input ReLU networks every
  activation pattern is a polyhedron of the input box, on which the network is
  affine; the minimum of the margin over the box (or over a sub-domain, whose
  split constraints select the patterns) is the least LP optimum over the
  patterns.  Every bound the search computes lies below the exact minimum of its
  sub-domain, and the search proves exactly the inputs whose minimum is
  positive (the cases are chosen with a clear margin either way).
"""
import itertools

import numpy as np
import pytest
import torch
from scipy.optimize import linprog

import workloads as wk
from oracle import Oracle, intermediate_bounds, spec_bounds_crown
from oracle.bab import bab, beta_crown, clamp_bounds
from oracle.bounds import backward, _domain


def _tiny(seed, widths=(2, 5, 5, 2), eps=0.3):
    wl = wk.tiny_mlp(list(widths), eps, 700 + seed, batch=1)
    return wl


def _affine_layers(wl):
    Ws = [n.weight.astype(np.float64) for n in wl.nodes if n.op == "linear"]
    bs = [n.bias.astype(np.float64) for n in wl.nodes if n.op == "linear"]
    return Ws, bs


def exact_min(wl, b, c_row, splits=None):
    """min over the input box of c_row . f(x), restricted to a sub-domain: splits
    {layer index: sign array} for the hidden layers (by LP per activation pattern)."""
    Ws, bs = _affine_layers(wl)
    x0 = wl.x0[b].astype(np.float64)
    e = float(np.float32(wl.eps))
    n_hidden = [W.shape[0] for W in Ws[:-1]]
    best = np.inf
    for pattern in itertools.product(*[itertools.product((0, 1), repeat=h) for h in n_hidden]):
        # affine maps of every pre-activation in x: z_l = A_l x + c_l
        A = np.eye(len(x0))
        c = np.zeros(len(x0))
        A_ub, b_ub, ok = [], [], True
        for li, (W, bb) in enumerate(zip(Ws[:-1], bs[:-1])):
            Az, cz = W @ A, W @ c + bb
            act = np.array(pattern[li], dtype=float)
            sg = None if splits is None else splits.get(li)
            for j in range(len(act)):
                if sg is not None and sg[j] != 0 and (sg[j] > 0) != (act[j] > 0):
                    ok = False
                # active: z >= 0  ->  -Az x <= cz ; inactive: z <= 0  ->  Az x <= -cz
                if act[j] > 0:
                    A_ub.append(-Az[j]); b_ub.append(cz[j])
                else:
                    A_ub.append(Az[j]); b_ub.append(-cz[j])
            A, c = act[:, None] * Az, act * cz
        if not ok:
            continue
        obj_A = c_row @ (Ws[-1] @ A)
        obj_c = c_row @ (Ws[-1] @ c + bs[-1])
        res = linprog(obj_A, A_ub=np.array(A_ub), b_ub=np.array(b_ub),
                      bounds=list(zip(x0 - e, x0 + e)), method="highs")
        if res.status == 0:
            best = min(best, res.fun + obj_c)
    return best


def test_no_split_and_zero_beta_is_crown():
    wl = _tiny(1)
    net = Oracle(wl.nodes)
    lo, hi = intermediate_bounds(net, wl.x0, wl.eps, "crown")
    ref, _ = spec_bounds_crown(net, lo, hi, wl.x0, wl.eps, wl.C)
    lo_b, hi_b = clamp_bounds(lo, hi, 0, {}, net)
    out, best, _ = beta_crown(wl, lo_b, hi_b, wl.x0[0], {}, wl.C[0], 0, 0.1)
    assert torch.equal(out[0], ref[0])


def test_splits_clamp_bounds_and_zero_beta_is_crown_over_them():
    wl = _tiny(2)
    net = Oracle(wl.nodes)
    lo, hi = intermediate_bounds(net, wl.x0, wl.eps, "crown")
    r = net.relu_nodes()[0]
    z = wl.nodes[r].inputs[0]
    unst = torch.nonzero((lo[z][0] < 0) & (hi[z][0] > 0)).reshape(-1)
    assert len(unst) >= 2
    sg = torch.zeros(net.shape[z], dtype=torch.float64)
    sg[unst[0]] = 1.0
    sg[unst[1]] = -1.0
    lo_b, hi_b = clamp_bounds(lo, hi, 0, {r: sg}, net)
    assert lo_b[z][0, unst[0]] == 0.0 and hi_b[z][0, unst[1]] == 0.0
    assert hi_b[z][0, unst[0]] == hi[z][0, unst[0]] and lo_b[z][0, unst[1]] == lo[z][0, unst[1]]
    out, _, _ = beta_crown(wl, lo_b, hi_b, wl.x0[0], {r: sg}, wl.C[0], 0, 0.1)
    dc, dr = _domain(net, lo_b, hi_b, torch.as_tensor(wl.x0[:1], dtype=torch.float64), wl.eps, 0, 0)
    plain = backward(net, lo_b, hi_b, 0, len(wl.nodes) - 1, torch.as_tensor(wl.C[0], dtype=torch.float64), 0, dc, dr)
    assert torch.equal(out[0], plain)


def test_beta_gradient_matches_finite_differences():
    wl = _tiny(3, widths=(3, 6, 5, 3))
    net = Oracle(wl.nodes)
    lo, hi = intermediate_bounds(net, wl.x0, wl.eps, "crown")
    r1, r2 = net.relu_nodes()
    splits = {}
    for r in (r1, r2):
        z = wl.nodes[r].inputs[0]
        unst = torch.nonzero((lo[z][0] < 0) & (hi[z][0] > 0)).reshape(-1)
        sg = torch.zeros(net.shape[z], dtype=torch.float64)
        sg[unst[:2]] = torch.tensor([1.0, -1.0], dtype=torch.float64)[: len(unst[:2])]
        splits[r] = sg
    lo_b, hi_b = clamp_bounds(lo, hi, 0, splits, net)
    dc, dr = _domain(net, lo_b, hi_b, torch.as_tensor(wl.x0[:1], dtype=torch.float64), wl.eps, 0, 0)
    C = torch.as_tensor(wl.C[0], dtype=torch.float64)
    L = len(wl.nodes) - 1
    rng = np.random.default_rng(4)
    be = {r: torch.as_tensor(rng.uniform(0.1, 1.0, (C.shape[0],) + tuple(s.shape))) for r, s in splits.items()}
    leaf = {k: v.clone().requires_grad_(True) for k, v in be.items()}
    backward(net, lo_b, hi_b, 0, L, C, 0, dc, dr, beta=leaf, splits=splits).sum().backward()
    checked = 0
    for r, s in splits.items():
        for idx in zip(*np.nonzero(s.numpy())):
            for row in range(C.shape[0]):
                h = 1e-6
                bp = {k: v.clone() for k, v in be.items()}
                bm = {k: v.clone() for k, v in be.items()}
                bp[r][(row,) + idx] += h
                bm[r][(row,) + idx] -= h
                fp = backward(net, lo_b, hi_b, 0, L, C, 0, dc, dr, beta=bp, splits=splits).sum()
                fm = backward(net, lo_b, hi_b, 0, L, C, 0, dc, dr, beta=bm, splits=splits).sum()
                assert leaf[r].grad[(row,) + idx].item() == pytest.approx(((fp - fm) / (2 * h)).item(),
                                                                          abs=1e-7, rel=1e-6)
                checked += 1
        # neurons without a split constraint get no gradient
        assert bool((leaf[r].grad[:, s == 0] == 0).all())
    assert checked > 0


def _cases():
    """Tiny 2-input nets (2 hidden layers of 5) with one margin spec and the exact
    minimum of the margin over the input box, keeping clear-cut cases."""
    out = []
    for seed in range(40):
        wl = _tiny(seed)
        m = exact_min(wl, 0, wl.C[0, 0].astype(np.float64))
        wl.C = wl.C[:, :1]
        if abs(m) > 0.05:
            out.append((wl, m))
    return out


CASES = _cases()


def test_cases_cover_both_outcomes():
    pos = sum(m > 0 for _, m in CASES)
    assert pos >= 3 and len(CASES) - pos >= 3


@pytest.mark.parametrize("i", range(min(12, len(CASES))))
def test_bab_verdict_equals_the_exact_minimum_and_bounds_are_sound(i):
    wl, m = CASES[i]
    net = Oracle(wl.nodes)
    lo, hi = intermediate_bounds(net, wl.x0, wl.eps, "crown")
    res = bab(wl, 0, lo, hi, steps=30, lr=0.1, batch=4, max_domains=600)
    assert res["verdict"] == ("verified" if m > 0 else "undecided"), (m, res["verdict"], res["domains"])
    # every processed sub-domain's bound is below the exact minimum over that sub-domain
    relus = net.relu_nodes()
    for rec in res["record"][:40]:
        splits = {relus.index(r): s.numpy() for r, s in rec["splits"].items()}
        em = exact_min(wl, 0, wl.C[0, 0].astype(np.float64), splits)
        assert rec["lb"][0].item() <= em + 1e-9
