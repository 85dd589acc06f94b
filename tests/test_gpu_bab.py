"""GPU parity of beta-CROWN (split constraints with Lagrange multipliers) and of
branch and bound, against the float64 oracle (oracle/bab.py) and exact minima.

* Sub-domains with split constraints on both hidden layers of an MLP, bounded
  together as one batch: every alpha-beta Adam step's spec lower bounds equal the
  oracle's trajectory.
* Branch and bound (vb_bab) on tiny two-input networks proves exactly the inputs
  whose exact minimum (linear programming per activation pattern) is positive.
* On the 784-100-100-10 workload, an input alpha-CROWN does not prove is proved
  by branch and bound, with the oracle's verdict and number of sub-domains, and
  an input the oracle leaves undecided within the budget is left undecided.
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads as wk
from helpers import assert_close, ensure_built
from oracle import Oracle, ibp as oracle_ibp, intermediate_bounds
from oracle.bab import bab as oracle_bab, beta_crown, clamp_bounds

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lbp():
    ensure_built()
    import linear_bound_propagation_amd as m
    return m


def test_beta_steps_match_the_oracle(lbp):
    wl = wk.tiny_mlp([20, 30, 30, 5], 0.12, 51, batch=1)
    steps, lr = 8, 0.1
    onet = Oracle(wl.nodes)
    lo, hi = oracle_ibp(onet, wl.x0, wl.eps)
    relus = onet.relu_nodes()
    rng = np.random.default_rng(52)
    domains = []
    for d in range(4):
        sp = {}
        for r in relus:
            z = wl.nodes[r].inputs[0]
            unst = np.nonzero(((lo[z][0] < 0) & (hi[z][0] > 0)).numpy())[0]
            pick = rng.choice(unst, min(len(unst), 1 + d % 3), replace=False)
            s = torch.zeros(wl.nodes[z].shape, dtype=torch.float64)
            s[torch.as_tensor(pick)] = torch.as_tensor(rng.choice([-1.0, 1.0], len(pick)))
            sp[r] = s
        domains.append(sp)
    D, m = len(domains), wl.m
    net, x, C = lbp.prepare(wl)
    lo1, hi1, _, _ = lbp.ibp(net, x, float(wl.eps))
    xd = x.repeat(D, 1)
    Cd = C.repeat(D, 1, 1).contiguous()
    dlo = [None] + [t.repeat(D, 1).contiguous() for t in lo1[1:]]
    dhi = [None] + [t.repeat(D, 1).contiguous() for t in hi1[1:]]
    mk = lambda shape_fn: [shape_fn(k) if op == "relu" else None for k, op in enumerate(net.ops)]
    split = mk(lambda k: torch.stack([domains[d][k].float() for d in range(D)]).reshape(D, -1).to(x.device))
    alpha, am, av = (mk(lambda k: torch.empty(D, m, net.sizes[k], device=x.device)) for _ in range(3))
    beta, bm, bv = (mk(lambda k: torch.zeros(D, m, net.sizes[k], device=x.device)) for _ in range(3))
    lbp.apply_splits(net, split, dlo, dhi)
    lbp.alpha_init(net, dlo, dhi, alpha, am, av, m)
    nb = ctypes.c_size_t(0)
    lbp._check(lbp.lib().vb_bab_workspace_size(net.gp, m, D, ctypes.byref(nb)), "ws")
    ws = net.workspace(int(nb.value))
    lb = torch.empty(steps + 1, D, m, device=x.device)
    best = torch.empty(D, m, device=x.device)
    for t in list(range(1, steps + 1)) + [0]:
        row = t - 1 if t > 0 else steps
        lbp.alpha_step_rows(net, len(wl.nodes) - 1, Cd, dlo, dhi, xd, float(wl.eps), alpha, am, av, t, lr, ws,
                            lb_out=lb[row], best_lb=best, beta=(split, beta, bm, bv))
    torch.cuda.synchronize()
    for d, sp in enumerate(domains):
        lo_b, hi_b = clamp_bounds(lo, hi, 0, sp, onet)
        out, ref_best, _ = beta_crown(wl, lo_b, hi_b, wl.x0[0], sp, wl.C[0], steps, lr)
        for t in range(steps + 1):
            assert_close(lb[t, d], out[t], f"domain {d} step {t}")
        assert_close(best[d], ref_best, f"domain {d} best")
        # beta moved the bound: better than beta = 0 at the end
        assert bool((ref_best >= out[0] - 1e-9).all())
    assert bool((beta[relus[0]] > 0).any() or (beta[relus[1]] > 0).any())


def _gpu_bab(lbp, wl, b, steps, batch, max_domains, method="crown"):
    w1 = wl.subset([b])
    net, x, C = lbp.prepare(w1)
    out = lbp.crown(net, x, float(w1.eps), C, method)
    torch.cuda.synchronize()
    return lbp.bab(net, x[0].contiguous(), float(w1.eps), C[0].contiguous(), out["lo"], out["hi"], steps=steps,
                   lr=0.1, batch=batch, max_domains=max_domains)


def test_bab_config1_proves_what_alpha_crown_does_not(lbp):
    wl = wk.config(1)
    net = Oracle(wl.nodes)
    lo, hi = intermediate_bounds(net, wl.x0, wl.eps, "crown")
    for b, budget in ((4, 200), (1, 40)):
        ref = oracle_bab(wl, b, lo, hi, steps=20, lr=0.1, batch=8, max_domains=budget)
        ok, doms, root = _gpu_bab(lbp, wl, b, 20, 8, budget)
        print(f"input {b}: GPU {'verified' if ok else 'undecided'} after {doms} sub-domains, oracle "
              f"{ref['verdict']} after {ref['domains']}", flush=True)
        assert ok == (ref["verdict"] == "verified")
        assert doms == ref["domains"]
        assert_close(root, ref["record"][0]["lb"], "root bound")
        if b == 4:
            assert ok and float(root.min()) < 0.0   # alpha-CROWN alone does not prove it


def test_bab_tiny_nets_match_exact_minima(lbp):
    import test_oracle_bab as tob
    for wl, m in tob.CASES[:12]:
        ok, doms, _ = _gpu_bab(lbp, wl, 0, 30, 4, 600)
        print(f"{wl.name} seed {wl.cfg}: exact min {m:+.4f}, GPU {'verified' if ok else 'undecided'} "
              f"after {doms}", flush=True)
        assert ok == (m > 0)
