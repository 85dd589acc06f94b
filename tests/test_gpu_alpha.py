"""GPU parity: alpha-CROWN (evaluation, exact adjoint, projected Adam) against the float64 oracle."""
import numpy as np
import pytest
import torch

import workloads as wk
from helpers import assert_close, ensure_built
from oracle import Oracle, ibp, spec_bounds_crown
from oracle.alpha import alpha_crown as oracle_alpha

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lbp():
    ensure_built()
    import linear_bound_propagation_amd as m
    return m


def _gpu_alpha(lbp, wl, steps, compact=False):
    net, x, C = lbp.prepare(wl)
    out = lbp.crown(net, x, float(wl.eps), C, "ibp")
    lay = lbp.alpha_layout(net, out["lo"], out["hi"]) if compact else None
    best, lb_steps, state = lbp.alpha_crown(net, x, float(wl.eps), C, out["lo"], out["hi"], steps, wl.alpha_lr,
                                            layout=lay)
    torch.cuda.synchronize()
    return out, best, lb_steps, state, lay


def _oracle(wl, steps, batch_idx=None):
    net = Oracle(wl.nodes)
    lo, hi = ibp(net, wl.x0, wl.eps)
    crown_lb, _ = spec_bounds_crown(net, lo, hi, wl.x0, wl.eps, wl.C, batch_idx=batch_idx)
    res = oracle_alpha(wl, lo, hi, steps=steps, batch_idx=batch_idx)
    return crown_lb, res


# first convs with 16 to 64 output channels over 2 to 4 input channels take the
# direct kernels (the domain step keeps Psi; the adjoint runs without im2col);
# the others take the im2col + GEMM adjoint
CNN_KINDS = {
    "cnn": dict(seed=22, convs=((6, 1), (12, 2)), in_shape=(3, 8, 8)),
    "cnn8": dict(seed=24, convs=((8, 1), (12, 2)), in_shape=(3, 8, 8)),
    "cnn16": dict(seed=25, convs=((16, 1), (12, 2)), in_shape=(3, 8, 8)),
    "cnn32s2": dict(seed=26, convs=((32, 2), (8, 1)), in_shape=(2, 9, 9)),
    "cnn64c4": dict(seed=27, convs=((64, 1), (8, 2)), in_shape=(4, 6, 6)),
    "cnn48c1": dict(seed=28, convs=((48, 1), (8, 2)), in_shape=(1, 7, 7)),
    # 900 output pixels: bands of 256 start and end inside image rows
    "cnn16w30": dict(seed=29, convs=((16, 1), (8, 2)), in_shape=(3, 30, 30)),
}


@pytest.mark.parametrize("compact", [False, True])
@pytest.mark.parametrize("kind", ["mlp"] + list(CNN_KINDS))
def test_alpha_small(lbp, kind, compact):
    if kind == "mlp":
        wl = wk.tiny_mlp([40, 70, 50, 8], 0.08, 21, batch=3)
        wl.intermediate = "ibp"
    else:
        k = CNN_KINDS[kind]
        wl = wk.cnn(2, 0.02, k["seed"], convs=k["convs"], fcs=(30, 10), in_shape=k["in_shape"])
    steps = 8
    print(f"alpha {kind} steps {steps} compact {compact}", flush=True)
    out, best, lb_steps, (alpha, _, _), lay = _gpu_alpha(lbp, wl, steps, compact)
    crown_lb, ref = _oracle(wl, steps)
    if compact:
        # the same arithmetic as the dense layout: identical bounds at every step
        _, best_d, lb_d, _, _ = _gpu_alpha(lbp, wl, steps)
        assert torch.equal(lb_steps, lb_d) and torch.equal(best, best_d)
    # the first evaluation uses the adaptive CROWN slopes
    assert_close(lb_steps[0], crown_lb, "lb at alpha init vs oracle CROWN")
    assert_close(lb_steps[0], out["lb"].double().cpu(), "lb at alpha init vs GPU CROWN", atol=1e-6, rtol=1e-6)
    for t in range(steps + 1):
        assert_close(lb_steps[t], ref["lb_steps"][t], f"lb after {t} Adam steps")
    assert_close(best, ref["best"], "best")
    assert bool((best >= lb_steps[0] - 1e-6).all())
    assert bool((best > lb_steps[0] + 1e-4).any()), "alpha optimisation should tighten some bound"
    for k, a in enumerate(alpha):
        if a is None:
            continue
        if lay is None:
            assert bool(((a >= 0) & (a <= 1)).all())
        else:
            # compact rows: only the columns of each input's unstable neurons hold slopes
            for b in range(a.shape[0]):
                cols = lay.index[k][b][lay.index[k][b] >= 0].long()
                v = a[b][:, cols]
                assert bool(((v >= 0) & (v <= 1)).all())


@pytest.fixture(scope="module")
def config4_oracle():
    wl = wk.config(4)
    idx = [0, 15]
    crown_lb, ref = _oracle(wl, wl.alpha_steps, batch_idx=idx)
    return wl, idx, crown_lb, ref


@pytest.mark.parametrize("compact", [True, False])
def test_config4_full_size_sampled_inputs(lbp, config4_oracle, compact):
    wl, idx, crown_lb, ref = config4_oracle
    print(wl.name, "compact", compact, flush=True)
    out, best, lb_steps, _, _ = _gpu_alpha(lbp, wl, wl.alpha_steps, compact)
    assert_close(lb_steps[0][idx], crown_lb[idx], "lb at alpha init")
    assert_close(best[idx], ref["best"][idx], "best lower bound after 20 Adam steps")
    for t in (1, 5, 10, 20):
        assert_close(lb_steps[t][idx], ref["lb_steps"][t][idx], f"lb after {t} steps")
    gain = (best - lb_steps[0]).double()
    print(f"mean improvement over CROWN: {gain.mean().item():.4g} (max {gain.max().item():.4g})", flush=True)
    assert bool((gain >= -1e-3).all())


def test_alpha_upper_bounds_via_negated_specs(lbp):
    """alpha-CROWN on the upper side: optimising slopes for the rows -C gives
    ub = -lb(-C); parity with the oracle run on -C, and the optimised upper bound
    is no looser than CROWN's."""
    wl = wk.tiny_mlp([40, 70, 50, 8], 0.08, 23, batch=2)
    wl.intermediate = "ibp"
    wl.C = -wl.C
    steps = 6
    out, best, lb_steps, _, _ = _gpu_alpha(lbp, wl, steps)
    crown_lb, ref = _oracle(wl, steps)
    for t in range(steps + 1):
        assert_close(lb_steps[t], ref["lb_steps"][t], f"lb(-C) after {t} Adam steps")
    assert_close(best, ref["best"], "best lb(-C)")
    ub_alpha = -best.double().cpu()
    ub_crown = -crown_lb
    assert bool((ub_alpha <= ub_crown + 1e-5).all())


# ---------------------------------------------------------------------------
# alpha-CROWN on intermediate bounds (identity rows of every refined layer)

def _alpha_intermediate_check(lbp, wl, steps, batch_idx):
    from oracle.alpha import alpha_intermediate_bounds, alpha_rows
    from oracle.bounds import _identity_rows
    from helpers import nhwc
    net, x, C = lbp.prepare(wl)
    ws = net.workspace(net.workspace_size(wl.batch, wl.m, "ibp", alpha_rows=True))
    lo, hi, _, _ = lbp.ibp(net, x, float(wl.eps), ws=ws)
    trace = {}
    lbp.alpha_intermediate(net, x, float(wl.eps), lo, hi, steps, wl.alpha_lr, ws, trace=trace)
    torch.cuda.synchronize()
    lo_ref, hi_ref = alpha_intermediate_bounds(wl, steps, wl.alpha_lr, batch_idx=batch_idx)
    onet = Oracle(wl.nodes)
    lo_ibp, hi_ibp = ibp(onet, wl.x0, wl.eps)
    assert list(trace) == lbp.relu_inputs_refined(net)
    for z, (ls, us) in trace.items():
        shape = wl.nodes[z].shape
        n = wl.nodes[z].size
        # every Adam step of the first refined layer against the oracle's trajectory on
        # the same (IBP) bounds below it; the final bounds of every layer end to end
        if z == min(trace):
            rows = torch.cat([_identity_rows(shape, 1.0).reshape(n, -1), _identity_rows(shape, -1.0).reshape(n, -1)])
            rows = rows.reshape((2 * n,) + tuple(shape))
            for b in batch_idx:
                lbs, _ = alpha_rows(wl, lo_ibp, hi_ibp, b, z, rows, steps, wl.alpha_lr)
                for t in range(steps + 1):
                    assert_close(ls[t, b], nhwc(lbs[t, :n].reshape((1,) + tuple(shape)), shape)[0],
                                 f"l of node {z}, step {t}, input {b}")
                    assert_close(us[t, b], nhwc(-lbs[t, n:].reshape((1,) + tuple(shape)), shape)[0],
                                 f"u of node {z}, step {t}, input {b}")
        assert_close(lo[z][batch_idx], nhwc(lo_ref[z][batch_idx], shape), f"best l of node {z}")
        assert_close(hi[z][batch_idx], nhwc(hi_ref[z][batch_idx], shape), f"best u of node {z}")
        # alpha tightens the CROWN iterate (step 0 evaluates the adaptive slopes)
        assert bool((lo[z] >= ls[0] - 1e-6).all() and (hi[z] <= us[0] + 1e-6).all())
    return net, lo, hi


def test_alpha_intermediate_bounds_mlp(lbp):
    wl = wk.tiny_mlp([30, 60, 50, 40, 6], 0.06, 41, batch=3)
    wl.alpha_lr = 0.1
    print("alpha intermediate bounds, tiny MLP", flush=True)
    _alpha_intermediate_check(lbp, wl, 8, [0, 1, 2])


def test_alpha_intermediate_bounds_config1(lbp):
    """The 784-100-100-10 workload: alpha on the second layer's 200 identity rows per
    input, 20 Adam steps, every step compared with the oracle on inputs 0 and 7."""
    wl = wk.config(1)
    wl.alpha_lr = 0.1
    print("alpha intermediate bounds,", wl.name, flush=True)
    _alpha_intermediate_check(lbp, wl, 20, [0, 7])


def test_alpha_intermediate_bounds_small_cnn(lbp):
    wl = wk.cnn(2, 0.02, 42, convs=((8, 1), (16, 2)), fcs=(20, 5), in_shape=(3, 8, 8), intermediate="ibp")
    wl.alpha_lr = 0.1
    print("alpha intermediate bounds, small CNN", flush=True)
    _alpha_intermediate_check(lbp, wl, 5, [0, 1])
