"""alpha-CROWN: projected Adam ascent on per-neuron, per-spec lower ReLU slopes.

Test infrastructure only (see the package docstring).

Page: "Scaling Neural Network Verification with Tensor Parallelism and Fully
Sharded Data Parallelism" -- the per-neuron alpha tensors are ReLU slopes
(Sec. 3, Sec. 4.3).  Reading used here (the page gives no formulas): every
unstable ReLU neuron gets its own lower slope alpha in [0, 1] per input and
per spec row, initialised with the adaptive CROWN slope; the objective is the
sum of the spec lower bounds; the ascent is bias-corrected Adam followed by
clipping to [0, 1]; the result is the best lower bound seen over the
iterates.  The gradient is torch's reverse mode through the float64 CROWN
evaluation of ``bounds.backward`` (at Psi = 0 the branch Psi >= 0 is taken,
|.| has derivative sign(.) with sign(0) = 0).
"""
from __future__ import annotations

import numpy as np
import torch

from .bounds import Oracle, backward, relaxation, _domain, _t

f64 = torch.float64


def adam_ascent_step(x, g, m, v, t: int, lr: float, b1: float = 0.9, b2: float = 0.999,
                     eps: float = 1e-8):
    """One bias-corrected Adam step that increases the objective, then clip to [0, 1].
    Returns new (x, m, v)."""
    m = b1 * m + (1 - b1) * g
    v = b2 * v + (1 - b2) * g * g
    mh = m / (1 - b1 ** t)
    vh = v / (1 - b2 ** t)
    x = (x + lr * mh / (vh.sqrt() + eps)).clamp(0.0, 1.0)
    return x, m, v


def compact_columns(lo, hi):
    """Compact storage of alpha (the page stresses that the alpha tensors dominate
    alpha-CROWN's memory, Sec. 3 and Sec. 4.3; a slope only matters on an unstable
    neuron, l < 0 < u).  lo, hi: one node's bounds [B][n] in any fixed neuron order.
    Returns (col [B][n] int32, width): col[b][j] = the number of unstable neurons of
    input b before j when j is unstable, else -1; width = the largest number of
    unstable neurons of any input."""
    lo = np.asarray(lo, dtype=np.float64)
    hi = np.asarray(hi, dtype=np.float64)
    col = np.full(lo.shape, -1, dtype=np.int32)
    width = 0
    for b in range(lo.shape[0]):
        count = 0
        for j in range(lo.shape[1]):
            if lo[b, j] < 0.0 and hi[b, j] > 0.0:
                col[b, j] = count
                count += 1
        width = max(width, count)
    return col, width


def alpha_init(net: Oracle, lo, hi, b: int, m: int):
    """Adaptive CROWN slopes broadcast over the m spec rows, one tensor per ReLU node."""
    out = {}
    for r in net.relu_nodes():
        z = net.nodes[r].inputs[0]
        a, _, _, _ = relaxation(lo[z][b], hi[z][b])
        out[r] = a.unsqueeze(0).expand((m,) + tuple(a.shape)).clone()
    return out


def alpha_crown(wl, lo, hi, steps: int = None, lr: float = None, stop: int = 0,
                batch_idx=None, b1=0.9, b2=0.999, adam_eps=1e-8):
    """Lower bounds of C f(x) over the iterates of alpha optimisation.

    For each input: `steps` rounds of (evaluate lb_t, gradient of sum(lb_t), Adam
    ascent + clip), then one final evaluation.  Returns dict with
    "lb_steps" [steps+1][B][m], "best" [B][m] (max over the iterates) and the
    final alphas per input.
    """
    net = Oracle(wl.nodes)
    steps = wl.alpha_steps if steps is None else steps
    lr = wl.alpha_lr if lr is None else lr
    C = _t(wl.C)
    B, m = C.shape[0], C.shape[1]
    batch_idx = range(B) if batch_idx is None else batch_idx
    L = len(net.nodes) - 1
    lb_steps = torch.full((steps + 1, B, m), float("nan"), dtype=f64)
    alphas_out = {}
    for b in batch_idx:
        dc, dr = _domain(net, lo, hi, wl.x0, wl.eps, b, stop)
        al = alpha_init(net, lo, hi, b, m)
        mom = {k: torch.zeros_like(v) for k, v in al.items()}
        vel = {k: torch.zeros_like(v) for k, v in al.items()}
        for t in range(1, steps + 1):
            leaf = {k: v.clone().requires_grad_(True) for k, v in al.items()}
            lb = backward(net, lo, hi, b, L, C[b], stop, dc, dr, alpha=leaf)
            lb_steps[t - 1, b] = lb.detach()
            lb.sum().backward()
            for k in al:
                g = leaf[k].grad if leaf[k].grad is not None else torch.zeros_like(al[k])
                al[k], mom[k], vel[k] = adam_ascent_step(al[k], g, mom[k], vel[k], t, lr, b1, b2, adam_eps)
        with torch.no_grad():
            lb_steps[steps, b] = backward(net, lo, hi, b, L, C[b], stop, dc, dr, alpha=al)
        alphas_out[b] = al
    best = lb_steps.max(dim=0).values
    return {"lb_steps": lb_steps, "best": best, "alpha": alphas_out}


def alpha_gradient(wl, lo, hi, b: int, alpha: dict, stop: int = 0):
    """(lb, d sum(lb) / d alpha) for one input at the given slopes (float64 autograd)."""
    net = Oracle(wl.nodes)
    C = _t(wl.C)
    dc, dr = _domain(net, lo, hi, wl.x0, wl.eps, b, stop)
    leaf = {k: v.clone().requires_grad_(True) for k, v in alpha.items()}
    lb = backward(net, lo, hi, b, len(net.nodes) - 1, C[b], stop, dc, dr, alpha=leaf)
    lb.sum().backward()
    return lb.detach(), {k: (v.grad if v.grad is not None else torch.zeros_like(v)) for k, v in leaf.items()}


def evaluate(wl, lo, hi, b: int, alpha: dict, stop: int = 0) -> torch.Tensor:
    net = Oracle(wl.nodes)
    C = _t(wl.C)
    dc, dr = _domain(net, lo, hi, wl.x0, wl.eps, b, stop)
    with torch.no_grad():
        return backward(net, lo, hi, b, len(net.nodes) - 1, C[b], stop, dc, dr, alpha=alpha)


def alpha_rows(wl, lo, hi, b: int, start: int, rows, steps: int, lr: float, stop: int = 0,
               b1=0.9, b2=0.999, adam_eps=1e-8):
    """alpha-CROWN on arbitrary rows over node `start` for input b: every row is a
    linear function of that node bounded from below; each row has its own slopes
    (one per ReLU neuron between `stop` and `start`), initialised with the adaptive
    CROWN slopes, and `steps` rounds of (evaluate, gradient of the sum of the rows'
    lower bounds, Adam ascent + clip to [0, 1]) are followed by one evaluation.
    Rows are independent, so each row's slopes follow the gradient of its own bound.
    Returns (lower bound per evaluation [steps+1][R], final slopes)."""
    net = Oracle(wl.nodes)
    dc, dr = _domain(net, lo, hi, wl.x0, wl.eps, b, stop)
    rows = torch.as_tensor(rows, dtype=f64)
    R = rows.shape[0]
    al = {r: v for r, v in alpha_init(net, lo, hi, b, R).items() if stop < r < start}
    mom = {k: torch.zeros_like(v) for k, v in al.items()}
    vel = {k: torch.zeros_like(v) for k, v in al.items()}
    out = torch.empty((steps + 1, R), dtype=f64)
    for t in range(1, steps + 1):
        leaf = {k: v.clone().requires_grad_(True) for k, v in al.items()}
        lb = backward(net, lo, hi, b, start, rows, stop, dc, dr, alpha=leaf)
        out[t - 1] = lb.detach()
        lb.sum().backward()
        for k in al:
            g = leaf[k].grad if leaf[k].grad is not None else torch.zeros_like(al[k])
            al[k], mom[k], vel[k] = adam_ascent_step(al[k], g, mom[k], vel[k], t, lr, b1, b2, adam_eps)
    with torch.no_grad():
        out[steps] = backward(net, lo, hi, b, start, rows, stop, dc, dr, alpha=al)
    return out, al


def alpha_intermediate_bounds(wl, steps: int, lr: float, batch_idx=None):
    """Intermediate bounds by alpha-CROWN (the per-neuron alpha tensors of the page,
    Sec. 3 and Sec. 4.3, here also on the intermediate layers): IBP first; then for
    every ReLU input z in topological order that is more than one affine step from
    the input, its identity rows (+e_j for the lower bound, -e_j for the upper) are
    optimised with `alpha_rows` over the bounds of the earlier layers, and
    l_j = max over the iterates of lb(+e_j), u_j = min over the iterates of
    -lb(-e_j).  Returns (lo, hi) lists [B][*shape] (only inputs in batch_idx refined)."""
    from .bounds import ibp, _identity_rows, _one_affine_step
    net = Oracle(wl.nodes)
    lo, hi = ibp(net, wl.x0, wl.eps)
    B = lo[0].shape[0]
    batch_idx = range(B) if batch_idx is None else batch_idx
    for r in net.relu_nodes():
        z = net.nodes[r].inputs[0]
        if z <= 0 or _one_affine_step(net, z, 0):
            continue
        shape = net.shape[z]
        n = int(np.prod(shape))
        rows = torch.cat([_identity_rows(shape, 1.0).reshape(n, -1), _identity_rows(shape, -1.0).reshape(n, -1)])
        rows = rows.reshape((2 * n,) + tuple(shape))
        for b in batch_idx:
            lbs, _ = alpha_rows(wl, lo, hi, b, z, rows, steps, lr)
            best = lbs.max(dim=0).values
            lo[z][b] = best[:n].reshape(shape)
            hi[z][b] = -best[n:].reshape(shape)
    return lo, hi
