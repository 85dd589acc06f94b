"""beta-CROWN bounds of sub-domains and branch-and-bound, in float64.

Test infrastructure only (see the package docstring).

Page: "Scaling Neural Network Verification with Tensor Parallelism and Fully
Sharded Data Parallelism" -- complete verification with beta-CROWN and
branch-and-bound, which proved a ResNet on CIFAR-100 (Sec. 2.2, Sec. 3 and
Sec. 4.3).  The page gives no formulas; the readings used here:

* A sub-domain of one input is a set of ReLU split constraints: for the input
  neuron j of ReLU node k, +1 means z_j >= 0 and -1 means z_j <= 0.  Its
  intermediate bounds are the root's, with every split neuron clamped to its
  side (l_j = max(l_j, 0) for +1, u_j = min(u_j, 0) for -1); they are not
  recomputed below the splits.
* Its spec lower bounds: for multipliers beta >= 0 (one per row and split
  neuron), min over the relaxed network of  C f(x) - sum_j beta_j s_j z_j(x),
  which bounds C f from below on the sub-domain (there s_j z_j >= 0); alpha
  (lower ReLU slopes) and beta are raised together by projected Adam
  (alpha clipped to [0, 1], beta to [0, inf)), `steps` steps from the adaptive
  slopes and beta = 0, then one evaluation; the bound is the best iterate.
* Branch and bound: a first-in first-out queue of sub-domains processed in
  batches; a sub-domain is proved when every spec lower bound is > 0; otherwise
  it is split in two on the unstable neuron (under its bounds) with the largest
  score sum over the unproved rows of max(-Psi_j, 0) * t_j (the part of the
  bound lost to that neuron's upper relaxation offset; Psi over the ReLU output,
  t = -u l / (u - l)), ties to the lowest (node, index).  The input is proved
  when the queue empties; the search stops undecided when a sub-domain has no
  unstable neuron left or the domain budget is spent.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np
import torch

from .bounds import Oracle, backward, relaxation, _domain, _t
from .alpha import adam_ascent_step

f64 = torch.float64


def clamp_bounds(lo, hi, b: int, splits: Dict[int, torch.Tensor], net: Oracle):
    """Copies of input b's node bounds ([1][*shape] per node) with the split neurons
    clamped to their sides.  splits: ReLU node -> sign tensor over its input's shape."""
    lo_b = [t[b:b + 1].clone() for t in lo]
    hi_b = [t[b:b + 1].clone() for t in hi]
    for r, sg in splits.items():
        z = net.nodes[r].inputs[0]
        lo_b[z][0] = torch.where(sg > 0, lo_b[z][0].clamp(min=0.0), lo_b[z][0])
        hi_b[z][0] = torch.where(sg < 0, hi_b[z][0].clamp(max=0.0), hi_b[z][0])
    return lo_b, hi_b


def beta_crown(wl, lo_b, hi_b, x0_b, splits: Dict[int, torch.Tensor], C_b, steps: int, lr: float,
               b1=0.9, b2=0.999, adam_eps=1e-8, keep_psi=False):
    """Spec lower bounds of one sub-domain (bounds lo_b, hi_b already clamped, [1][*]).
    Returns (lb per evaluation [steps+1][m], best [m], Psi per ReLU node of the best
    evaluation's slopes if keep_psi)."""
    net = Oracle(wl.nodes)
    x0 = _t(x0_b)[None]
    dc, dr = _domain(net, lo_b, hi_b, x0, wl.eps, 0, 0)
    C = _t(C_b)
    m = C.shape[0]
    L = len(net.nodes) - 1
    al = {}
    for r in net.relu_nodes():
        z = net.nodes[r].inputs[0]
        a, _, _, _ = relaxation(lo_b[z][0], hi_b[z][0])
        al[r] = a.unsqueeze(0).expand((m,) + tuple(a.shape)).clone()
    be = {r: torch.zeros((m,) + tuple(sg.shape), dtype=f64) for r, sg in splits.items()}
    state = {("a", k): (torch.zeros_like(v), torch.zeros_like(v)) for k, v in al.items()}
    state.update({("b", k): (torch.zeros_like(v), torch.zeros_like(v)) for k, v in be.items()})
    out = torch.empty((steps + 1, m), dtype=f64)
    for t in range(1, steps + 1):
        la = {k: v.clone().requires_grad_(True) for k, v in al.items()}
        lbeta = {k: v.clone().requires_grad_(True) for k, v in be.items()}
        lb = backward(net, lo_b, hi_b, 0, L, C, 0, dc, dr, alpha=la, beta=lbeta, splits=splits)
        out[t - 1] = lb.detach()
        lb.sum().backward()
        for k in al:
            g = la[k].grad if la[k].grad is not None else torch.zeros_like(al[k])
            mm, vv = state[("a", k)]
            al[k], mm, vv = adam_ascent_step(al[k], g, mm, vv, t, lr, b1, b2, adam_eps)
            state[("a", k)] = (mm, vv)
        for k in be:
            g = lbeta[k].grad if lbeta[k].grad is not None else torch.zeros_like(be[k])
            mm, vv = state[("b", k)]
            mm = b1 * mm + (1 - b1) * g
            vv = b2 * vv + (1 - b2) * g * g
            step = lr * (mm / (1 - b1 ** t)) / ((vv / (1 - b2 ** t)).sqrt() + adam_eps)
            be[k] = (be[k] + step).clamp(min=0.0)
            state[("b", k)] = (mm, vv)
    keep = {} if keep_psi else None
    with torch.no_grad():
        out[steps] = backward(net, lo_b, hi_b, 0, L, C, 0, dc, dr, alpha=al, beta=be, splits=splits, keep=keep)
    best = out.max(dim=0).values
    return out, best, keep


def branch_scores(net: Oracle, lo_b, hi_b, psi: Dict[int, torch.Tensor], open_rows: torch.Tensor):
    """Score of every unstable neuron (ReLU node -> tensor over its input's shape):
    sum over the open rows of max(-Psi, 0) * t, t = -u l / (u - l); stable neurons -inf."""
    out = {}
    for r in net.relu_nodes():
        z = net.nodes[r].inputs[0]
        l, u = lo_b[z][0], hi_b[z][0]
        unstable = (l < 0) & (u > 0)
        t = torch.where(unstable, -u * l / torch.where(unstable, u - l, torch.ones_like(u)), torch.zeros_like(u))
        P = psi[r][open_rows]
        sc = (torch.clamp(-P, min=0.0) * t).sum(0)
        out[r] = torch.where(unstable, sc, torch.full_like(sc, -float("inf")))
    return out


def pick_neuron(scores: Dict[int, torch.Tensor]):
    """(ReLU node, flat index) of the largest score; ties to the lowest (node, index);
    None when no neuron is unstable."""
    best = None
    for r in sorted(scores):
        v = scores[r].reshape(-1)
        if not bool(torch.isfinite(v).any()):
            continue
        i = int(torch.argmax(v))          # first index of the maximum
        if best is None or v[i] > best[2]:
            best = (r, i, v[i])
    return None if best is None else (best[0], best[1])


def bab(wl, b: int, lo, hi, steps: int, lr: float, batch: int = 8, max_domains: int = 256):
    """Branch and bound for input b of a workload (root bounds lo, hi of every node,
    from any intermediate method).  Returns a dict: verdict ("verified",
    "undecided"), domains processed, and the record of every processed domain
    (its splits, its best spec lower bounds, proved or not)."""
    net = Oracle(wl.nodes)
    relus = net.relu_nodes()
    shapes = {r: net.shape[net.nodes[r].inputs[0]] for r in relus}
    queue: List[Dict[int, torch.Tensor]] = [{}]
    record = []
    done = 0
    while queue:
        if done >= max_domains:
            return {"verdict": "undecided", "domains": done, "record": record, "reason": "budget"}
        todo, queue = queue[:batch], queue[batch:]
        children = []
        for splits in todo:
            full = {r: splits.get(r, torch.zeros(shapes[r], dtype=f64)) for r in relus}
            lo_b, hi_b = clamp_bounds(lo, hi, b, {r: s for r, s in full.items() if bool((s != 0).any())}, net)
            used = {r: s for r, s in full.items() if bool((s != 0).any())}
            _, best, keep = beta_crown(wl, lo_b, hi_b, wl.x0[b], used, wl.C[b], steps, lr, keep_psi=True)
            proved = bool((best > 0).all())
            record.append({"splits": {r: s.clone() for r, s in used.items()}, "lb": best, "proved": proved})
            done += 1
            if proved:
                continue
            open_rows = best <= 0
            pick = pick_neuron(branch_scores(net, lo_b, hi_b, keep, open_rows))
            if pick is None:
                return {"verdict": "undecided", "domains": done, "record": record, "reason": "no unstable neuron"}
            r, i = pick
            for sign in (1.0, -1.0):
                child = {k: v.clone() for k, v in used.items()}
                s = child.get(r, torch.zeros(shapes[r], dtype=f64)).reshape(-1).clone()
                s[i] = sign
                child[r] = s.reshape(shapes[r])
                children.append(child)
        queue.extend(children)
    return {"verdict": "verified", "domains": done, "record": record, "reason": ""}
