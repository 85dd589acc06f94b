"""IBP, ReLU relaxation, CROWN back-substitution and concretisation in float64.

Test infrastructure only (see the package docstring).  All tensors are torch
float64 on the CPU; conv activations are [C][H][W] per input (PyTorch layout).

Page: "Scaling Neural Network Verification with Tensor Parallelism and Fully
Sharded Data Parallelism" -- Sec. 1 (the verification problem and the A
matrices), Sec. 2.1 (slopes lambda_i from intermediate bounds; IBP substituted
for intermediate bounds), Sec. 2.2 (bound propagation through convolutions).
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np
import torch
import torch.nn.functional as F

f64 = torch.float64


def _t(a) -> torch.Tensor:
    return torch.as_tensor(np.asarray(a), dtype=f64)


class Oracle:
    """A network (list of ``workloads.Node``) with float64 copies of its parameters."""

    def __init__(self, nodes):
        self.nodes = nodes
        self.W = [None if n.weight is None else _t(n.weight) for n in nodes]
        self.b = [None if n.bias is None else _t(n.bias) for n in nodes]
        self.shape = [tuple(n.shape) for n in nodes]
        self.consumers: List[List[int]] = [[] for _ in nodes]
        for k, n in enumerate(nodes):
            for i in n.inputs:
                self.consumers[i].append(k)

    def relu_nodes(self) -> List[int]:
        return [k for k, n in enumerate(self.nodes) if n.op == "relu"]


# ---------------------------------------------------------------------------
# IBP: interval bound propagation in centre/radius form


def _affine(net: Oracle, k: int, c: torch.Tensor, absw: bool) -> torch.Tensor:
    """Apply node k's weight (or |weight|) to a batch [B][*in]; no bias."""
    nd = net.nodes[k]
    W = net.W[k].abs() if absw else net.W[k]
    if nd.op == "linear":
        return c @ W.T
    return F.conv2d(c, W, None, stride=nd.stride, padding=nd.pad)


def _add_bias(net: Oracle, k: int, y: torch.Tensor) -> torch.Tensor:
    if net.nodes[k].op == "linear":
        return y + net.b[k]
    return y + net.b[k][None, :, None, None]


def ibp(net: Oracle, x0, eps) -> (List[torch.Tensor], List[torch.Tensor]):
    """Interval bounds [B][*shape] of every node over the L-inf ball x0 +- eps.

    Affine nodes use the centre/radius form: c' = W c + b, r' = |W| r, with
    (c, r) = ((l+u)/2, (u-l)/2) taken from the producer's bounds; the input node
    hands over (x0, eps) directly.  ReLU clamps both ends at 0, Add sums, GAP
    averages over space, Flatten reindexes in (C, H, W) order.
    """
    x0 = _t(x0)
    eps = float(np.float32(eps))
    lo: List[torch.Tensor] = []
    hi: List[torch.Tensor] = []
    for k, nd in enumerate(net.nodes):
        if nd.op == "input":
            lo.append(x0 - eps)
            hi.append(x0 + eps)
            continue
        i = nd.inputs[0]
        if nd.op in ("linear", "conv"):
            if net.nodes[i].op == "input":
                c, r = x0, torch.full_like(x0, eps)
            else:
                c, r = (lo[i] + hi[i]) / 2, (hi[i] - lo[i]) / 2
            cc = _add_bias(net, k, _affine(net, k, c, False))
            rr = _affine(net, k, r, True)
            lo.append(cc - rr)
            hi.append(cc + rr)
        elif nd.op == "relu":
            lo.append(lo[i].clamp(min=0))
            hi.append(hi[i].clamp(min=0))
        elif nd.op == "add":
            j = nd.inputs[1]
            lo.append(lo[i] + lo[j])
            hi.append(hi[i] + hi[j])
        elif nd.op == "gap":
            lo.append(lo[i].mean(dim=(2, 3)))
            hi.append(hi[i].mean(dim=(2, 3)))
        elif nd.op == "flatten":
            lo.append(lo[i].reshape(lo[i].shape[0], -1))
            hi.append(hi[i].reshape(hi[i].shape[0], -1))
        else:
            raise ValueError(nd.op)
    return lo, hi


def spec_bounds_ibp(net: Oracle, lo, hi, C) -> (torch.Tensor, torch.Tensor):
    """IBP bounds of C f(x): C is folded into the last Linear (W' = C W, b' = C b)
    and one centre/radius affine step is taken over the box of its input."""
    L = len(net.nodes) - 1
    assert net.nodes[L].op == "linear"
    i = net.nodes[L].inputs[0]
    C = _t(C)
    c, r = (lo[i] + hi[i]) / 2, (hi[i] - lo[i]) / 2
    Wf = C @ net.W[L]                         # [B][m][n_in]
    bf = C @ net.b[L]                         # [B][m]
    cc = torch.einsum("bmn,bn->bm", Wf, c) + bf
    rr = torch.einsum("bmn,bn->bm", Wf.abs(), r)
    return cc - rr, cc + rr


# ---------------------------------------------------------------------------
# ReLU relaxation


def relaxation(l: torch.Tensor, u: torch.Tensor):
    """Per-neuron linear bounds a z <= relu(z) <= s z + t on [l, u].

    inactive (u <= 0, tested first): a = s = t = 0; active (l >= 0): a = s = 1,
    t = 0; unstable: s = u / (u - l), t = -s l and the adaptive lower slope
    a = 1 if u >= -l else 0 (the tie u = -l takes a = 1).
    Returns (a, s, t, unstable mask).
    """
    inactive = u <= 0
    active = (l >= 0) & ~inactive
    unstable = ~inactive & ~active
    denom = torch.where(unstable, u - l, torch.ones_like(u))
    s = torch.where(unstable, u / denom, active.to(f64))
    t = torch.where(unstable, -s * l, torch.zeros_like(u))
    a = torch.where(unstable, (u >= -l).to(f64), active.to(f64))
    return a, s, t, unstable


# ---------------------------------------------------------------------------
# CROWN back-substitution


def _push(lam: Dict[int, torch.Tensor], k: int, v: torch.Tensor):
    lam[k] = lam[k] + v if k in lam else v


def backward(net: Oracle, lo, hi, b: int, start: int, rows: torch.Tensor, stop: int,
             dom_c: torch.Tensor, dom_r: torch.Tensor, alpha: Optional[Dict[int, torch.Tensor]] = None,
             keep: Optional[dict] = None, beta: Optional[Dict[int, torch.Tensor]] = None,
             splits: Optional[Dict[int, torch.Tensor]] = None,
             decide: Optional[Dict[int, torch.Tensor]] = None, tau: float = 1e-6) -> torch.Tensor:
    """Lower bound of each row of `rows` (linear functions of node `start`) for input b.

    Lambda starts as `rows` over node `start` with the constant term d = 0 and is
    pushed to the producers in reverse topological order:
      Linear:  d += Lambda b;  Lambda_in += Lambda W
      Conv:    d += sum_{c,h,w} Lambda[c,h,w] b_c;  Lambda_in += conv^T(Lambda, W)
      ReLU:    with Psi = Lambda over the ReLU output, Lambda_z += Psi+ a + Psi- s and
               d += Psi- . t  (a replaced by alpha on unstable neurons if given)
      Add:     Lambda flows unchanged into both inputs
      GAP:     Lambda_in[c,h,w] += Lambda[c] / (H W)
      Flatten: reindex
    At `stop` (the domain) the bound is concretised over the box (dom_c, dom_r).
    `keep`, if given, receives Psi per ReLU node and the final Lambda.
    Split constraints (beta-CROWN): for ReLU node k, splits[k] holds +1 where the
    input neuron is constrained to z >= 0, -1 where z <= 0, 0 elsewhere, and
    beta[k] [R][*shape] >= 0 the rows' multipliers; the Lagrangian term
    -beta * split * z is added to Lambda over z (for points of the sub-domain it
    is <= 0, so the bound stays a lower bound there).
    Decision alignment at the adaptive-slope tie: where an unstable neuron's
    |u + l| <= tau (u - l), both choices of a are sound and float32 and float64
    bounds may choose differently; if `decide` holds for its ReLU input z a
    [B][*shape] boolean tensor (another implementation's choice a = 1), that
    choice is taken there (and only there).
    """
    R = rows.shape[0]
    lam: Dict[int, torch.Tensor] = {start: rows}
    bias_acc = torch.zeros(R, dtype=f64)
    for k in range(start, stop, -1):
        if k not in lam:
            continue
        L = lam.pop(k)
        nd = net.nodes[k]
        if nd.op == "linear":
            bias_acc = bias_acc + L @ net.b[k]
            _push(lam, nd.inputs[0], L @ net.W[k])
        elif nd.op == "conv":
            bias_acc = bias_acc + L.sum(dim=(2, 3)) @ net.b[k]
            in_shape = (R,) + net.shape[nd.inputs[0]]
            psi = torch.nn.grad.conv2d_input(in_shape, net.W[k], L, stride=nd.stride, padding=nd.pad)
            _push(lam, nd.inputs[0], psi)
        elif nd.op == "relu":
            z = nd.inputs[0]
            a, s, t, unstable = relaxation(lo[z][b], hi[z][b])
            if decide is not None and z in decide:
                l_, u_ = lo[z][b], hi[z][b]
                tie = unstable & ((u_ + l_).abs() <= tau * (u_ - l_))
                a = torch.where(tie, decide[z][b].to(f64), a)
            if alpha is not None and k in alpha:
                a = torch.where(unstable, alpha[k], a)
            if keep is not None:
                keep[k] = L
            lz = torch.where(L >= 0, L * a, L * s)
            beta_acc = (torch.where(L < 0, L, torch.zeros_like(L)) * t).reshape(R, -1).sum(1)
            bias_acc = bias_acc + beta_acc
            if beta is not None and k in beta:
                lz = lz - beta[k] * splits[k]
            _push(lam, z, lz)
        elif nd.op == "add":
            _push(lam, nd.inputs[0], L)
            _push(lam, nd.inputs[1], L)
        elif nd.op == "gap":
            C_, H, W_ = net.shape[nd.inputs[0]]
            _push(lam, nd.inputs[0], (L / (H * W_))[:, :, None, None].expand(R, C_, H, W_))
        elif nd.op == "flatten":
            _push(lam, nd.inputs[0], L.reshape((R,) + net.shape[nd.inputs[0]]))
        else:
            raise ValueError(f"cannot back-substitute through {nd.op} before reaching the domain")
    L = lam.pop(stop)
    assert not lam, "rows reach nodes outside the region bounded by the domain node"
    if keep is not None:
        keep["domain"] = L
    return concretize(L, bias_acc, dom_c, dom_r)


def concretize(L: torch.Tensor, beta: torch.Tensor, c: torch.Tensor, r: torch.Tensor) -> torch.Tensor:
    """min over the box |x - c| <= r of L x + beta  =  L c - |L| r + beta (per row)."""
    R = L.shape[0]
    Lf = L.reshape(R, -1)
    return Lf @ c.reshape(-1) - Lf.abs() @ r.reshape(-1) + beta


def _domain(net: Oracle, lo, hi, x0, eps, b: int, stop: int):
    if net.nodes[stop].op == "input":
        c = _t(x0[b])
        return c, torch.full_like(c, float(np.float32(eps)))
    return (lo[stop][b] + hi[stop][b]) / 2, (hi[stop][b] - lo[stop][b]) / 2


def _identity_rows(shape, sign: float, lo_row=0, hi_row=None) -> torch.Tensor:
    n = int(np.prod(shape))
    hi_row = n if hi_row is None else hi_row
    I = torch.zeros((hi_row - lo_row, n), dtype=f64)
    idx = torch.arange(lo_row, hi_row)
    I[idx - lo_row, idx] = sign
    return I.reshape((hi_row - lo_row,) + tuple(shape))


def _one_affine_step(net: Oracle, z: int, stop: int) -> bool:
    nd = net.nodes[z]
    if nd.op not in ("linear", "conv"):
        return False
    i = nd.inputs[0]
    while net.nodes[i].op == "flatten":
        i = net.nodes[i].inputs[0]
    return i == stop


def intermediate_bounds(net: Oracle, x0, eps, mode: str, region_start: Optional[int] = None,
                        batch_idx: Optional[Sequence[int]] = None, row_chunk: int = 4096,
                        decide: Optional[Dict[int, torch.Tensor]] = None):
    """Pre-activation bounds used for the ReLU relaxations.

    mode "ibp": IBP everywhere.  mode "crown": every ReLU input z, in topological
    order, gets l = lb(I), u = -lb(-I) by back-substitution to the input domain,
    using the bounds already computed for earlier ReLUs; a z one affine step
    from the domain keeps its IBP bounds (exact there).  mode "hybrid": IBP up
    to and including `region_start`, CROWN inside the region with the IBP box of
    `region_start` as the domain.  A suffix "+ibp" ("crown+ibp", "hybrid+ibp")
    intersects each CROWN result with that node's bounds from the initial IBP
    pass: l = max(l_crown, l_ibp), u = min(u_crown, u_ibp), before later layers
    use them.  A suffix "+unstable" computes rows only for the neurons the initial
    IBP pass leaves unstable (l < 0 < u); the other neurons keep their IBP bounds.
    Rows are independent, so they are processed in chunks of `row_chunk`.  Returns (lo, hi) lists [B][*shape] (float64); only the inputs
    in batch_idx are refined (all by default).  `decide`: tie decisions, see backward().
    """
    lo, hi = ibp(net, x0, eps)
    base, *flags = mode.split("+")
    assert base in ("ibp", "crown", "hybrid") and set(flags) <= {"ibp", "unstable"}, mode
    if base == "ibp":
        return lo, hi
    intersect = "ibp" in flags
    unstable_only = "unstable" in flags
    lo_ibp = [t.clone() for t in lo]
    hi_ibp = [t.clone() for t in hi]
    stop = 0 if base == "crown" else region_start
    B = lo[0].shape[0]
    batch_idx = range(B) if batch_idx is None else batch_idx
    for r in net.relu_nodes():
        z = net.nodes[r].inputs[0]
        if z <= stop or _one_affine_step(net, z, stop):
            continue
        shape = net.shape[z]
        n = int(np.prod(shape))
        for b in batch_idx:
            dc, dr = _domain(net, lo, hi, x0, eps, b, stop)
            lz = lo[z][b].reshape(-1).clone()
            uz = hi[z][b].reshape(-1).clone()
            for r0 in range(0, n, row_chunk):
                r1 = min(n, r0 + row_chunk)
                rows_p = _identity_rows(shape, 1.0, r0, r1)
                rows_m = _identity_rows(shape, -1.0, r0, r1)
                sel = torch.arange(r0, r1)
                if unstable_only:
                    # rows only for neurons the initial IBP pass leaves unstable; the
                    # others keep their IBP bounds (their relaxation is already exact)
                    keep = ((lo_ibp[z][b].reshape(-1) < 0) & (hi_ibp[z][b].reshape(-1) > 0))[r0:r1]
                    sel, rows_p, rows_m = sel[keep], rows_p[keep], rows_m[keep]
                    if sel.numel() == 0:
                        continue
                lz[sel] = backward(net, lo, hi, b, z, rows_p, stop, dc, dr, decide=decide)
                uz[sel] = -backward(net, lo, hi, b, z, rows_m, stop, dc, dr, decide=decide)
            if intersect:
                lz = torch.maximum(lz, lo_ibp[z][b].reshape(-1))
                uz = torch.minimum(uz, hi_ibp[z][b].reshape(-1))
            lo[z][b] = lz.reshape(shape)
            hi[z][b] = uz.reshape(shape)
    return lo, hi


def spec_bounds_crown(net: Oracle, lo, hi, x0, eps, C, stop: int = 0,
                      batch_idx: Optional[Sequence[int]] = None,
                      decide: Optional[Dict[int, torch.Tensor]] = None):
    """CROWN bounds of C f(x): lb = lb(C) and ub = -lb(-C) per input."""
    C = _t(C)
    B = C.shape[0]
    batch_idx = range(B) if batch_idx is None else batch_idx
    L = len(net.nodes) - 1
    lb = torch.full(C.shape[:2], float("nan"), dtype=f64)
    ub = torch.full(C.shape[:2], float("nan"), dtype=f64)
    for b in batch_idx:
        dc, dr = _domain(net, lo, hi, x0, eps, b, stop)
        lb[b] = backward(net, lo, hi, b, L, C[b], stop, dc, dr, decide=decide)
        ub[b] = -backward(net, lo, hi, b, L, -C[b], stop, dc, dr, decide=decide)
    return lb, ub


def crown_bounds(wl, batch_idx: Optional[Sequence[int]] = None, row_chunk: int = 4096,
                 decide: Optional[Dict[int, torch.Tensor]] = None):
    """Whole pipeline for a workload: IBP, intermediate bounds per wl.intermediate,
    then spec bounds by IBP and by CROWN.  Returns a dict of float64 tensors.
    `decide`: adaptive-slope choices to take at near-ties (see backward())."""
    net = Oracle(wl.nodes)
    lo_ibp, hi_ibp = ibp(net, wl.x0, wl.eps)
    ibp_lb, ibp_ub = spec_bounds_ibp(net, lo_ibp, hi_ibp, wl.C)
    lo, hi = intermediate_bounds(net, wl.x0, wl.eps, wl.intermediate, wl.region_start,
                                 batch_idx, row_chunk, decide)
    stop = wl.region_start if wl.intermediate.startswith("hybrid") else 0
    lb, ub = spec_bounds_crown(net, lo, hi, wl.x0, wl.eps, wl.C, stop, batch_idx, decide)
    return {"ibp_lo": lo_ibp, "ibp_hi": hi_ibp, "ibp_lb": ibp_lb, "ibp_ub": ibp_ub,
            "lo": lo, "hi": hi, "lb": lb, "ub": ub}
