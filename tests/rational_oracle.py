"""Exact rational-arithmetic reference for IBP, CROWN and alpha-CROWN evaluation.

Test infrastructure: it exists only to pin the float64 oracle (``oracle/``) on
tiny networks.  It is a separate implementation written with plain Python
loops over ``fractions.Fraction`` values (no torch, no numpy arithmetic), so
every result is the exact value of the method on the float32 parameters.
IBP, CROWN and the alpha-CROWN evaluation use only +, -, *, /, max, abs and
sign, so nothing here is rounded.

The method: "Scaling Neural Network Verification with Tensor Parallelism and
Fully Sharded Data Parallelism" names IBP, CROWN and alpha-CROWN (Sec. 1), the
relaxation slopes from intermediate bounds and the IBP substitute for them
(Sec. 2.1), bound propagation through convolutions (Sec. 2.2) and the alpha
slopes (Sec. 3, Sec. 4.3).  The arithmetic is the standard definition of each
algorithm: centre/radius interval propagation; the adaptive ReLU relaxation
(inactive if u <= 0, else active if l >= 0, else slope s = u/(u-l), offset
-s*l, lower slope 1 when u >= -l and 0 otherwise, or alpha); back-substitution
of linear bounds to a box domain; min over the box of a linear function =
A c - |A| r + beta.

Tensors are flat lists in the networks' (C, H, W) order.
"""
from __future__ import annotations

from fractions import Fraction
from typing import Dict, List, Optional

import numpy as np

ZERO = Fraction(0)
ONE = Fraction(1)


def exact(values) -> List[Fraction]:
    """Exact rationals of float32 / float64 values (the binary value itself)."""
    return [Fraction(float(v)) for v in np.asarray(values, dtype=np.float64).reshape(-1)]


class ExactNet:
    def __init__(self, nodes):
        self.nodes = nodes
        self.size = [int(np.prod(n.shape)) for n in nodes]
        self.W = []
        self.b = []
        for n in nodes:
            if n.op in ("linear", "conv"):
                self.W.append(np.asarray(n.weight, dtype=np.float64))
                self.b.append(exact(n.bias))
            else:
                self.W.append(None)
                self.b.append(None)
        self._wq: Dict[int, Dict] = {}

    def _weights(self, k):
        # cached exact weights of node k, indexed like the float array
        if k not in self._wq:
            w = self.W[k]
            self._wq[k] = {idx: Fraction(float(v)) for idx, v in np.ndenumerate(w)}
        return self._wq[k]

    # --- the affine map of node k without its bias, and its transpose
    def _taps(self, k):
        """Yields (out_index, in_index, weight index) of every product of node k."""
        nd = self.nodes[k]
        if nd.op == "linear":
            n_out, n_in = self.W[k].shape
            for o in range(n_out):
                for i in range(n_in):
                    yield o, i, (o, i)
            return
        co, ci, kh, kw = self.W[k].shape
        _, H, Wd = self.nodes[nd.inputs[0]].shape
        _, Ho, Wo = nd.shape
        s, p = nd.stride, nd.pad
        for o in range(co):
            for y in range(Ho):
                for x in range(Wo):
                    out = (o * Ho + y) * Wo + x
                    for i in range(ci):
                        for ky in range(kh):
                            yy = y * s + ky - p
                            if yy < 0 or yy >= H:
                                continue
                            for kx in range(kw):
                                xx = x * s + kx - p
                                if xx < 0 or xx >= Wd:
                                    continue
                                yield out, (i * H + yy) * Wd + xx, (o, i, ky, kx)

    def forward_map(self, k, v, use_abs=False):
        wq = self._weights(k)
        out = [ZERO] * self.size[k]
        for o, i, w in self._taps(k):
            c = wq[w]
            out[o] += (abs(c) if use_abs else c) * v[i]
        return out

    def transpose_map(self, k, lam):
        wq = self._weights(k)
        res = [ZERO] * self.size[self.nodes[k].inputs[0]]
        for o, i, w in self._taps(k):
            if lam[o] != 0:
                res[i] += lam[o] * wq[w]
        return res

    def bias_dot(self, k, lam):
        """sum over the outputs of node k of lam * bias (conv: bias per channel)."""
        nd = self.nodes[k]
        if nd.op == "linear":
            return sum((l * b for l, b in zip(lam, self.b[k])), ZERO)
        _, Ho, Wo = nd.shape
        per = Ho * Wo
        return sum((lam[j] * self.b[k][j // per] for j in range(len(lam))), ZERO)

    def add_bias(self, k, v):
        nd = self.nodes[k]
        if nd.op == "linear":
            return [a + b for a, b in zip(v, self.b[k])]
        _, Ho, Wo = nd.shape
        per = Ho * Wo
        return [v[j] + self.b[k][j // per] for j in range(len(v))]


def ibp(net: ExactNet, x0, eps) -> (List[List[Fraction]], List[List[Fraction]]):
    """Interval bounds of every node for one input (x0 flat, eps a float32 scalar)."""
    x = exact(x0)
    e = Fraction(float(np.float32(eps)))
    lo, hi = [], []
    for k, nd in enumerate(net.nodes):
        if nd.op == "input":
            lo.append([v - e for v in x])
            hi.append([v + e for v in x])
            continue
        i = nd.inputs[0]
        if nd.op in ("linear", "conv"):
            c = [(a + b) / 2 for a, b in zip(lo[i], hi[i])]
            r = [(b - a) / 2 for a, b in zip(lo[i], hi[i])]
            cc = net.add_bias(k, net.forward_map(k, c))
            rr = net.forward_map(k, r, use_abs=True)
            lo.append([a - b for a, b in zip(cc, rr)])
            hi.append([a + b for a, b in zip(cc, rr)])
        elif nd.op == "relu":
            lo.append([max(v, ZERO) for v in lo[i]])
            hi.append([max(v, ZERO) for v in hi[i]])
        elif nd.op == "add":
            j = nd.inputs[1]
            lo.append([a + b for a, b in zip(lo[i], lo[j])])
            hi.append([a + b for a, b in zip(hi[i], hi[j])])
        elif nd.op == "gap":
            C, H, W = net.nodes[i].shape
            P = H * W
            lo.append([sum(lo[i][c * P:(c + 1) * P], ZERO) / P for c in range(C)])
            hi.append([sum(hi[i][c * P:(c + 1) * P], ZERO) / P for c in range(C)])
        elif nd.op == "flatten":
            lo.append(list(lo[i]))
            hi.append(list(hi[i]))
        else:
            raise ValueError(nd.op)
    return lo, hi


def spec_ibp(net: ExactNet, lo, hi, C):
    """IBP bounds of C f(x) with C folded into the last Linear."""
    L = len(net.nodes) - 1
    i = net.nodes[L].inputs[0]
    Wl = net._weights(L)
    n_out, n_in = net.W[L].shape
    Cq = [exact(row) for row in np.asarray(C)]
    out_lo, out_hi = [], []
    for row in Cq:
        wf = [sum((row[o] * Wl[(o, j)] for o in range(n_out)), ZERO) for j in range(n_in)]
        bf = sum((row[o] * net.b[L][o] for o in range(n_out)), ZERO)
        c = sum(((a + b) / 2 * w for a, b, w in zip(lo[i], hi[i], wf)), ZERO) + bf
        r = sum(((b - a) / 2 * abs(w) for a, b, w in zip(lo[i], hi[i], wf)), ZERO)
        out_lo.append(c - r)
        out_hi.append(c + r)
    return out_lo, out_hi


def relax(l: Fraction, u: Fraction, alpha: Optional[Fraction] = None):
    """(lower slope, upper slope, upper offset) of ReLU on [l, u]."""
    if u <= 0:
        return ZERO, ZERO, ZERO
    if l >= 0:
        return ONE, ONE, ZERO
    s = u / (u - l)
    a = alpha if alpha is not None else (ONE if u >= -l else ZERO)
    return a, s, -s * l


def lower_bound(net: ExactNet, lo, hi, start: int, row: List[Fraction], stop: int, dom_c, dom_r,
                alpha: Optional[Dict[int, List[Fraction]]] = None) -> Fraction:
    """min over the relaxed network between `stop` (box dom_c +- dom_r) and `start`
    of row . (node start), by back-substitution."""
    pending: Dict[int, List[Fraction]] = {start: list(row)}
    beta = ZERO
    for k in range(start, stop, -1):
        if k not in pending:
            continue
        L = pending.pop(k)
        nd = net.nodes[k]

        def push(t, vec):
            if t in pending:
                pending[t] = [a + b for a, b in zip(pending[t], vec)]
            else:
                pending[t] = vec
        if nd.op in ("linear", "conv"):
            beta += net.bias_dot(k, L)
            push(nd.inputs[0], net.transpose_map(k, L))
        elif nd.op == "relu":
            z = nd.inputs[0]
            out = []
            for j, v in enumerate(L):
                a, s, t = relax(lo[z][j], hi[z][j], None if alpha is None else alpha[k][j])
                if v >= 0:
                    out.append(v * a)
                else:
                    out.append(v * s)
                    beta += v * t
            push(z, out)
        elif nd.op == "add":
            push(nd.inputs[0], list(L))
            push(nd.inputs[1], list(L))
        elif nd.op == "gap":
            C, H, W = net.nodes[nd.inputs[0]].shape
            P = H * W
            push(nd.inputs[0], [L[j // P] / P for j in range(C * P)])
        elif nd.op == "flatten":
            push(nd.inputs[0], list(L))
        else:
            raise ValueError(nd.op)
    L = pending.pop(stop)
    assert not pending
    return sum((v * c - abs(v) * r for v, c, r in zip(L, dom_c, dom_r)), ZERO) + beta


def _box(lo, hi, x0, eps, net, stop):
    if net.nodes[stop].op == "input":
        e = Fraction(float(np.float32(eps)))
        x = exact(x0)
        return x, [e] * len(x)
    return ([(a + b) / 2 for a, b in zip(lo[stop], hi[stop])], [(b - a) / 2 for a, b in zip(lo[stop], hi[stop])])


def _one_affine_step_from(net, z, stop):
    nd = net.nodes[z]
    if nd.op not in ("linear", "conv"):
        return False
    i = nd.inputs[0]
    while net.nodes[i].op == "flatten":
        i = net.nodes[i].inputs[0]
    return i == stop


def bounds(wl, b: int, mode: str):
    """IBP, intermediate bounds by `mode` (ibp | crown | hybrid, optionally +ibp and/or
    +unstable) and the spec bounds by IBP and CROWN for input b of a workload; all
    exact.  +ibp: each new bound is clipped to the first IBP pass's; +unstable: only
    neurons that IBP pass leaves with l < 0 < u get new bounds."""
    net = ExactNet(wl.nodes)
    x0 = wl.x0[b].reshape(-1)
    lo, hi = ibp(net, x0, wl.eps)
    ibp_lb, ibp_ub = spec_ibp(net, lo, hi, wl.C[b])
    base, *flags = mode.split("+")
    suffix = "ibp" if "ibp" in flags else ""
    only_unstable = "unstable" in flags
    ibp_lo = [list(v) for v in lo]
    ibp_hi = [list(v) for v in hi]
    stop = 0
    if base != "ibp":
        stop = 0 if base == "crown" else wl.region_start
        for k, nd in enumerate(wl.nodes):
            if nd.op != "relu":
                continue
            z = nd.inputs[0]
            if z <= stop or _one_affine_step_from(net, z, stop):
                continue
            dc, dr = _box(lo, hi, x0, wl.eps, net, stop)
            n = net.size[z]
            new_lo, new_hi = [], []
            for j in range(n):
                if only_unstable and not (ibp_lo[z][j] < 0 < ibp_hi[z][j]):
                    new_lo.append(lo[z][j])
                    new_hi.append(hi[z][j])
                    continue
                e = [ZERO] * n
                e[j] = ONE
                lj = lower_bound(net, lo, hi, z, e, stop, dc, dr)
                e[j] = -ONE
                uj = -lower_bound(net, lo, hi, z, e, stop, dc, dr)
                if suffix == "ibp":
                    lj = max(lj, ibp_lo[z][j])
                    uj = min(uj, ibp_hi[z][j])
                new_lo.append(lj)
                new_hi.append(uj)
            lo[z], hi[z] = new_lo, new_hi
    dc, dr = _box(lo, hi, x0, wl.eps, net, stop)
    L = len(wl.nodes) - 1
    lb, ub = [], []
    for row in np.asarray(wl.C[b]):
        r = exact(row)
        lb.append(lower_bound(net, lo, hi, L, r, stop, dc, dr))
        ub.append(-lower_bound(net, lo, hi, L, [-v for v in r], stop, dc, dr))
    return {"lo": lo, "hi": hi, "ibp_lb": ibp_lb, "ibp_ub": ibp_ub, "lb": lb, "ub": ub}


def row_lower_bounds(wl, lo, hi, b: int, start: int, rows, alpha: Dict[int, np.ndarray], stop: int = 0):
    """Lower bounds of arbitrary rows over node `start` with per-row lower slopes:
    alpha[k] [R][n] for the ReLU nodes k between stop and start."""
    net = ExactNet(wl.nodes)
    x0 = wl.x0[b].reshape(-1)
    dc, dr = _box(lo, hi, x0, wl.eps, net, stop)
    out = []
    for i, row in enumerate(np.asarray(rows)):
        al = {k: exact(np.asarray(v)[i]) for k, v in alpha.items()}
        out.append(lower_bound(net, lo, hi, start, exact(row), stop, dc, dr, al))
    return out


def alpha_lower_bounds(wl, lo, hi, b: int, alpha: Dict[int, np.ndarray], stop: int = 0):
    """Spec lower bounds of input b with the given lower slopes: alpha[k] [m][n] per
    ReLU node k (float values, taken exactly), bounds lo/hi exact lists per node."""
    net = ExactNet(wl.nodes)
    x0 = wl.x0[b].reshape(-1)
    dc, dr = _box(lo, hi, x0, wl.eps, net, stop)
    L = len(wl.nodes) - 1
    out = []
    for i, row in enumerate(np.asarray(wl.C[b])):
        al = {k: exact(np.asarray(v)[i]) for k, v in alpha.items()}
        out.append(lower_bound(net, lo, hi, L, exact(row), stop, dc, dr, al))
    return out
