"""Seeded synthetic networks, inputs and margin specifications.

This module is the only code shared by the float64 oracle and the HIP path.
It draws random numbers and lays out shapes; it holds none of the bound
arithmetic (no IBP, no relaxation, no back-substitution).  The one piece of
network arithmetic here is a plain float64 forward pass used to pick each
input's label (the predicted class), from which the margin specification
matrix C is built as data.

Recipe (stated once, used everywhere):
  * every workload has a config id `cfg`; weights come from
    ``numpy.random.default_rng([cfg, 0])`` and inputs from
    ``default_rng([cfg, 1])`` (PCG64), drawn in float64 and cast to float32;
  * weights and biases are drawn layer by layer in node order, the weight
    before the bias;
  * MLP weights ~ N(0, 1/fan_in); conv and residual-net weights ~ N(0, 2/fan_in)
    (He), fan_in = C_in*kh*kw or n_in; biases ~ N(0, 0.01), read as variance
    0.01 (standard deviation 0.1);
  * inputs ~ U[0, 1] per pixel / feature; the L-inf ball around an input is
    not clipped to [0, 1];
  * label = argmax of the float64 forward pass at x0 (lowest index on ties);
    C[b] has one row e_label - e_j per class j != label, ascending j.

These stand in for the networks of "Scaling Neural Network Verification with
Tensor Parallelism and Fully Sharded Data Parallelism" (wide MLPs, CNNs and a
ResNet-large CIFAR-100 model, Sec. 4), whose trained weights and datasets are
not available.

Conv tensors follow the PyTorch convention here: activations [B][C][H][W],
weights [C_out][C_in][kh][kw].  Flatten is in (C, H, W) order.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

__all__ = [
    "Node", "Workload", "NetBuilder", "forward", "margin_specs",
    "mlp", "cnn", "resnet", "wide", "WIDE_NAME", "config", "CONFIG_NAMES", "tiny_mlp",
]


@dataclass
class Node:
    op: str                      # input | linear | conv | relu | add | gap | flatten
    inputs: Tuple[int, ...]      # producer node indices (topological order)
    shape: Tuple[int, ...]       # output shape: (n,) or (C, H, W)
    weight: Optional[np.ndarray] = None   # linear [out][in]; conv [O][I][kh][kw]; float32
    bias: Optional[np.ndarray] = None     # [out] / [O]; float32
    stride: int = 1
    pad: int = 0

    @property
    def size(self) -> int:
        return int(np.prod(self.shape))


@dataclass
class Workload:
    name: str
    cfg: int
    nodes: List[Node]
    x0: np.ndarray               # [B][*input shape] float32
    eps: np.float32
    labels: np.ndarray           # [B] int64
    C: np.ndarray                # [B][m][n_out] float32
    intermediate: str            # "crown" | "ibp" | "hybrid"
    region_start: Optional[int] = None   # hybrid: node whose IBP box is the domain
    alpha_steps: int = 0
    alpha_lr: float = 0.1
    seeds: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.x0.shape[0])

    @property
    def m(self) -> int:
        return int(self.C.shape[1])

    def subset(self, idx) -> "Workload":
        idx = np.asarray(idx)
        return Workload(self.name, self.cfg, self.nodes, self.x0[idx].copy(), self.eps,
                        self.labels[idx].copy(), self.C[idx].copy(), self.intermediate,
                        self.region_start, self.alpha_steps, self.alpha_lr, dict(self.seeds))


class NetBuilder:
    """Appends nodes in topological order, drawing parameters from one generator."""

    def __init__(self, rng: np.random.Generator, init: str, draw32: bool = False):
        self.rng = rng
        self.init = init          # "lecun": N(0, 1/fan_in); "he": N(0, 2/fan_in)
        self.draw32 = draw32      # draw directly in float32 (same distributions; for > 1e9 weights)
        self.nodes: List[Node] = []

    def _add(self, node: Node) -> int:
        self.nodes.append(node)
        return len(self.nodes) - 1

    def _w(self, shape, fan_in, zero=False):
        var = (1.0 if self.init == "lecun" else 2.0) / fan_in
        if self.draw32:
            w = self.rng.standard_normal(shape, dtype=np.float32)
            w *= np.float32(np.sqrt(var))
            b = self.rng.standard_normal(shape[0], dtype=np.float32) * np.float32(0.1)
            return w, b
        w = self.rng.standard_normal(shape) * np.sqrt(var)
        b = self.rng.standard_normal(shape[0]) * 0.1
        if zero:
            w = np.zeros(shape)
            b = np.zeros(shape[0])
        return w.astype(np.float32), b.astype(np.float32)

    def input(self, shape) -> int:
        return self._add(Node("input", (), tuple(shape)))

    def linear(self, x: int, n_out: int, zero=False) -> int:
        n_in = self.nodes[x].size
        assert len(self.nodes[x].shape) == 1, "linear needs a flat input"
        w, b = self._w((n_out, n_in), n_in, zero)
        return self._add(Node("linear", (x,), (n_out,), w, b))

    def conv(self, x: int, c_out: int, k=3, stride=1, pad=1, zero=False) -> int:
        c, h, w_ = self.nodes[x].shape
        w, b = self._w((c_out, c, k, k), c * k * k, zero)
        ho = (h + 2 * pad - k) // stride + 1
        wo = (w_ + 2 * pad - k) // stride + 1
        return self._add(Node("conv", (x,), (c_out, ho, wo), w, b, stride, pad))

    def relu(self, x: int) -> int:
        return self._add(Node("relu", (x,), self.nodes[x].shape))

    def add(self, a: int, b: int) -> int:
        assert self.nodes[a].shape == self.nodes[b].shape
        return self._add(Node("add", (a, b), self.nodes[a].shape))

    def gap(self, x: int) -> int:
        return self._add(Node("gap", (x,), (self.nodes[x].shape[0],)))

    def flatten(self, x: int) -> int:
        return self._add(Node("flatten", (x,), (self.nodes[x].size,)))


# ---------------------------------------------------------------------------
# plain float64 forward pass (labels only)


def _conv_fwd(x, w, b, stride, pad):
    bsz, c, h, wd = x.shape
    o, _, kh, kw = w.shape
    ho = (h + 2 * pad - kh) // stride + 1
    wo = (wd + 2 * pad - kw) // stride + 1
    xp = np.zeros((bsz, c, h + 2 * pad, wd + 2 * pad))
    xp[:, :, pad:pad + h, pad:pad + wd] = x
    out = np.zeros((bsz, o, ho, wo))
    for ky in range(kh):
        for kx in range(kw):
            patch = xp[:, :, ky:ky + stride * (ho - 1) + 1:stride, kx:kx + stride * (wo - 1) + 1:stride]
            out += np.einsum("oi,bihw->bohw", w[:, :, ky, kx].astype(np.float64), patch)
    return out + b.astype(np.float64)[None, :, None, None]


def forward(nodes: List[Node], x: np.ndarray) -> List[np.ndarray]:
    """Float64 values of every node for a batch x [B][*input shape]."""
    vals: List[np.ndarray] = []
    for nd in nodes:
        if nd.op == "input":
            v = x.astype(np.float64)
        elif nd.op == "linear":
            v = vals[nd.inputs[0]] @ nd.weight.astype(np.float64).T + nd.bias.astype(np.float64)
        elif nd.op == "conv":
            v = _conv_fwd(vals[nd.inputs[0]], nd.weight, nd.bias, nd.stride, nd.pad)
        elif nd.op == "relu":
            v = np.maximum(vals[nd.inputs[0]], 0.0)
        elif nd.op == "add":
            v = vals[nd.inputs[0]] + vals[nd.inputs[1]]
        elif nd.op == "gap":
            v = vals[nd.inputs[0]].mean(axis=(2, 3))
        elif nd.op == "flatten":
            src = vals[nd.inputs[0]]
            v = src.reshape(src.shape[0], -1)
        else:
            raise ValueError(nd.op)
        vals.append(v)
    return vals


def margin_specs(nodes: List[Node], x0: np.ndarray):
    """labels [B] and C [B][n_out-1][n_out]: rows e_label - e_j, j != label ascending."""
    logits = forward(nodes, x0)[-1]
    labels = np.argmax(logits, axis=1)
    n_out = logits.shape[1]
    C = np.zeros((x0.shape[0], n_out - 1, n_out), dtype=np.float32)
    for b, lab in enumerate(labels):
        others = [j for j in range(n_out) if j != lab]
        for i, j in enumerate(others):
            C[b, i, lab] = 1.0
            C[b, i, j] = -1.0
    return labels.astype(np.int64), C


# ---------------------------------------------------------------------------
# architecture families


def mlp(widths, batch, eps, cfg, intermediate="crown", name=None, init="lecun") -> Workload:
    rng_w = np.random.default_rng([cfg, 0])
    rng_x = np.random.default_rng([cfg, 1])
    nb = NetBuilder(rng_w, init)
    x = nb.input((widths[0],))
    for i, n in enumerate(widths[1:]):
        x = nb.linear(x, n)
        if i < len(widths) - 2:
            x = nb.relu(x)
    x0 = rng_x.random((batch, widths[0])).astype(np.float32)
    labels, C = margin_specs(nb.nodes, x0)
    return Workload(name or "mlp_" + "-".join(map(str, widths)), cfg, nb.nodes, x0, np.float32(eps),
                    labels, C, intermediate, seeds={"weights": [cfg, 0], "inputs": [cfg, 1]})


WIDE_NAME = "wide_4096-262144-100_b8_ibp"


def wide(batch=8, eps=2.0 / 255, n_in=4096, width=262144, n_out=100, cfg=6, name=None) -> Workload:
    """One hidden ReLU layer n_in-width-n_out, the shape of the page's widest networks
    (Sec. 1: a 262 144-wide layer whose weights exceed 4 GB in fp32).  Interval bounds
    over it are limited by reading the weights once: the memory-bound IBP case.
    Same recipe as `mlp` (N(0, 1/fan_in) weights, N(0, 0.01) biases, U[0,1] inputs),
    drawn directly in float32 so the 1.07e9 weights take seconds."""
    rng_w = np.random.default_rng([cfg, 0])
    rng_x = np.random.default_rng([cfg, 1])
    nb = NetBuilder(rng_w, "lecun", draw32=True)
    x = nb.input((n_in,))
    x = nb.relu(nb.linear(x, width))
    nb.linear(x, n_out)
    x0 = rng_x.random((batch, n_in)).astype(np.float32)
    labels, C = margin_specs(nb.nodes, x0)
    return Workload(name or f"wide_{n_in}-{width}-{n_out}_b{batch}_ibp", cfg, nb.nodes, x0, np.float32(eps),
                    labels, C, "ibp", seeds={"weights": [cfg, 0], "inputs": [cfg, 1]})


def cnn(batch, eps, cfg, convs=((64, 1), (64, 2), (128, 1), (128, 2)), fcs=(512, 100),
        in_shape=(3, 32, 32), intermediate="ibp", name=None, x_rng_draw=None) -> Workload:
    """conv3x3 (pad 1) + ReLU per (channels, stride), flatten, FC layers (ReLU except the last)."""
    rng_w = np.random.default_rng([cfg, 0])
    rng_x = np.random.default_rng([cfg, 1])
    nb = NetBuilder(rng_w, "he")
    x = nb.input(in_shape)
    for c, s in convs:
        x = nb.relu(nb.conv(x, c, 3, s, 1))
    x = nb.flatten(x)
    for i, n in enumerate(fcs):
        x = nb.linear(x, n)
        if i < len(fcs) - 1:
            x = nb.relu(x)
    n_draw = batch if x_rng_draw is None else x_rng_draw
    x0 = rng_x.random((n_draw,) + tuple(in_shape)).astype(np.float32)[:batch]
    labels, C = margin_specs(nb.nodes, x0)
    return Workload(name or "cnn", cfg, nb.nodes, x0, np.float32(eps), labels, C, intermediate,
                    seeds={"weights": [cfg, 0], "inputs": [cfg, 1]})


def resnet(batch, eps, cfg, widths=(64, 128, 256), blocks=(3, 3, 2), n_out=100,
           in_shape=(3, 32, 32), name=None, zero_branch_block: Optional[int] = None) -> Workload:
    """Stem conv3x3 + ReLU; stages of basic blocks y = ReLU(x + conv_b(ReLU(conv_a(x)))).

    The first block of every stage after the first has conv_a with stride 2 and a
    1x1 stride-2 projection on the skip path.  Then global average pool and FC.
    The CROWN region is the last stage: its input node is the hybrid domain.
    """
    rng_w = np.random.default_rng([cfg, 0])
    rng_x = np.random.default_rng([cfg, 1])
    nb = NetBuilder(rng_w, "he")
    x = nb.input(in_shape)
    x = nb.relu(nb.conv(x, widths[0], 3, 1, 1))
    region_start = None
    blk = 0
    for si, (wd, nbk) in enumerate(zip(widths, blocks)):
        if si == len(widths) - 1:
            region_start = x
        for bi in range(nbk):
            down = si > 0 and bi == 0
            zero = zero_branch_block == blk
            a = nb.relu(nb.conv(x, wd, 3, 2 if down else 1, 1, zero=zero))
            bb = nb.conv(a, wd, 3, 1, 1, zero=zero)
            skip = nb.conv(x, wd, 1, 2, 0) if down else x
            x = nb.relu(nb.add(bb, skip))
            blk += 1
    x = nb.gap(x)
    x = nb.linear(x, n_out)
    x0 = rng_x.random((batch,) + tuple(in_shape)).astype(np.float32)
    labels, C = margin_specs(nb.nodes, x0)
    return Workload(name or "resnet", cfg, nb.nodes, x0, np.float32(eps), labels, C, "hybrid",
                    region_start=region_start, seeds={"weights": [cfg, 0], "inputs": [cfg, 1]})


CONFIG_NAMES = {
    1: "mlp_784-100-100-10_b16_crown",
    2: "mlp_3072-1024x5-100_b64_crown",
    3: "cnn_c64s1-c64s2-c128s1-c128s2-fc512-fc100_b32_ibp",
    4: "cnn_alpha_crown_b16_20steps",
    5: "resnet_64-128-256_blocks332_b32_hybrid",
}


def config(cfg: int, batch: Optional[int] = None) -> Workload:
    """The five workloads the measurements are quoted on (optionally a smaller batch).

    A smaller batch takes the first `batch` inputs of the full draw, so sampled
    parity at full size and the full run see the same inputs.
    """
    if cfg == 1:
        w = mlp([784, 100, 100, 10], 16, 0.01, 1, "crown", CONFIG_NAMES[1])
    elif cfg == 2:
        w = mlp([3072, 1024, 1024, 1024, 1024, 1024, 100], 64, 2.0 / 255, 2, "crown", CONFIG_NAMES[2])
    elif cfg == 3:
        w = cnn(32, 1.0 / 255, 3, name=CONFIG_NAMES[3])
    elif cfg == 4:
        # same weights and the first 16 of the inputs of config 3, larger ball
        w = cnn(16, 2.0 / 255, 3, name=CONFIG_NAMES[4], x_rng_draw=32)
        w.cfg = 4
        w.alpha_steps = 20
        w.alpha_lr = 0.1
    elif cfg == 5:
        w = resnet(32, 1.0 / 255, 5, name=CONFIG_NAMES[5])
    else:
        raise ValueError(cfg)
    if batch is not None and batch < w.batch:
        w = w.subset(np.arange(batch))
    return w


def tiny_mlp(widths, eps, seed, batch=1, init="lecun") -> Workload:
    """Small MLP for brute-force checks (same recipe, config id = seed + 1000)."""
    return mlp(list(widths), batch, eps, 1000 + seed, "crown", "tiny_mlp", init)
