"""Write the float64 oracle's bounds for full-size workloads (tests/golden/full_size_*.npz).

The oracle needs minutes per input at these sizes, so its results are computed
once here and compared with the GPU in tests/test_gpu_full_size.py.  This
script calls only the oracle and the seeded workload generators.  Stored per
workload: the inputs used, the spec bounds by CROWN and by IBP, and for every
CROWN-refined ReLU input a seeded sample of neurons (flat (C, H, W) index) with
their lower and upper bounds, plus a fingerprint of the seeded parameters so a
change of the recipe is detected.

  python tests/golden/make_full_size.py [name ...]
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import workloads as wk  # noqa: E402
from oracle import crown_bounds  # noqa: E402

# name: (config id, intermediate method or None for the workload's own, inputs, neurons sampled per layer)
CASES = {
    "resnet_hybrid": (5, None, [0, 1], 2048),
    "cnn_crown": (3, "crown", [0], 2048),
}


def fingerprint(wl):
    """Sums of the float32 parameters and inputs in float64 (detects a changed recipe)."""
    s = [float(np.sum(np.abs(n.weight.astype(np.float64)))) for n in wl.nodes if n.weight is not None]
    s += [float(np.sum(n.bias.astype(np.float64))) for n in wl.nodes if n.bias is not None]
    return np.array(s + [float(np.sum(wl.x0.astype(np.float64)))])


def refined_layers(wl):
    """ReLU inputs whose bounds the oracle refines by CROWN (not one affine step from the domain)."""
    stop = wl.region_start if wl.intermediate.startswith("hybrid") else 0
    out = []
    for nd in wl.nodes:
        if nd.op != "relu":
            continue
        z = nd.inputs[0]
        zn = wl.nodes[z]
        if z <= stop:
            continue
        if zn.op in ("linear", "conv"):
            i = zn.inputs[0]
            while wl.nodes[i].op == "flatten":
                i = wl.nodes[i].inputs[0]
            if i == stop:
                continue
        out.append(z)
    return out


def make(name):
    cfg, method, inputs, n_sample = CASES[name]
    wl = wk.config(cfg, batch=max(inputs) + 1)
    if method:
        wl.intermediate = method
    t0 = time.time()
    ref = crown_bounds(wl, batch_idx=inputs)
    print(f"{name}: oracle {time.time() - t0:.0f} s", flush=True)
    rng = np.random.default_rng([cfg, 7])
    data = {"inputs": np.array(inputs), "fingerprint": fingerprint(wl), "intermediate": np.array(wl.intermediate)}
    for key in ("lb", "ub", "ibp_lb", "ibp_ub"):
        data[key] = ref[key][inputs].numpy()
    layers = refined_layers(wl)
    data["layers"] = np.array(layers)
    for z in layers:
        n = wl.nodes[z].size
        idx = np.sort(rng.choice(n, min(n, n_sample), replace=False))
        data[f"idx_{z}"] = idx
        data[f"lo_{z}"] = ref["lo"][z][inputs].reshape(len(inputs), -1)[:, idx].numpy()
        data[f"hi_{z}"] = ref["hi"][z][inputs].reshape(len(inputs), -1)[:, idx].numpy()
    np.savez_compressed(os.path.join(HERE, f"full_size_{name}.npz"), **data)


if __name__ == "__main__":
    for n in (sys.argv[1:] or list(CASES)):
        make(n)
