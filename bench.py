"""Benchmark of the bound-propagation hot path on one MI355X.

One step = one whole bound computation for one batch: IBP of every node, the
intermediate bounds of every ReLU input (CROWN back-substitution per layer for
the MLP workloads), and the spec bounds by IBP and by CROWN.  Inputs are
resident in HBM before the timed region.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload N] [--no-cpu]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CROWN bound-propagation TFLOP/s (fp32, % MFMA peak) + verified specs/sec"
PEAK_FP32_MFMA_TFLOPS = 157.3   # MI355X dense fp32 matrix peak (AMD public spec)


def _mac_per_row(nd, nodes):
    """Forward multiply-adds of one affine node for one row of Lambda."""
    if nd.op == "linear":
        return nd.weight.shape[0] * nd.weight.shape[1]
    co, ci, kh, kw = nd.weight.shape
    return co * ci * kh * kw * nd.shape[1] * nd.shape[2]


def _active(nodes, start, stop):
    act, stack = set(), [start]
    while stack:
        k = stack.pop()
        if k in act or k < stop:
            continue
        act.add(k)
        if k != stop and k != 0:
            stack.extend(nodes[k].inputs)
    return act


def _src(nodes, k):
    while nodes[k].op == "flatten":
        k = nodes[k].inputs[0]
    return k


def _identity_consumers(nodes, z):
    """Affine nodes that receive identity rows over z directly (z itself, or the
    affine inputs of an ADD z): their step is a copy of the weight footprint."""
    nd = nodes[z]
    if nd.op in ("linear", "conv"):
        return {z}
    if nd.op == "add":
        out = set()
        for i in nd.inputs:
            out |= _identity_consumers(nodes, i)
        return out
    return set()


def _footprint_macs(nodes, z, stop):
    """Multiply-adds of the identity rows over conv node z (one row per neuron, both
    signs counted by the caller) when each row is carried on its footprint window
    through a conv -> ReLU -> conv chain down to `stop`: at every conv only the
    output cells inside both the row's window and the image count.  None if the
    back-substitution from z is not such a chain."""
    nd = nodes[z]
    if nd.op != "conv":
        return None
    c_z, h_z, w_z = nd.shape
    total = 0.0
    k, wh, ww, sy, oy, sx, ox = z, 1, 1, 1, 0, 1, 0
    while True:
        nk = nodes[k]
        if nk.op != "conv":
            return None
        co, ci, kh, kw = nk.weight.shape
        _, ho, wo = nk.shape
        # cells of k's output window that exist, summed over the start node's pixels
        ys = np.arange(h_z)[:, None] * sy + oy + np.arange(wh)[None, :]
        xs = np.arange(w_z)[:, None] * sx + ox + np.arange(ww)[None, :]
        ny = ((ys >= 0) & (ys < ho)).sum(1)
        nx = ((xs >= 0) & (xs < wo)).sum(1)
        cells = float(ny.sum()) * float(nx.sum())      # sum over (py, px) of ny[py] * nx[px]
        if k != z:   # the first step is a copy of the weight footprint: free
            total += c_z * cells * co * ci * kh * kw
        t = nk.inputs[0]
        wh, ww = (wh - 1) * nk.stride + kh, (ww - 1) * nk.stride + kw
        sy, oy = sy * nk.stride, oy * nk.stride - nk.pad
        sx, ox = sx * nk.stride, ox * nk.stride - nk.pad
        if t == stop:
            return total
        if nodes[t].op != "relu":
            return None
        k = nodes[t].inputs[0]


def algorithmic_flops(wl):
    """FLOPs the method itself performs for the whole batch (no padding, no tile waste):
    2 * rows * multiply-adds of each affine node a row of Lambda passes through; the
    first step of identity rows (a copy of the weight footprint) costs nothing; IBP
    is two passes (centre and radius) of the forward multiply-adds."""
    nodes, B, m = wl.nodes, wl.batch, wl.m
    total = {"ibp": 0.0, "intermediate": 0.0, "spec": 0.0}
    for nd in nodes:
        if nd.op in ("linear", "conv"):
            total["ibp"] += 2 * 2 * _mac_per_row(nd, nodes) * B
    L = len(nodes) - 1
    # spec IBP: C folded into the last Linear
    total["spec"] += 2 * (2 * m * B) * _mac_per_row(nodes[L], nodes)
    stop = wl.region_start if wl.intermediate.startswith("hybrid") else 0
    if wl.intermediate != "ibp":
        for r, nd in enumerate(nodes):
            if nd.op != "relu":
                continue
            z = nd.inputs[0]
            zn = nodes[z]
            if z <= stop or (zn.op in ("linear", "conv") and _src(nodes, zn.inputs[0]) == stop):
                continue
            rows = 2 * zn.size * B
            fp = _footprint_macs(nodes, z, stop)
            if fp is not None:
                # rows on footprint windows: count only the cells that exist
                total["intermediate"] += 2 * 2 * B * fp
                continue
            free = _identity_consumers(nodes, z)
            for k in _active(nodes, z, stop):
                if nodes[k].op not in ("linear", "conv") or k in free:
                    continue
                total["intermediate"] += 2 * rows * _mac_per_row(nodes[k], nodes)
    rows = 2 * m * B
    for k in _active(nodes, L, stop):
        if nodes[k].op in ("linear", "conv"):
            total["spec"] += 2 * rows * _mac_per_row(nodes[k], nodes)
    if wl.alpha_steps:
        # alpha loop: steps+1 evaluations of the m lower rows (spec fold + every
        # affine node) and `steps` adjoints (forward through every affine node but the last)
        rows = m * B
        ev = sum(2 * rows * _mac_per_row(nodes[k], nodes) for k in _active(nodes, L, 0)
                 if nodes[k].op in ("linear", "conv"))
        adj = ev - 2 * rows * _mac_per_row(nodes[L], nodes)
        total["alpha"] = (wl.alpha_steps + 1) * ev + wl.alpha_steps * adj
    total["all"] = sum(v for k, v in total.items())
    return total


def cpu_baseline(wl, flops_total, budget_s=12.0):
    """The float64 oracle on the host cores over the first k inputs (k grows until
    about budget_s of CPU work), scaled to TFLOP/s of the same algorithmic work."""
    import torch
    from oracle import crown_bounds
    k, elapsed = 0, 0.0
    while k < wl.batch and elapsed < budget_s:
        t0 = time.perf_counter()
        crown_bounds(wl, batch_idx=[k])
        elapsed += time.perf_counter() - t0
        k += 1
    per_input = flops_total / wl.batch
    return {"value": per_input * k / elapsed / 1e12, "unit": "TFLOP/s", "cores": torch.get_num_threads(),
            "kind": "oracle", "specs_per_s": k * wl.m / elapsed,
            "sample": f"first {k} of {wl.batch} inputs, all {wl.m} specs, float64 torch-CPU oracle, {elapsed:.1f} s"}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_backsub_traffic_mlp3072.txt")
GEMM_SOURCE = os.path.join(ROOT, "linear_bound_propagation_amd", "csrc", "vb_gemm.hip")


def measured_traffic(workload_name):
    """HBM bytes per back-substitution GEMM launch from the committed counter summary,
    or None when it is missing, for another workload, or taken on a different kernel source."""
    import hashlib
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    sha = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    if kv.get("kernel_source_sha256") != sha or kv.get("workload") != workload_name:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_probe(nbytes):
    """A plain device-to-device copy of `nbytes` (read + write), run a few times:
    the calibration kernel for the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    x = torch.empty(nbytes // 4, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "launches": 3}))


PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E (AMD public spec)


def _time_calls(fn, reps, warmup=2):
    """Average ms per call of fn() over reps calls, HIP events on torch's current stream
    (the stream the library launches on)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        fn()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def hbm_kernels(reps=20):
    """The memory-bound kernels, timed live: IBP over the wide one-hidden-layer network
    (weights read once per call), a standalone concretisation of an intermediate-layer
    Lambda of the MLP workload, and a plain device copy for scale."""
    import torch
    import workloads as wk
    import linear_bound_propagation_amd as lbp
    out = []
    dev = "cuda:0"
    # plain copy of 1 GiB: read + write
    a = torch.empty(1 << 28, device=dev)
    b = torch.empty_like(a)
    ms = _time_calls(lambda: b.copy_(a), reps)
    copy_gbps = 2 * a.numel() * 4 / (ms * 1e-3) / 1e9
    del a, b
    # IBP over the 4096-262144-100 network, batch 8
    print("[bench] hbm: building the wide network", file=sys.stderr, flush=True)
    wl = wk.wide()
    net, x, _ = lbp.prepare(wl, dev)
    lo, hi = net.alloc_bounds(wl.batch)
    ws = net.workspace(net.workspace_size(wl.batch, 0, "ibp"))
    ms = _time_calls(lambda: lbp.ibp(net, x, float(wl.eps), lo=lo, hi=hi, ws=ws), reps)
    n_w = sum(nd.weight.size + nd.bias.size for nd in wl.nodes if nd.op == "linear")
    # activations: input read; hidden bounds and their ReLU written (4 arrays) and two read back; outputs
    hid = wl.nodes[1].size
    act = wl.batch * (wl.nodes[0].size + 6 * hid + 2 * wl.nodes[-1].size)
    nbytes = 4 * (n_w + act)
    out.append({"kernel": "ibp_narrow_kernel (+ split-K finish): vb_ibp over every node", "workload": wl.name,
                "bound": "hbm", "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                "frac_of_copy": round(nbytes / (ms * 1e-3) / 1e9 / copy_gbps, 4),
                "bytes_per_call": nbytes, "ms_per_call": round(ms, 4)})
    del net, x, lo, hi, ws, wl
    torch.cuda.empty_cache()
    # standalone concretisation: 64 inputs x 2048 rows over a 3072-wide input (1.6 GB of Lambda)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    B, R, n = 64, 2048, 3072
    A = torch.randn(B * R, n, device=dev, generator=g)
    center = torch.rand(B, n, device=dev, generator=g)
    lb = torch.empty(B * R, device=dev)
    ub = torch.empty_like(lb)
    ms = _time_calls(lambda: lbp.concretize(A, None, center, 2.0 / 255, R, lb=lb, ub=ub), reps)
    nbytes = 4 * A.numel() + 8 * B * R
    out.append({"kernel": "concretize_rows_kernel: vb_concretize", "workload": f"Lambda {B}x{R}x{n} fp32, ball",
                "bound": "hbm", "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                "frac_of_copy": round(nbytes / (ms * 1e-3) / 1e9 / copy_gbps, 4),
                "bytes_per_call": nbytes, "ms_per_call": round(ms, 4)})
    return out, round(copy_gbps, 1)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-hbm", action="store_true", help="skip the memory-bound kernel measurements")
    ap.add_argument("--dense-alpha", action="store_true",
                    help="alpha-CROWN workloads: keep alpha for every neuron instead of the unstable ones only")
    ap.add_argument("--intermediate", default=None,
                    help="override the workload's intermediate-bound method (ibp, crown, hybrid, crown+ibp, ...)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    args = ap.parse_args()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the bound computation is not "
              "sharded across GPUs in this build", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as wk
    import linear_bound_propagation_amd as lbp

    wl = wk.config(args.workload)
    if args.intermediate:
        wl.intermediate = args.intermediate
        wl.name += "_" + args.intermediate.replace("+", "_")
    print(f"[bench] workload {wl.name}: building device copies", file=sys.stderr, flush=True)
    net, x, C = lbp.prepare(wl, "cuda:0")
    lo, hi = net.alloc_bounds(wl.batch)
    out = {"lo": lo, "hi": hi}
    for k in ("ibp_lb", "ibp_ub", "lb", "ub"):
        out[k] = torch.empty(wl.batch, wl.m, device=net.device)
    ws_bytes = net.workspace_size(wl.batch, wl.m, wl.intermediate, wl.region_start or 0)
    free = torch.cuda.mem_get_info()[0]
    ws = net.workspace(min(ws_bytes, int(free * 0.85)))
    alpha_info = {}
    if wl.alpha_steps:
        lb_steps = torch.empty(wl.alpha_steps + 1, wl.batch, wl.m, device=net.device)
        best = torch.empty(wl.batch, wl.m, device=net.device)
        states = {}

        def step():
            lbp.crown(net, x, float(wl.eps), C, wl.intermediate, wl.region_start, ws=ws, out=out)
            # compact alpha: the state of the unstable neurons only (the layout call
            # synchronises the stream to size it; it is part of the timed step)
            lay = None if args.dense_alpha else lbp.alpha_layout(net, out["lo"], out["hi"])
            key = None if lay is None else tuple(lay.width)
            if key not in states:
                states[key] = lbp.alpha_state(net, wl.batch, wl.m, lay)
            state = states[key]
            alpha_info["alpha_storage"] = "dense" if lay is None else "compact (unstable neurons)"
            alpha_info["alpha_adam_state_gb"] = round(sum(t.numel() * 4 for part in state for t in part
                                                          if t is not None) / 1e9, 3)
            lbp.alpha_crown(net, x, float(wl.eps), C, out["lo"], out["hi"], wl.alpha_steps, wl.alpha_lr, ws=ws,
                            state=state, lb_steps=lb_steps, best=best, layout=lay)
            out["lb"] = best
    else:
        def step():
            lbp.crown(net, x, float(wl.eps), C, wl.intermediate, wl.region_start, ws=ws, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    lbp.profile_start()
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    k_ms, k_flops, k_launches = lbp.profile_stop()
    ms = e0.elapsed_time(e1) / args.steps
    print(f"[bench] timed {args.steps} steps: {ms:.3f} ms/step", file=sys.stderr, flush=True)

    fl = algorithmic_flops(wl)
    tflops = fl["all"] / (ms * 1e-3) / 1e12
    lb = out["lb"]
    verified = float((lb > 0).all(dim=1).float().mean().item())
    achieved = k_flops / (k_ms * 1e-3) / 1e12 if k_ms > 0 else None
    line = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "specs": wl.m, "eps": float(wl.eps),
                   "intermediate": wl.intermediate, "alpha_steps": wl.alpha_steps,
                   "algorithmic_tflop_per_step": round(fl["all"] / 1e12, 4),
                   "workspace_gb": round(ws.numel() / 1e9, 2), **alpha_info},
        "frac_of_fp32_mfma_peak": round(tflops / PEAK_FP32_MFMA_TFLOPS, 4),
        "specs_per_s": round(wl.batch * wl.m / (ms * 1e-3), 1),
        "verified_frac": verified,
        "roofline": {
            "kernel": "gemm_kernel: back-substitution GEMM (relaxation / concretisation epilogues)",
            "bound": "mfma",
            "achieved": None if achieved is None else round(achieved, 3),
            "peak": PEAK_FP32_MFMA_TFLOPS,
            "unit": "TFLOP/s",
            "frac": None if achieved is None else round(achieved / PEAK_FP32_MFMA_TFLOPS, 4),
            "traffic": measured_traffic(wl.name),
            "launches": k_launches,
            "avg_launch_ms": round(k_ms / max(k_launches, 1), 4),
            "alg_flop_per_launch": k_flops / max(k_launches, 1),
        },
        "cpu_baseline": None,
    }
    if not args.no_hbm:
        print("[bench] timing the memory-bound kernels", file=sys.stderr, flush=True)
        del ws
        torch.cuda.empty_cache()
        line["hbm_kernels"], line["copy_GBps"] = hbm_kernels()
    if not args.no_cpu:
        print("[bench] timing the float64 oracle on the host cores", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl, fl["all"])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
