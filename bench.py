"""Benchmark of the bound-propagation hot path on one MI355X.

One step = one whole bound computation for one batch: IBP of every node, the
intermediate bounds of every ReLU input (CROWN back-substitution per layer for
the MLP workloads), and the spec bounds by IBP and by CROWN.  Inputs are
resident in HBM before the timed region.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload N] [--no-cpu] [--no-hbm] [--no-extra]

Default workload: the residual network (configuration 5, the largest that fits one
GPU), hybrid bounds (IBP up to the last stage, CROWN inside it).  `value` is
algorithmic TFLOP/s of the whole step, counting identity rows over the conv region
on their footprint windows (structurally non-zero multiply-adds only); the dense
count is reported beside it.  The other workloads run briefly as extra keys.
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


def _windows(nodes, z, stop):
    """Footprint windows of identity rows over node z on every node they reach on the
    way to `stop`: node k -> ((ay, y0, y1), (ax, x0, x1)), the rows of pixel (py, px) of
    z being non-zero over k's output only at y in [ay*py + y0, ay*py + y1] (and the same
    in x), before clipping to the image.  A conv widens the window by its kernel and
    scales it by its stride; ReLU and ADD pass it on (an ADD input reached by several
    paths takes the bounding box of their windows).  None if the rows leave the
    convolution region (GAP, Linear, Flatten) before `stop`, or if two paths reach a
    node with different scales."""
    if nodes[z].op not in ("conv", "add", "relu"):
        return None
    W = {z: ((1, 0, 0), (1, 0, 0))}
    for k in range(z, stop, -1):
        if k not in W:
            continue
        nd = nodes[k]
        (ay, y0, y1), (ax, x0, x1) = W[k]
        if nd.op == "conv":
            s, p = nd.stride, nd.pad
            kh, kw = nd.weight.shape[2], nd.weight.shape[3]
            win = ((ay * s, y0 * s - p, y1 * s - p + kh - 1), (ax * s, x0 * s - p, x1 * s - p + kw - 1))
        elif nd.op in ("relu", "add"):
            win = W[k]
        else:
            return None
        for t in nd.inputs:
            if t in W:
                (by, a0, a1), (bx, b0, b1) = W[t]
                if by != win[0][0] or bx != win[1][0]:
                    return None
                W[t] = ((by, min(a0, win[0][1]), max(a1, win[0][2])), (bx, min(b0, win[1][1]), max(b1, win[1][2])))
            else:
                W[t] = win
    return W


def _clipped_cells(win, shape_z, shape_k):
    """Per pixel (py, px) of z: the cells of k's output inside both the window and the
    image, as two factors ny[py], nx[px] (the count is ny[py] * nx[px])."""
    (ay, y0, y1), (ax, x0, x1) = win
    _, hz, wz = shape_z
    _, hk, wk = shape_k
    ys = ay * np.arange(hz)
    xs = ax * np.arange(wz)
    ny = np.clip(np.minimum(ys + y1, hk - 1) - np.maximum(ys + y0, 0) + 1, 0, None)
    nx = np.clip(np.minimum(xs + x1, wk - 1) - np.maximum(xs + x0, 0) + 1, 0, None)
    return ny, nx


def _cell_taps(win_axis, n_z, n_out, n_in, stride, pad, k):
    """Per pixel of z along one axis: the (output cell, tap) pairs of one conv whose
    output cell lies inside the row's window and the image and whose tap lands inside
    the conv's input image (a tap into the zero padding multiplies nothing)."""
    a, lo, hi = win_axis
    out = np.zeros(n_z)
    for pz in range(n_z):
        for yo in range(max(a * pz + lo, 0), min(a * pz + hi, n_out - 1) + 1):
            yi = yo * stride - pad + np.arange(k)
            out[pz] += np.count_nonzero((yi >= 0) & (yi < n_in))
    return out


def footprint_row_macs(nodes, z, stop):
    """Multiply-adds of one identity row over conv-region node z, per pixel of z
    ([h_z][w_z]), when every row is carried on its footprint window: at each conv on
    the way to `stop` only the products that can be non-zero count, i.e. output cells
    inside the row's window and the image, through taps that land inside the conv's
    input image; the first step (a copy of the weight footprint into the rows) costs
    nothing.  None if the rows do not stay in the convolution region."""
    W = _windows(nodes, z, stop)
    if W is None or len(nodes[z].shape) != 3:
        return None
    free = _identity_consumers(nodes, z)
    _, hz, wz = nodes[z].shape
    per = np.zeros((hz, wz))
    for k, win in W.items():
        nk = nodes[k]
        if nk.op != "conv" or k in free or k == stop:
            continue
        co, ci, kh, kw = nk.weight.shape
        _, hi_, wi_ = nodes[_src(nodes, nk.inputs[0])].shape
        ty = _cell_taps(win[0], hz, nk.shape[1], hi_, nk.stride, nk.pad, kh)
        tx = _cell_taps(win[1], wz, nk.shape[2], wi_, nk.stride, nk.pad, kw)
        per += np.outer(ty, tx) * (co * ci)
    return per


def algorithmic_flops(wl):
    """FLOPs the method itself performs for the whole batch (no padding, no tile waste):
    2 * rows * multiply-adds of each affine node a row of Lambda passes through; the
    first step of identity rows (a copy of the weight footprint) costs nothing; IBP
    is two passes (centre and radius) of the forward multiply-adds."""
    nodes, B, m = wl.nodes, wl.batch, wl.m
    total = {"ibp": 0.0, "intermediate": 0.0, "spec": 0.0, "dense_intermediate": 0.0}
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
            free = _identity_consumers(nodes, z)
            dense = sum(2 * rows * _mac_per_row(nodes[k], nodes) for k in _active(nodes, z, stop)
                        if nodes[k].op in ("linear", "conv") and k not in free)
            total["dense_intermediate"] += dense
            fp = footprint_row_macs(nodes, z, stop)
            if fp is not None:
                # identity rows on footprint windows: count only the cells that exist
                total["intermediate"] += 2 * 2 * B * zn.shape[0] * float(fp.sum())
            else:
                total["intermediate"] += dense
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
    total["all"] = sum(v for k, v in total.items() if k != "dense_intermediate")
    total["all_dense"] = total["all"] - total["intermediate"] + total["dense_intermediate"]
    return total


def _host_cpu():
    """(threads the process may use, CPU model) of the host."""
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return cores, model


def _oracle_rows_sample(wl, budget_s, fl):
    """Oracle timing for workloads whose single input takes the oracle minutes (CROWN
    intermediate bounds over conv layers): input 0, its IBP bounds, then rounds of 32
    seeded neurons of every CROWN-refined layer (both signs, the IBP bounds of the
    layers below as relaxation bounds) and once the spec rows, until the budget is
    spent.  The work credited is the algorithmic count of exactly those rows."""
    import torch
    from oracle import Oracle, ibp as oracle_ibp
    from oracle.bounds import backward, _domain
    nodes = wl.nodes
    net = Oracle(nodes)
    stop = wl.region_start if wl.intermediate.startswith("hybrid") else 0
    t0 = time.perf_counter()
    lo, hi = oracle_ibp(net, wl.x0[:1], wl.eps)
    dc, dr = _domain(net, lo, hi, wl.x0, wl.eps, 0, stop)
    L = len(nodes) - 1
    C = torch.as_tensor(wl.C[0], dtype=torch.float64)
    backward(net, lo, hi, 0, L, C, stop, dc, dr)
    backward(net, lo, hi, 0, L, -C, stop, dc, dr)
    work = fl["ibp"] / wl.batch + fl["spec"] / wl.batch
    layers = []
    for nd in nodes:
        if nd.op != "relu":
            continue
        z = nd.inputs[0]
        zn = nodes[z]
        if z <= stop or (zn.op in ("linear", "conv") and _src(nodes, zn.inputs[0]) == stop):
            continue
        per = footprint_row_macs(nodes, z, stop)
        layers.append((z, per))
    rng = np.random.default_rng(0)
    rows = 0
    while time.perf_counter() - t0 < budget_s:
        for z, per in layers:
            shape = nodes[z].shape
            n = nodes[z].size
            idx = rng.choice(n, 32, replace=False)
            eye = torch.zeros((32, n), dtype=torch.float64)
            eye[torch.arange(32), torch.as_tensor(idx)] = 1.0
            eye = eye.reshape((32,) + tuple(shape))
            backward(net, lo, hi, 0, z, eye, stop, dc, dr)
            backward(net, lo, hi, 0, z, -eye, stop, dc, dr)
            if per is not None:
                _, hz, wz = shape
                pix = idx % (hz * wz)
                work += 2 * 2 * float(per.reshape(-1)[pix].sum())
            else:
                free = _identity_consumers(nodes, z)
                work += 2 * 2 * 32 * sum(_mac_per_row(nodes[k], nodes) for k in _active(nodes, z, stop)
                                         if nodes[k].op in ("linear", "conv") and k not in free)
            rows += 64
    elapsed = time.perf_counter() - t0
    return work, elapsed, (f"input 0: IBP, the {2 * wl.m} spec rows and {rows} identity rows (32 seeded neurons "
                           f"x 2 signs per round over {len(layers)} CROWN-refined layers, IBP bounds below)")


def cpu_baseline(wl, fl, budget_s=12.0):
    """The float64 oracle on the host cores, on a bounded sample of the workload (about
    budget_s of CPU work), scaled to TFLOP/s of the same algorithmic work (the count
    credited is exactly the sample's).  Whole inputs where one input takes the oracle
    less than the budget (for alpha-CROWN: its intermediate bounds and the whole
    alpha loop of that input); otherwise a sample of rows of the first input."""
    import torch
    from oracle import crown_bounds
    cores, model = _host_cpu()
    per_input = fl["all"] / wl.batch
    heavy = wl.intermediate != "ibp" and any(nd.op == "conv" for nd in wl.nodes)
    if heavy:
        work, elapsed, sample = _oracle_rows_sample(wl, budget_s, fl)
        specs_per_s = None
    else:
        k, elapsed = 0, 0.0
        while k < wl.batch and elapsed < budget_s:
            t0 = time.perf_counter()
            res = crown_bounds(wl, batch_idx=[k])
            if wl.alpha_steps:
                from oracle.alpha import alpha_crown
                alpha_crown(wl, res["lo"], res["hi"], batch_idx=[k])
            elapsed += time.perf_counter() - t0
            k += 1
        work = per_input * k
        specs_per_s = k * wl.m / elapsed
        what = "IBP + CROWN" + (f" + {wl.alpha_steps}-step alpha-CROWN" if wl.alpha_steps else "")
        sample = f"first {k} of {wl.batch} inputs ({what}), all {wl.m} specs"
    out = {"value": work / elapsed / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
           "sample": f"{sample}; float64 torch-CPU oracle (BLAS / oneDNN-backed), {elapsed:.1f} s",
           "cpu_model": model, "threads": torch.get_num_threads()}
    if specs_per_s is not None:
        out["specs_per_s"] = specs_per_s
    # one single-thread run of the small MLP workload (784-100-100-10, 16 inputs)
    import workloads as wk
    w1 = wk.config(1)
    nt = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        t0 = time.perf_counter()
        crown_bounds(w1)
        dt = time.perf_counter() - t0
    finally:
        torch.set_num_threads(nt)
    out["single_thread_mlp784"] = {"specs_per_s": round(w1.batch * w1.m / dt, 1),
                                   "tflops": algorithmic_flops(w1)["all"] / dt / 1e12, "seconds": round(dt, 3)}
    return out


GEMM_SOURCE = os.path.join(ROOT, "linear_bound_propagation_amd", "csrc", "vb_gemm.hip")


def measured_traffic(workload_name):
    """HBM bytes per back-substitution GEMM launch from the committed counter summary of
    this workload (profiles/gemm_backsub_traffic_*.txt), or None when there is none or it
    was taken on a different kernel source."""
    import glob
    import hashlib
    sha = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "gemm_backsub_traffic_*.txt"))):
        kv = {}
        for line in open(path):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        if kv.get("workload") != workload_name or kv.get("kernel_source_sha256") != sha:
            continue
        try:
            return float(kv["hbm_bytes_per_launch"])
        except (KeyError, ValueError):
            return None
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


PROBE_LIB = os.path.join(ROOT, "linear_bound_propagation_amd", "libvbprobe.so")


def probes(reps=10):
    """Measured ceilings of the GPU at hand (libvbprobe.so, built with the library):
    an MFMA-only loop (v_mfma_f32_32x32x2f32, four independent accumulator chains per
    wavefront, 2048 workgroups of 4 wavefronts, no memory traffic) and HBM read, write
    and copy streams over 4 GiB buffers (16-byte non-temporal accesses, one contiguous
    16 KB segment per workgroup)."""
    import ctypes
    import torch
    lib = ctypes.CDLL(PROBE_LIB)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong
    lib.vbp_mfma_loop.argtypes = [i32, i32, P, P]
    lib.vbp_read.argtypes = [P, i64, P, P]
    lib.vbp_write.argtypes = [P, i64, ctypes.c_float, P]
    lib.vbp_copy.argtypes = [P, P, i64, P]
    lib.vbp_stream_blocks.restype = i64
    lib.vbp_stream_blocks.argtypes = [i64]
    st = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def ok(rc):
        if rc != 0:
            raise RuntimeError(f"probe launch failed: {rc}")
    dev = "cuda:0"
    blocks, iters = 2048, 50000
    sink = torch.empty(max(blocks, 1 << 16), device=dev)
    ms = _time_calls(lambda: ok(lib.vbp_mfma_loop(blocks, iters, ctypes.c_void_p(sink.data_ptr()), st())), 3, 1)
    mfma = blocks * 4 * iters * 4 * 4096 / (ms * 1e-3) / 1e12
    n = 1 << 30
    a = torch.empty(n, device=dev)
    b = torch.empty(n, device=dev)
    a.fill_(1.0)
    sink = torch.empty(max(int(lib.vbp_stream_blocks(n)), 1 << 16), device=dev)   # one float per read workgroup
    rd = _time_calls(lambda: ok(lib.vbp_read(ctypes.c_void_p(a.data_ptr()), n, ctypes.c_void_p(sink.data_ptr()),
                                            st())), reps)
    wr = _time_calls(lambda: ok(lib.vbp_write(ctypes.c_void_p(b.data_ptr()), n, 0.5, st())), reps)
    cp = _time_calls(lambda: ok(lib.vbp_copy(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()), n,
                                            st())), reps)
    tc = _time_calls(lambda: b.copy_(a), reps)
    del a, b
    torch.cuda.empty_cache()
    gb = lambda nbytes, t: round(nbytes / (t * 1e-3) / 1e9, 1)
    return {"mfma_fp32_tflops": round(mfma, 2), "mfma_fp32_frac_of_peak": round(mfma / PEAK_FP32_MFMA_TFLOPS, 4),
            "hbm_read_GBps": gb(4 * n, rd), "hbm_write_GBps": gb(4 * n, wr), "hbm_copy_GBps": gb(8 * n, cp),
            "torch_copy_GBps": gb(8 * n, tc), "peak_fp32_mfma_tflops": PEAK_FP32_MFMA_TFLOPS,
            "peak_hbm_GBps": PEAK_HBM_GBPS, "stream_bytes": 4 * n}


def hbm_kernels(stream_ceiling, reps=20):
    """The memory-bound kernels, timed live: IBP over the wide one-hidden-layer network
    (weights read once per call) and a standalone concretisation of an intermediate-layer
    Lambda of the MLP workload; each against 8 TB/s and against the measured read
    stream (both kernels read far more than they write)."""
    import torch
    import workloads as wk
    import linear_bound_propagation_amd as lbp
    out = []
    dev = "cuda:0"
    copy_gbps = stream_ceiling
    # IBP over the 4096-262144-100 network, batch 8
    print("[bench] hbm: building the wide network", file=sys.stderr, flush=True)
    wl = wk.wide()
    net, x, _ = lbp.prepare(wl, dev)
    lo, hi = net.alloc_bounds(wl.batch)
    ws = net.workspace(net.workspace_size(wl.batch, 0, "ibp"))
    n_w = sum(nd.weight.size + nd.bias.size for nd in wl.nodes if nd.op == "linear")
    # activations: input read; hidden bounds and their ReLU written (4 arrays) and two read back; outputs
    hid = wl.nodes[1].size
    act = wl.batch * (wl.nodes[0].size + 6 * hid + 2 * wl.nodes[-1].size)
    nbytes = 4 * (n_w + act)
    # row-major weights, then the packed copies (vb_pack_linear, once before timing: a
    # weight-layout step like any weight pre-packing; the bytes read per call are the same)
    ms_rm = _time_calls(lambda: lbp.ibp(net, x, float(wl.eps), lo=lo, hi=hi, ws=ws), reps)
    held = net.pack_linear()
    torch.cuda.synchronize()
    ms = _time_calls(lambda: lbp.ibp(net, x, float(wl.eps), lo=lo, hi=hi, ws=ws), reps)
    out.append({"kernel": "ibp_narrow_kernel (+ split-K finish): vb_ibp over every node, packed weights",
                "workload": wl.name,
                "bound": "hbm", "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                "frac_of_read_stream": round(nbytes / (ms * 1e-3) / 1e9 / copy_gbps, 4),
                "bytes_per_call": nbytes, "ms_per_call": round(ms, 4),
                "packed_weight_bytes": held,
                "row_major_weights": {"ms_per_call": round(ms_rm, 4),
                                      "achieved": round(nbytes / (ms_rm * 1e-3) / 1e9, 1),
                                      "frac": round(nbytes / (ms_rm * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}})
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
                "frac_of_read_stream": round(nbytes / (ms * 1e-3) / 1e9 / copy_gbps, 4),
                "bytes_per_call": nbytes, "ms_per_call": round(ms, 4)})
    return out


def run_workload(wl, steps, warmup, dense_alpha=False, profile=True):
    """Time `steps` whole bound computations of a workload (after `warmup`), inputs
    resident in HBM.  Returns (ms per step, GEMM profile (ms, flops, launches), last
    outputs, workspace bytes, alpha info)."""
    import torch
    import linear_bound_propagation_amd as lbp
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
            lay = None if dense_alpha else lbp.alpha_layout(net, out["lo"], out["hi"])
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

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({warmup} steps)", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    if profile:
        lbp.profile_start()
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    prof = lbp.profile_stop() if profile else (0.0, 0.0, 0)
    ms = e0.elapsed_time(e1) / steps
    print(f"[bench] timed {steps} steps: {ms:.3f} ms/step", file=sys.stderr, flush=True)
    res = {"lb": out["lb"].clone(), "ub": out["ub"].clone()}
    nbytes = ws.numel()
    del ws, out, net, x, C
    torch.cuda.empty_cache()
    return ms, prof, res, nbytes, alpha_info


def gemm_roofline(prof, name):
    k_ms, k_flops, k_launches = prof
    achieved = k_flops / (k_ms * 1e-3) / 1e12 if k_ms > 0 else None
    return {
        "kernel": "gemm_kernel: back-substitution GEMM (relaxation / concretisation / store epilogues)",
        "bound": "mfma",
        "achieved": None if achieved is None else round(achieved, 3),
        "peak": PEAK_FP32_MFMA_TFLOPS,
        "unit": "TFLOP/s",
        "frac": None if achieved is None else round(achieved / PEAK_FP32_MFMA_TFLOPS, 4),
        "traffic": measured_traffic(name),
        "launches": k_launches,
        "avg_launch_ms": round(k_ms / max(k_launches, 1), 4),
        "alg_flop_per_launch": k_flops / max(k_launches, 1),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=5,
                    help="1-5: the measured configurations (default 5: the residual network, the largest)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-hbm", action="store_true", help="skip the probes and the memory-bound kernels")
    ap.add_argument("--no-extra", action="store_true", help="skip the short runs of the other workloads")
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

    import workloads as wk

    wl = wk.config(args.workload)
    if args.intermediate:
        wl.intermediate = args.intermediate
        wl.name += "_" + args.intermediate.replace("+", "_")
    ms, prof, res, ws_bytes, alpha_info = run_workload(wl, args.steps, args.warmup, args.dense_alpha)
    fl = algorithmic_flops(wl)
    tflops = fl["all"] / (ms * 1e-3) / 1e12
    lb = res["lb"]
    import linear_bound_propagation_amd as lbp
    flags, n_ver = lbp.verify(lb.contiguous())           # the library's verdict per input
    verified = float(n_ver.item()) / wl.batch
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
                   "dense_tflop_per_step": round(fl["all_dense"] / 1e12, 4),
                   "workspace_gb": round(ws_bytes / 1e9, 2), **alpha_info},
        "frac_of_fp32_mfma_peak": round(tflops / PEAK_FP32_MFMA_TFLOPS, 4),
        "dense_equivalent_tflops": round(fl["all_dense"] / (ms * 1e-3) / 1e12, 3),
        "specs_per_s": round(wl.batch * wl.m / (ms * 1e-3), 1),
        "verified_frac": verified,
        "roofline": gemm_roofline(prof, wl.name),
        "cpu_baseline": None,
    }
    if not args.no_extra:
        extra = {}
        for cfg in (1, 2, 3, 4, 5, "3crown"):
            if cfg == args.workload:
                continue
            if cfg == "3crown":
                # the CNN with CROWN intermediate bounds (footprint rows through its convs)
                w = wk.config(3)
                w.intermediate = "crown"
                w.name = w.name.replace("_ibp", "_crown")
            else:
                w = wk.config(cfg)
            e_ms, e_prof, e_res, _, e_alpha = run_workload(w, 5 if cfg != 5 else 2, 2)
            e_fl = algorithmic_flops(w)
            extra[w.name] = {"ms_per_step": round(e_ms, 4),
                             "tflops": round(e_fl["all"] / (e_ms * 1e-3) / 1e12, 3),
                             "algorithmic_tflop_per_step": round(e_fl["all"] / 1e12, 4),
                             "specs_per_s": round(w.batch * w.m / (e_ms * 1e-3), 1),
                             "verified_frac": float(lbp.verify(e_res["lb"].contiguous())[1].item()) / w.batch,
                             "gemm": {k: v for k, v in gemm_roofline(e_prof, w.name).items()
                                      if k in ("achieved", "frac", "launches", "avg_launch_ms")}, **e_alpha}
        line["other_workloads"] = extra
    if not args.no_hbm:
        print("[bench] probes and memory-bound kernels", file=sys.stderr, flush=True)
        line["probes"] = probes()
        line["hbm_kernels"] = hbm_kernels(line["probes"]["hbm_read_GBps"])
    if not args.no_cpu:
        print("[bench] timing the float64 oracle on the host cores", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl, fl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
