"""MI355X-native linear bound propagation (IBP, CROWN, alpha-CROWN).

Thin ctypes binding over libvbprop.so (the C ABI declared in include/vb.h).
PyTorch is used only for device memory and the current HIP stream; every
step of the bound computation runs in the library's HIP kernels.  The
binding marshals arguments: it lays a network out in the library's formats
(channels-last activations, [kh][kw][c_out][c_in] conv weights, Linear
columns after a flatten in (h, w, c) order) and passes device pointers.

The shared library is loaded on first use; if it is missing, that first call
raises ImportError: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvbprop.so")

VB_INPUT, VB_LINEAR, VB_CONV2D, VB_RELU, VB_ADD, VB_GAP, VB_FLATTEN = range(7)
METHODS = {"ibp": 0, "crown": 1, "hybrid": 2, "crown+ibp": 1 | 16, "hybrid+ibp": 2 | 16,
           "crown+unstable": 1 | 64, "hybrid+unstable": 2 | 64, "crown+ibp+unstable": 1 | 16 | 64,
           "hybrid+ibp+unstable": 2 | 16 | 64}
VB_ALPHA_ROWS = 32
STATUS = {0: "VB_OK", -1: "VB_EINVAL", -2: "VB_ESHAPE", -3: "VB_ENOMEM", -4: "VB_EDEVICE",
          -5: "VB_EUNSUPPORTED"}
_OPS = {"input": VB_INPUT, "linear": VB_LINEAR, "conv": VB_CONV2D, "relu": VB_RELU, "add": VB_ADD,
        "gap": VB_GAP, "flatten": VB_FLATTEN}

EXPORTS = ["vb_last_error", "vb_workspace_size", "vb_ibp", "vb_crown_backward", "vb_concretize",
           "vb_alpha_layout", "vb_alpha_init", "vb_alpha_step", "vb_alpha_step_rows", "vb_apply_splits",
           "vb_bab_workspace_size", "vb_bab", "vb_crown", "vb_crown_noalloc", "vb_verify",
           "vb_profile_start", "vb_profile_stop", "vb_profile_record", "vb_pack_linear_bytes", "vb_pack_linear"]
# host-only helpers declared in include/vb_testing.h (used by the CPU tests)
TESTING_EXPORTS = ["vb_testing_fastdiv", "vb_testing_conv_tile_n", "vb_testing_identity_path"]


class vb_node(ctypes.Structure):
    _fields_ = [("op", ctypes.c_int32), ("in0", ctypes.c_int32), ("in1", ctypes.c_int32),
                ("c", ctypes.c_int32), ("h", ctypes.c_int32), ("w", ctypes.c_int32),
                ("kh", ctypes.c_int32), ("kw", ctypes.c_int32), ("stride", ctypes.c_int32),
                ("pad", ctypes.c_int32), ("weight", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("weight_packed", ctypes.c_void_p)]


class vb_graph(ctypes.Structure):
    _fields_ = [("n_nodes", ctypes.c_int32), ("nodes", ctypes.POINTER(vb_node))]


class vb_beta(ctypes.Structure):
    _fields_ = [("split", ctypes.POINTER(ctypes.c_void_p)), ("beta", ctypes.POINTER(ctypes.c_void_p)),
                ("beta_m", ctypes.POINTER(ctypes.c_void_p)), ("beta_v", ctypes.POINTER(ctypes.c_void_p))]


class vb_bab_params(ctypes.Structure):
    _fields_ = [("steps", ctypes.c_int32), ("lr", ctypes.c_float), ("beta1", ctypes.c_float),
                ("beta2", ctypes.c_float), ("adam_eps", ctypes.c_float), ("batch", ctypes.c_int32),
                ("max_domains", ctypes.c_int32)]


class vb_alpha_compact(ctypes.Structure):
    _fields_ = [("index", ctypes.POINTER(ctypes.c_void_p)), ("width", ctypes.POINTER(ctypes.c_int32))]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built: run `python -m linear_bound_propagation_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    PP = ctypes.POINTER(ctypes.c_void_p)
    G = ctypes.POINTER(vb_graph)
    i32, f32, sz = ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.vb_last_error.restype = ctypes.c_char_p
    lib.vb_last_error.argtypes = []
    lib.vb_workspace_size.restype = i32
    lib.vb_workspace_size.argtypes = [G, i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.vb_ibp.restype = i32
    lib.vb_ibp.argtypes = [G, i32, P, P, f32, PP, PP, P, i32, P, P, P, sz, P]
    lib.vb_pack_linear_bytes.restype = i32
    lib.vb_pack_linear_bytes.argtypes = [i32, i32, ctypes.POINTER(sz)]
    lib.vb_pack_linear.restype = i32
    lib.vb_pack_linear.argtypes = [P, i32, i32, P, sz, P]
    lib.vb_crown_backward.restype = i32
    AC = ctypes.POINTER(vb_alpha_compact)
    lib.vb_crown_backward.argtypes = [G, i32, i32, i32, P, i32, PP, PP, AC, PP, P, P, f32, P, P, P, P, P, sz, P]
    lib.vb_concretize.restype = i32
    lib.vb_concretize.argtypes = [i32, i32, i32, P, P, P, P, f32, P, P, P]
    lib.vb_alpha_init.restype = i32
    lib.vb_alpha_layout.restype = i32
    lib.vb_alpha_layout.argtypes = [G, i32, PP, PP, PP, ctypes.POINTER(i32), P, sz, P]
    lib.vb_alpha_init.argtypes = [G, i32, i32, PP, PP, AC, PP, PP, PP, P]
    lib.vb_alpha_step.restype = i32
    lib.vb_alpha_step.argtypes = [G, i32, P, i32, PP, PP, P, P, f32, AC, PP, PP, PP, i32, f32, f32, f32, f32,
                                  P, P, P, sz, P]
    lib.vb_alpha_step_rows.restype = i32
    BT = ctypes.POINTER(vb_beta)
    lib.vb_alpha_step_rows.argtypes = [G, i32, i32, P, i32, PP, PP, P, P, f32, AC, BT, PP, PP, PP, i32, f32, f32, f32,
                                       f32, P, P, P, P, P, sz, P]
    lib.vb_apply_splits.restype = i32
    lib.vb_apply_splits.argtypes = [G, i32, PP, PP, PP, P]
    lib.vb_bab_workspace_size.restype = i32
    lib.vb_bab_workspace_size.argtypes = [G, i32, i32, ctypes.POINTER(sz)]
    lib.vb_bab.restype = i32
    lib.vb_bab.argtypes = [G, P, P, f32, P, i32, PP, PP, ctypes.POINTER(vb_bab_params), ctypes.POINTER(i32),
                           ctypes.POINTER(i32), P, P, sz, P]
    lib.vb_crown.restype = i32
    lib.vb_crown.argtypes = [G, i32, P, P, f32, i32, i32, PP, PP, P, i32, P, P, P, P, P, sz, P]
    lib.vb_verify.restype = i32
    lib.vb_verify.argtypes = [i32, i32, P, P, P, P]
    lib.vb_crown_noalloc.restype = i32
    lib.vb_crown_noalloc.argtypes = [G, i32, P, P, f32, i32, i32, PP, PP, P, i32, P, P, P, P, P]
    lib.vb_profile_start.restype = i32
    lib.vb_profile_start.argtypes = []
    lib.vb_profile_stop.restype = i32
    lib.vb_profile_stop.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_int64)]
    lib.vb_profile_record.restype = i32
    lib.vb_profile_record.argtypes = [ctypes.c_int64, ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32)]
    return lib


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded libvbprop.so (loaded once; raises ImportError if it is not built)."""
    global _LIB
    if _LIB is None:
        _LIB = load_library()
    return _LIB


class VBError(RuntimeError):
    def __init__(self, status: int, fn: str):
        msg = lib().vb_last_error().decode(errors="replace")
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {msg}")
        self.status = status


def _check(status: int, fn: str):
    if status != 0:
        raise VBError(status, fn)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ptr_array(ts: Sequence[Optional[torch.Tensor]]):
    arr = (ctypes.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = None if t is None else t.data_ptr()
    return arr


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _f32(x, device):
    return torch.as_tensor(np.ascontiguousarray(x), dtype=torch.float32, device=device)


def to_channels_last(x: np.ndarray) -> np.ndarray:
    """[B][C][H][W] -> [B][H][W][C] (flat [B][n] unchanged)."""
    x = np.asarray(x)
    return np.ascontiguousarray(x.transpose(0, 2, 3, 1)) if x.ndim == 4 else x


def from_channels_last(t: torch.Tensor, shape) -> torch.Tensor:
    """Device bounds [B][h*w*c] (or [B][h][w][c]) of a node with shape (C, H, W) -> [B][C][H][W]."""
    if len(shape) == 1:
        return t.reshape(t.shape[0], -1)
    c, h, w = shape
    return t.reshape(t.shape[0], h, w, c).permute(0, 3, 1, 2)


class DeviceNet:
    """A network from ``workloads`` laid out on the device in the library's formats."""

    def __init__(self, nodes, device="cuda"):
        self.device = torch.device(device)
        self.shapes = [tuple(n.shape) for n in nodes]
        self.ops = [n.op for n in nodes]
        self.inputs = [tuple(n.inputs) for n in nodes]
        self._keep: List[torch.Tensor] = []
        self._w: List[Optional[torch.Tensor]] = []  # device weights per node (None without)
        arr = (vb_node * len(nodes))()
        for k, n in enumerate(nodes):
            v = arr[k]
            v.op = _OPS[n.op]
            v.in0 = n.inputs[0] if len(n.inputs) > 0 else -1
            v.in1 = n.inputs[1] if len(n.inputs) > 1 else -1
            if len(n.shape) == 3:
                v.c, v.h, v.w = n.shape
            else:
                v.c, v.h, v.w = n.shape[0], 1, 1
            w = b = None
            if n.op == "linear":
                W = np.asarray(n.weight, dtype=np.float32)
                src = n.inputs[0]
                while nodes[src].op == "flatten":
                    src = nodes[src].inputs[0]
                if len(nodes[src].shape) == 3:      # columns (c, h, w) -> (h, w, c)
                    c_, h_, w_ = nodes[src].shape
                    W = W.reshape(W.shape[0], c_, h_, w_).transpose(0, 2, 3, 1).reshape(W.shape[0], -1)
                w = _f32(W, self.device)
                b = _f32(n.bias, self.device)
            elif n.op == "conv":
                W = np.asarray(n.weight, dtype=np.float32)       # OIHW -> [kh][kw][O][I]
                v.kh, v.kw = W.shape[2], W.shape[3]
                v.stride, v.pad = n.stride, n.pad
                w = _f32(W.transpose(2, 3, 0, 1), self.device)
                b = _f32(n.bias, self.device)
            if w is not None:
                self._keep += [w, b]
                v.weight = w.data_ptr()
                v.bias = b.data_ptr()
            self._w.append(w)
        self.nodes_c = arr
        self.graph = vb_graph(len(nodes), arr)
        self.gp = ctypes.pointer(self.graph)
        self.n_nodes = len(nodes)
        self.sizes = [int(np.prod(s)) for s in self.shapes]

    def pack_linear(self, min_weights: int = 0):
        """Packed copies (vb_pack_linear) of the Linear nodes' weights whose input
        size is a multiple of 16 and that hold at least `min_weights` weights;
        vb_ibp then reads those for batches of up to 16.  Returns the bytes held."""
        total = 0
        for k, op in enumerate(self.ops):
            if op != "linear":
                continue
            n_out, n_in = self.nodes_c[k].c, self._w[k].shape[1]
            if n_in % 16 or n_out * n_in < min_weights:
                continue
            nb = ctypes.c_size_t(0)
            _check(lib().vb_pack_linear_bytes(n_out, n_in, ctypes.byref(nb)), "vb_pack_linear_bytes")
            dst = torch.empty(nb.value // 4, dtype=torch.float32, device=self.device)
            _check(lib().vb_pack_linear(self._w[k].data_ptr(), n_out, n_in, dst.data_ptr(), nb.value,
                                        _stream()), "vb_pack_linear")
            self._keep.append(dst)
            self.nodes_c[k].weight_packed = dst.data_ptr()
            total += nb.value
        return total

    def unpack_linear(self):
        """Drop the packed copies from the node descriptions (vb_ibp reads weight again)."""
        for k in range(self.n_nodes):
            self.nodes_c[k].weight_packed = None

    # ------------------------------------------------------------------
    def alloc_bounds(self, batch: int):
        lo = [None] + [torch.empty(batch, s, device=self.device) for s in self.sizes[1:]]
        hi = [None] + [torch.empty(batch, s, device=self.device) for s in self.sizes[1:]]
        return lo, hi

    def workspace_size(self, batch: int, m: int, method: str = "crown", region_start: int = 0,
                       alpha_rows: bool = False) -> int:
        out = ctypes.c_size_t(0)
        flags = METHODS[method] | (VB_ALPHA_ROWS if alpha_rows else 0)
        _check(lib().vb_workspace_size(self.gp, batch, m, flags, region_start or 0, ctypes.byref(out)),
               "vb_workspace_size")
        return int(out.value)

    def workspace(self, nbytes: int) -> torch.Tensor:
        return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)


def ibp(net: DeviceNet, x_center: torch.Tensor, eps: float, lo=None, hi=None, C: torch.Tensor = None,
        spec_lo=None, spec_hi=None, ws: torch.Tensor = None, x_radius: torch.Tensor = None):
    batch = x_center.shape[0]
    if lo is None:
        lo, hi = net.alloc_bounds(batch)
    m = 0 if C is None else C.shape[1]
    if C is not None and spec_lo is None:
        spec_lo = torch.empty(batch, m, device=net.device)
        spec_hi = torch.empty(batch, m, device=net.device)
    _check(lib().vb_ibp(net.gp, batch, _ptr(x_center), _ptr(x_radius), float(eps), _ptr_array(lo), _ptr_array(hi),
                       _ptr(C), m, _ptr(spec_lo), _ptr(spec_hi), _ptr(ws), 0 if ws is None else ws.numel(),
                       _stream()), "vb_ibp")
    return lo, hi, spec_lo, spec_hi


class AlphaLayout:
    """Compact alpha layout (vb_alpha_layout): per node an int32 column map [batch][size]
    (ReLU nodes; None elsewhere) and the row width of each node's state."""

    def __init__(self, index, width):
        self.index = index
        self.width = list(width)
        self._idx = _ptr_array(index)
        self._w = (ctypes.c_int32 * len(self.width))(*self.width)
        self._s = vb_alpha_compact(ctypes.cast(self._idx, ctypes.POINTER(ctypes.c_void_p)),
                                   ctypes.cast(self._w, ctypes.POINTER(ctypes.c_int32)))

    def ref(self):
        return ctypes.byref(self._s)


def _compact(layout: Optional[AlphaLayout]):
    return None if layout is None else layout.ref()


def alpha_layout(net: "DeviceNet", lo, hi) -> AlphaLayout:
    """Columns of the unstable neurons of every ReLU node (synchronises the stream)."""
    batch = lo[1].shape[0]
    index = [torch.empty(batch, s, dtype=torch.int32, device=net.device) if op == "relu" else None
             for op, s in zip(net.ops, net.sizes)]
    width = (ctypes.c_int32 * len(index))()
    ws = torch.empty(max(4 * batch, 256), dtype=torch.uint8, device=net.device)
    _check(lib().vb_alpha_layout(net.gp, batch, _ptr_array(lo), _ptr_array(hi), _ptr_array(index), width,
                                 _ptr(ws), ws.numel(), _stream()), "vb_alpha_layout")
    return AlphaLayout(index, list(width))


def crown_backward(net: DeviceNet, start: int, stop: int, lo, hi, x_center: torch.Tensor, eps: float,
                   ws: torch.Tensor, C: torch.Tensor = None, lb=None, ub=None, x_radius=None, linear=False,
                   alpha=None, lower_only=False, layout: Optional[AlphaLayout] = None):
    """lb, ub [batch][R] (ub None with lower_only or alpha: spec rows C only); with linear=True
    also (A, bias): the linear bounds over node `stop`, A [batch][rows][size_stop] and bias
    [batch][rows] (rows +r then -r, or only +r when one-sided, each bounded from below)."""
    batch = lo[start].shape[0]
    R = C.shape[1] if C is not None else net.sizes[start]
    one_side = C is not None and (lower_only or alpha is not None)
    if lb is None:
        lb = torch.empty(batch, R, device=net.device)
        ub = None if one_side else torch.empty(batch, R, device=net.device)
    A = bias = None
    if linear:
        rows = R if one_side else 2 * R
        A = torch.empty(batch, rows, net.sizes[stop], device=net.device)
        bias = torch.empty(batch, rows, device=net.device)
    _check(lib().vb_crown_backward(net.gp, batch, start, stop, _ptr(C), 0 if C is None else C.shape[1],
                                  _ptr_array(lo), _ptr_array(hi), _compact(layout),
                                  None if alpha is None else _ptr_array(alpha),
                                  _ptr(x_center), _ptr(x_radius), float(eps), _ptr(lb), _ptr(ub), _ptr(A),
                                  _ptr(bias), _ptr(ws), ws.numel(), _stream()),
           "vb_crown_backward")
    return (lb, ub, A, bias) if linear else (lb, ub)


def concretize(A: torch.Tensor, bias: Optional[torch.Tensor], center: torch.Tensor, eps: float, rows_per_batch: int,
               radius: torch.Tensor = None, lb=None, ub=None):
    rows, n = A.shape
    if lb is None:
        lb = torch.empty(rows, device=A.device)
        ub = torch.empty(rows, device=A.device)
    _check(lib().vb_concretize(rows, n, rows_per_batch, _ptr(A), _ptr(bias), _ptr(center), _ptr(radius), float(eps),
                              _ptr(lb), _ptr(ub), _stream()), "vb_concretize")
    return lb, ub


def crown(net: DeviceNet, x_center: torch.Tensor, eps: float, C: torch.Tensor, method: str = "crown",
          region_start: Optional[int] = None, ws: torch.Tensor = None, out=None, x_radius=None):
    """Whole pipeline (vb_crown).  Returns dict of device tensors:
    lo/hi per node (channels-last), ibp_lb/ibp_ub and lb/ub [B][m]."""
    batch = x_center.shape[0]
    m = C.shape[1]
    if out is None:
        lo, hi = net.alloc_bounds(batch)
        out = {"lo": lo, "hi": hi}
        for k in ("ibp_lb", "ibp_ub", "lb", "ub"):
            out[k] = torch.empty(batch, m, device=net.device)
    if ws is None:
        ws = net.workspace(net.workspace_size(batch, m, method, region_start or 0))
    _check(lib().vb_crown(net.gp, batch, _ptr(x_center), _ptr(x_radius), float(eps), METHODS[method],
                         region_start or 0, _ptr_array(out["lo"]), _ptr_array(out["hi"]), _ptr(C), m,
                         _ptr(out["ibp_lb"]), _ptr(out["ibp_ub"]), _ptr(out["lb"]), _ptr(out["ub"]), _ptr(ws),
                         ws.numel(), _stream()), "vb_crown")
    return out


def crown_noalloc(net: DeviceNet, x_center: torch.Tensor, eps: float, C: torch.Tensor, method: str = "crown",
                  region_start: Optional[int] = None, out=None, x_radius=None):
    """vb_crown on the library's fixed device scratch (vb_crown_noalloc): no workspace
    argument and no device allocation inside the call (the caller's outputs excepted:
    pass `out` to allocate nothing at all)."""
    batch = x_center.shape[0]
    m = C.shape[1]
    if out is None:
        lo, hi = net.alloc_bounds(batch)
        out = {"lo": lo, "hi": hi}
        for k in ("ibp_lb", "ibp_ub", "lb", "ub"):
            out[k] = torch.empty(batch, m, device=net.device)
    _check(lib().vb_crown_noalloc(net.gp, batch, _ptr(x_center), _ptr(x_radius), float(eps), METHODS[method],
                                  region_start or 0, _ptr_array(out["lo"]), _ptr_array(out["hi"]), _ptr(C), m,
                                  _ptr(out["ibp_lb"]), _ptr(out["ibp_ub"]), _ptr(out["lb"]), _ptr(out["ub"]),
                                  _stream()), "vb_crown_noalloc")
    return out


def verify(lb: torch.Tensor, verified: torch.Tensor = None, count: torch.Tensor = None):
    """vb_verify: per input, 1 if every spec lower bound is positive (the property is
    proved for the whole domain), and the number of verified inputs (device int32)."""
    batch, m = lb.shape
    if verified is None:
        verified = torch.empty(batch, dtype=torch.int32, device=lb.device)
    if count is None:
        count = torch.empty(1, dtype=torch.int32, device=lb.device)
    _check(lib().vb_verify(batch, m, _ptr(lb), _ptr(verified), _ptr(count), _stream()), "vb_verify")
    return verified, count


def alpha_state(net: DeviceNet, batch: int, m: int, layout: Optional[AlphaLayout] = None):
    """Device tensors alpha, adam_m, adam_v per node ([batch][m][size] for ReLU nodes, or
    [batch][m][width] in a compact layout (None for width 0); None elsewhere)."""
    def width(k, s):
        return s if layout is None else layout.width[k]
    mk = lambda: [torch.empty(batch, m, width(k, s), device=net.device)
                  if op == "relu" and width(k, s) > 0 else None
                  for k, (op, s) in enumerate(zip(net.ops, net.sizes))]
    return mk(), mk(), mk()


def alpha_init(net: DeviceNet, lo, hi, alpha, adam_m, adam_v, m: int, layout: Optional[AlphaLayout] = None):
    batch = lo[1].shape[0]
    _check(lib().vb_alpha_init(net.gp, batch, m, _ptr_array(lo), _ptr_array(hi), _compact(layout),
                               _ptr_array(alpha), _ptr_array(adam_m), _ptr_array(adam_v), _stream()),
           "vb_alpha_init")


def alpha_step(net: DeviceNet, C: torch.Tensor, lo, hi, x_center: torch.Tensor, eps: float, alpha, adam_m, adam_v,
               step: int, lr: float, lb_out: torch.Tensor, best_lb: Optional[torch.Tensor], ws: torch.Tensor,
               beta1: float = 0.9, beta2: float = 0.999, adam_eps: float = 1e-8, x_radius=None,
               layout: Optional[AlphaLayout] = None):
    batch, m = C.shape[0], C.shape[1]
    _check(lib().vb_alpha_step(net.gp, batch, _ptr(C), m, _ptr_array(lo), _ptr_array(hi), _ptr(x_center),
                              _ptr(x_radius), float(eps), _compact(layout), _ptr_array(alpha), _ptr_array(adam_m),
                              _ptr_array(adam_v),
                              step, lr, beta1, beta2, adam_eps, _ptr(lb_out), _ptr(best_lb), _ptr(ws), ws.numel(),
                              _stream()), "vb_alpha_step")
    return lb_out


def alpha_step_rows(net: DeviceNet, start: int, C: Optional[torch.Tensor], lo, hi, x_center: torch.Tensor,
                    eps: float, alpha, adam_m, adam_v, step: int, lr: float, ws: torch.Tensor, lb_out=None,
                    best_lb=None, ub_out=None, best_ub=None, beta1: float = 0.9, beta2: float = 0.999,
                    adam_eps: float = 1e-8, x_radius=None, layout: Optional[AlphaLayout] = None,
                    beta=None):
    """vb_alpha_step_rows: one alpha-CROWN step on spec rows C over node `start`, or
    (C None) on the identity rows of `start` (l and u of every neuron).  beta: None, or
    (split, beta, beta_m, beta_v) per-node lists (split constraints of sub-domains)."""
    batch = x_center.shape[0]
    m = 0 if C is None else C.shape[1]
    bref = None
    if beta is not None:
        arrs = [_ptr_array(a) for a in beta]
        bst = vb_beta(*[ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p)) for a in arrs])
        bref = ctypes.byref(bst)
    _check(lib().vb_alpha_step_rows(net.gp, batch, start, _ptr(C), m, _ptr_array(lo), _ptr_array(hi),
                                    _ptr(x_center), _ptr(x_radius), float(eps), _compact(layout), bref,
                                    _ptr_array(alpha), _ptr_array(adam_m), _ptr_array(adam_v), step, lr, beta1, beta2,
                                    adam_eps, _ptr(lb_out), _ptr(best_lb), _ptr(ub_out), _ptr(best_ub), _ptr(ws),
                                    ws.numel(), _stream()), "vb_alpha_step_rows")


def apply_splits(net: DeviceNet, split, lo, hi):
    """vb_apply_splits: clamp the bounds of split neurons (in place)."""
    batch = lo[1].shape[0]
    _check(lib().vb_apply_splits(net.gp, batch, _ptr_array(split), _ptr_array(lo), _ptr_array(hi), _stream()),
           "vb_apply_splits")


def bab(net: DeviceNet, x_center: torch.Tensor, eps: float, C: torch.Tensor, lo, hi, steps: int = 20,
        lr: float = 0.1, batch: int = 8, max_domains: int = 256, x_radius=None, ws: torch.Tensor = None,
        beta1: float = 0.9, beta2: float = 0.999, adam_eps: float = 1e-8):
    """vb_bab: branch and bound with beta-CROWN for ONE input: x_center [n0] (or [1][n0]),
    C [m][n_out], lo / hi the root's node bounds [1][size].  Returns (verified (bool),
    sub-domains bounded, root best bound [m])."""
    m = C.shape[-2] if C.dim() == 3 else C.shape[0]
    params = vb_bab_params(steps, lr, beta1, beta2, adam_eps, batch, max_domains)
    if ws is None:
        need = ctypes.c_size_t(0)
        _check(lib().vb_bab_workspace_size(net.gp, m, batch, ctypes.byref(need)), "vb_bab_workspace_size")
        ws = net.workspace(int(need.value))
    verdict, doms = ctypes.c_int32(), ctypes.c_int32()
    root = torch.empty(m, device=net.device)
    _check(lib().vb_bab(net.gp, _ptr(x_center), _ptr(x_radius), float(eps), _ptr(C), m, _ptr_array(lo),
                        _ptr_array(hi), ctypes.byref(params), ctypes.byref(verdict), ctypes.byref(doms), _ptr(root),
                        _ptr(ws), ws.numel(), _stream()), "vb_bab")
    return bool(verdict.value), int(doms.value), root


def relu_inputs_refined(net: DeviceNet):
    """ReLU inputs whose bounds CROWN refines (more than one affine step from the input), in order."""
    out = []
    for k, op in enumerate(net.ops):
        if op != "relu":
            continue
        z = net.inputs[k][0]
        src = net.inputs[z][0] if net.ops[z] in ("linear", "conv") else None
        while src is not None and net.ops[src] == "flatten":
            src = net.inputs[src][0]
        if src == 0:
            continue
        out.append(z)
    return out


def alpha_intermediate(net: DeviceNet, x_center: torch.Tensor, eps: float, lo, hi, steps: int, lr: float,
                       ws: torch.Tensor, x_radius=None, trace: Optional[dict] = None):
    """alpha-CROWN intermediate bounds: for every refined ReLU input z in order, the
    identity rows of z are optimised (vb_alpha_init, `steps` calls of
    vb_alpha_step_rows with the Adam update, one evaluation), and the best l and u
    over the iterates are written into lo[z], hi[z] (which the later layers then
    relax with).  lo / hi must hold bounds of every node (e.g. from vb_ibp).
    With `trace` (a dict), trace[z] receives the l and u of every evaluation
    ([steps+1][batch][size] each)."""
    batch = x_center.shape[0]
    for z in relu_inputs_refined(net):
        n = net.sizes[z]
        R = 2 * n
        below = [k for k, op in enumerate(net.ops) if op == "relu" and k < z]
        mk = lambda: [torch.empty(batch, R, net.sizes[k], device=net.device) if k in below else None
                      for k in range(net.n_nodes)]
        alpha, am, av = mk(), mk(), mk()
        alpha_init(net, lo, hi, alpha, am, av, R)
        ls = torch.empty(steps + 1, batch, n, device=net.device)
        us = torch.empty(steps + 1, batch, n, device=net.device)
        for t in range(1, steps + 1):
            alpha_step_rows(net, z, None, lo, hi, x_center, eps, alpha, am, av, t, lr, ws, lb_out=ls[t - 1],
                            best_lb=lo[z], ub_out=us[t - 1], best_ub=hi[z], x_radius=x_radius)
        alpha_step_rows(net, z, None, lo, hi, x_center, eps, alpha, am, av, 0, lr, ws, lb_out=ls[steps],
                        best_lb=lo[z], ub_out=us[steps], best_ub=hi[z], x_radius=x_radius)
        if trace is not None:
            trace[z] = (ls, us)
    return lo, hi


def alpha_crown(net: DeviceNet, x_center: torch.Tensor, eps: float, C: torch.Tensor, lo, hi, steps: int,
                lr: float, ws: torch.Tensor = None, state=None, lb_steps: torch.Tensor = None,
                best: torch.Tensor = None, x_radius=None, layout: Optional[AlphaLayout] = None):
    """alpha-CROWN over fixed intermediate bounds lo/hi: vb_alpha_init, then `steps` calls of
    vb_alpha_step (evaluate, gradient, Adam ascent; the first sets `best`) and one
    evaluation-only call.  steps must be >= 1.  With a layout (alpha_layout) the state is
    compact (unstable neurons only).
    Returns (best [B][m], lb per evaluation [steps+1][B][m], (alpha, adam_m, adam_v))."""
    batch, m = C.shape[0], C.shape[1]
    if state is None:
        state = alpha_state(net, batch, m, layout)
    alpha, am, av = state
    if ws is None:
        ws = net.workspace(net.workspace_size(batch, m, "ibp"))
    if lb_steps is None:
        lb_steps = torch.empty(steps + 1, batch, m, device=net.device)
    if best is None:
        best = torch.empty(batch, m, device=net.device)
    alpha_init(net, lo, hi, alpha, am, av, m, layout=layout)
    for t in range(1, steps + 1):
        alpha_step(net, C, lo, hi, x_center, eps, alpha, am, av, t, lr, lb_steps[t - 1], best, ws, x_radius=x_radius,
                   layout=layout)
    alpha_step(net, C, lo, hi, x_center, eps, alpha, am, av, 0, lr, lb_steps[steps], best, ws, x_radius=x_radius,
               layout=layout)
    return best, lb_steps, state


def profile_start():
    _check(lib().vb_profile_start(), "vb_profile_start")


def profile_stop():
    """(total ms, total algorithmic FLOPs, launches) of the relaxation-epilogue GEMMs since profile_start()."""
    ms, fl, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int64()
    _check(lib().vb_profile_stop(ctypes.byref(ms), ctypes.byref(fl), ctypes.byref(n)), "vb_profile_stop")
    return ms.value, fl.value, n.value


def profile_records(n):
    """Per-launch records of the last profile_stop(): list of dicts (ms, flops, epi,
    patch, M, N, K, taps)."""
    out = []
    for i in range(n):
        ms, fl = ctypes.c_double(), ctypes.c_double()
        info = (ctypes.c_int32 * 6)()
        _check(lib().vb_profile_record(i, ctypes.byref(ms), ctypes.byref(fl), info), "vb_profile_record")
        out.append(dict(ms=ms.value, flops=fl.value, **dict(zip(("epi", "patch", "M", "N", "K", "taps"), list(info)))))
    return out


def prepare(wl, device="cuda"):
    """Device copies of a workload's network, input centres and spec matrix."""
    net = DeviceNet(wl.nodes, device)
    x = _f32(to_channels_last(wl.x0).reshape(wl.batch, -1), net.device)
    C = _f32(wl.C, net.device)
    return net, x, C
