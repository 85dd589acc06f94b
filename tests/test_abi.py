"""C-ABI contract on the CPU: the library loads, exports every declared symbol,
and rejects bad arguments on the host before touching a device."""
import ctypes
import os
import re

import pytest

from helpers import ROOT, ensure_built

ensure_built()
import linear_bound_propagation_amd as lbp  # noqa: E402

HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


def _declared(path):
    return set(re.findall(r"^(?:vb_status|const char\*|int32_t)\s+(vb_\w+)\s*\(", open(path).read(), flags=re.M))


def test_exports_every_declared_symbol():
    declared = set()
    for h in HEADERS:
        declared |= _declared(h)
    assert declared == set(lbp.EXPORTS) | set(lbp.TESTING_EXPORTS)
    lib = ctypes.CDLL(lbp.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def _graph(nodes):
    arr = (lbp.vb_node * len(nodes))()
    for i, nd in enumerate(nodes):
        for k, v in nd.items():
            setattr(arr[i], k, v)
    g = lbp.vb_graph(len(nodes), arr)
    return g, arr


def _mlp_graph(weight=16):
    return _graph([dict(op=0, in0=-1, in1=-1, c=4, h=1, w=1),
                   dict(op=1, in0=0, in1=-1, c=5, h=1, w=1, weight=weight, bias=32),
                   dict(op=3, in0=1, in1=-1, c=5, h=1, w=1),
                   dict(op=1, in0=2, in1=-1, c=3, h=1, w=1, weight=weight, bias=32)])


def ws_size(g, batch=2, m=2, method=1, region=0):
    out = ctypes.c_size_t(0)
    st = lbp.lib().vb_workspace_size(ctypes.pointer(g), batch, m, method, region, ctypes.byref(out))
    return st, out.value


def test_workspace_size_and_shape_errors():
    g, keep = _mlp_graph()
    st, n = ws_size(g)
    assert st == 0 and n > 0
    # whole-batch workspace grows with the batch
    assert ws_size(g, batch=8)[1] > n
    # NULL weight, bad input index, bad op, shape mismatch, bad method
    g2, k2 = _mlp_graph(weight=None)
    assert ws_size(g2)[0] == -1 and b"weight is NULL" in lbp.lib().vb_last_error()
    g3, k3 = _graph([dict(op=0, in0=-1, in1=-1, c=4, h=1, w=1), dict(op=1, in0=3, in1=-1, c=5, h=1, w=1, weight=16)])
    assert ws_size(g3)[0] == -2
    g4, k4 = _graph([dict(op=0, in0=-1, in1=-1, c=4, h=1, w=1), dict(op=9, in0=0, in1=-1, c=5, h=1, w=1)])
    assert ws_size(g4)[0] == -1
    g5, k5 = _graph([dict(op=0, in0=-1, in1=-1, c=4, h=1, w=1), dict(op=3, in0=0, in1=-1, c=5, h=1, w=1)])
    assert ws_size(g5)[0] == -2 and b"relu shape" in lbp.lib().vb_last_error()
    assert ws_size(g, method=7)[0] == -1
    assert ws_size(g, batch=0)[0] == -1


def test_conv_shape_checks():
    base = dict(op=0, in0=-1, in1=-1, c=3, h=8, w=8)
    ok = dict(op=2, in0=0, in1=-1, c=4, h=4, w=4, kh=3, kw=3, stride=2, pad=1, weight=16, bias=0)
    g, k = _graph([base, ok])
    assert ws_size(g, m=0, method=0)[0] == 0
    bad = dict(ok, h=5)
    g, k = _graph([base, bad])
    assert ws_size(g, m=0, method=0)[0] == -2 and b"conv output" in lbp.lib().vb_last_error()
    big = dict(ok, kh=5, kw=5, h=3, w=3)
    g, k = _graph([base, big])
    assert ws_size(g, m=0, method=0)[0] == -5


def test_entry_points_reject_bad_arguments_without_launching():
    g, keep = _mlp_graph()
    gp = ctypes.pointer(g)
    P = ctypes.c_void_p
    nulls = (ctypes.c_void_p * 4)()
    # NULL x_center
    assert lbp.lib().vb_crown(gp, 2, None, None, 0.1, 1, 0, nulls, nulls, None, 0, None, None, None, None,
                             P(64), 1 << 20, None) == -1
    # NULL bounds storage for a node
    assert lbp.lib().vb_crown(gp, 2, P(64), None, 0.1, 1, 0, nulls, nulls, None, 0, None, None, None, None,
                             P(64), 1 << 20, None) == -1
    assert b"bounds storage" in lbp.lib().vb_last_error()
    # negative eps without a radius array
    assert lbp.lib().vb_ibp(gp, 2, P(64), None, -1.0, nulls, nulls, None, 0, None, None, None, 0, None) == -1
    # crown_backward: stop >= start, missing workspace
    assert lbp.lib().vb_crown_backward(gp, 2, 1, 1, None, 0, nulls, nulls, None, None, P(64), None, 0.1, None, None, None, None,
                                      P(64), 1 << 20, None) == -1
    assert lbp.lib().vb_crown_backward(gp, 2, 3, 0, None, 0, nulls, nulls, None, None, P(64), None, 0.1, None, None, None, None,
                                      None, 0, None) == -1
    # crown_backward: bias_out without A_out, and no output at all
    assert lbp.lib().vb_crown_backward(gp, 2, 3, 0, None, 0, nulls, nulls, None, None, P(64), None, 0.1, None, None, None,
                                      P(64), P(64), 1 << 20, None) == -1
    assert b"bias_out needs A_out" in lbp.lib().vb_last_error()
    assert lbp.lib().vb_crown_backward(gp, 2, 3, 0, None, 0, nulls, nulls, None, None, P(64), None, 0.1, None, None, None, None,
                                      P(64), 1 << 20, None) == -1
    assert b"nothing to compute" in lbp.lib().vb_last_error()
    # alpha needs spec rows and a one-sided call
    assert lbp.lib().vb_crown_backward(gp, 2, 3, 0, None, 0, nulls, nulls, None, nulls, P(64), None, 0.1, P(64), None,
                                      None, None, P(64), 1 << 20, None) == -1
    assert b"alpha needs spec rows" in lbp.lib().vb_last_error()
    # compact alpha layout: needs alpha; widths within the node size; layout call checks
    idx = (ctypes.c_void_p * 4)(None, None, 64, None)
    wid = (ctypes.c_int32 * 4)(0, 0, 5, 0)
    cmp = lbp.vb_alpha_compact(ctypes.cast(idx, ctypes.POINTER(ctypes.c_void_p)),
                               ctypes.cast(wid, ctypes.POINTER(ctypes.c_int32)))
    assert lbp.lib().vb_crown_backward(gp, 2, 3, 0, P(64), 2, nulls, nulls, ctypes.byref(cmp), None, P(64), None,
                                      0.1, P(64), None, None, None, P(64), 1 << 20, None) == -1
    assert b"needs alpha" in lbp.lib().vb_last_error()
    wid[2] = 1 << 20  # wider than the ReLU node
    al = (ctypes.c_void_p * 4)(None, None, 64, None)
    assert lbp.lib().vb_crown_backward(gp, 2, 3, 0, P(64), 2, nulls, nulls, ctypes.byref(cmp), al, P(64), None,
                                      0.1, P(64), None, None, None, P(64), 1 << 20, None) == -1
    assert b"compact width" in lbp.lib().vb_last_error()
    width = (ctypes.c_int32 * 4)()
    assert lbp.lib().vb_alpha_layout(gp, 0, nulls, nulls, idx, width, P(64), 1024, None) == -1
    bounds = (ctypes.c_void_p * 4)(None, 64, 64, 64)
    assert lbp.lib().vb_alpha_layout(gp, 2, bounds, bounds, idx, width, P(64), 4, None) == -3
    assert lbp.lib().vb_alpha_layout(gp, 2, bounds, bounds, nulls, width, P(64), 1024, None) == -1
    assert b"index storage" in lbp.lib().vb_last_error()
    # workspace too small: reported before any launch
    bounds = (ctypes.c_void_p * 4)(None, 64, 64, 64)
    assert lbp.lib().vb_crown(gp, 2, P(64), None, 0.1, 1, 0, bounds, bounds, P(64), 2, None, None, P(64), P(64),
                             P(64), 16, None) in (-3,)
    assert b"too small" in lbp.lib().vb_last_error()
    # concretize argument checks
    assert lbp.lib().vb_concretize(0, 4, 1, P(64), None, P(64), None, 0.1, None, None, None) == -1
    assert lbp.lib().vb_concretize(2, 4, 1, None, None, P(64), None, 0.1, None, None, None) == -1


def test_fastdiv_magic_numbers_are_exact():
    """The library's own division by a runtime constant (its multiply-high magic
    numbers, exported for this test) equals integer division."""
    import numpy as np
    f = lbp.lib().vb_testing_fastdiv
    f.restype = ctypes.c_int32
    f.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_uint32)]
    rng = np.random.default_rng(0)
    for d in list(range(1, 300)) + [1024, 3072, 4097, 65536, 65537, 99991, 2 ** 20 + 7, 2 ** 30 + 1, 2 ** 31 - 1]:
        xs = np.concatenate([np.arange(0, 3000), rng.integers(0, 2 ** 31, 3000),
                             np.array([2 ** 31 - 1, d - 1, d, d + 1, 2 * d - 1, 2 * d])])
        xs = xs[(xs >= 0) & (xs < 2 ** 31)].astype(np.int32)
        q = np.empty_like(xs)
        mul, shr = ctypes.c_uint32(), ctypes.c_uint32()
        assert f(d, xs.ctypes.data, xs.size, q.ctypes.data, ctypes.byref(mul), ctypes.byref(shr)) == 0
        assert np.array_equal(q, xs // d), d
        assert (d == 1) == (mul.value == 0)
    xs = np.array([-1], dtype=np.int32)
    q = np.empty_like(xs)
    assert f(3, xs.ctypes.data, 1, q.ctypes.data, None, None) == -1
    assert f(0, xs.ctypes.data, 0, q.ctypes.data, None, None) == -1


def test_big_tiles_only_for_plain_epilogues():
    """256-wide tiles are chosen for large convolutions with the store, relaxation or
    concretisation epilogue only; the alpha-CROWN adjoint never takes them."""
    f = lbp.lib().vb_testing_conv_tile_n
    f.restype = ctypes.c_int32
    f.argtypes = [ctypes.c_int32] * 6
    rows = 4096  # 4096 rows x 64 pixels / 256 = 1024 M-tiles
    for mode in (0, 1, 2):
        assert f(mode, rows, 8, 8, 256, 256) == 256, mode
        assert f(mode, 8, 8, 8, 256, 256) == 128, mode      # too few tiles for two per CU
        assert f(mode, rows, 8, 8, 128, 256) == 128, mode   # N = c_in = 128
    assert f(4, rows, 8, 8, 256, 256) == 128
    assert f(4, rows, 8, 8, 256, 64) == 64
    assert f(3, rows, 8, 8, 256, 256) == -1
    assert f(0, 0, 8, 8, 256, 256) == -1


def test_crown_backward_workspace_checked_before_any_launch():
    """A workspace smaller than the weight copies plus one batch element is rejected
    with VB_ENOMEM before anything is enqueued (no stream, no device pointers read)."""
    g, keep = _mlp_graph()
    gp = ctypes.pointer(g)
    P = ctypes.c_void_p
    bounds = (ctypes.c_void_p * 4)(None, 64, 64, 64)
    for C, m in ((None, 0), (P(64), 2)):
        st = lbp.lib().vb_crown_backward(gp, 2, 3, 0, C, m, bounds, bounds, None, None, P(64), None, 0.1, P(64),
                                        P(64), None, None, P(64), 64, None)
        assert st == -3, st
        assert b"too small" in lbp.lib().vb_last_error()


def test_ibp_checks_every_node_before_launching():
    """IBP validates the whole graph first: a ReLU on the input node, or missing storage
    for a node whose bounds another node reads, fails with nothing enqueued; storage may
    be omitted for a node nothing reads (the last one)."""
    P = ctypes.c_void_p
    g, keep = _graph([dict(op=0, in0=-1, in1=-1, c=4, h=1, w=1),
                      dict(op=1, in0=0, in1=-1, c=4, h=1, w=1, weight=16, bias=32),
                      dict(op=3, in0=0, in1=-1, c=4, h=1, w=1)])
    b = (ctypes.c_void_p * 3)(None, 64, 64)
    assert lbp.lib().vb_ibp(ctypes.pointer(g), 2, P(64), None, 0.1, b, b, None, 0, None, None, None, 0, None) == -5
    g, keep = _mlp_graph()
    miss = (ctypes.c_void_p * 4)(None, None, 64, 64)    # node 1 feeds the ReLU
    assert lbp.lib().vb_ibp(ctypes.pointer(g), 2, P(64), None, 0.1, miss, miss, None, 0, None, None, None, 0,
                            None) == -1
    assert b"is read" in lbp.lib().vb_last_error() or b"are read" in lbp.lib().vb_last_error()
    half = (ctypes.c_void_p * 4)(None, 64, 64, None)
    other = (ctypes.c_void_p * 4)(None, 64, 64, 64)
    assert lbp.lib().vb_ibp(ctypes.pointer(g), 2, P(64), None, 0.1, half, other, None, 0, None, None, None, 0,
                            None) == -1
    assert b"only one of" in lbp.lib().vb_last_error()


def test_pack_linear_checks_arguments_before_any_launch():
    """vb_pack_linear_bytes gives whole 16-row blocks of n_in floats; both calls reject
    n_in not a multiple of 16, NULL or misaligned pointers and a short destination
    before enqueueing anything (fake device addresses: nothing is dereferenced)."""
    L = lbp.lib()
    nb = ctypes.c_size_t(0)
    assert L.vb_pack_linear_bytes(100, 4096, ctypes.byref(nb)) == 0 and nb.value == 112 * 4096 * 4
    assert L.vb_pack_linear_bytes(16, 16, ctypes.byref(nb)) == 0 and nb.value == 16 * 16 * 4
    assert L.vb_pack_linear_bytes(100, 4090, ctypes.byref(nb)) == -1
    assert L.vb_pack_linear_bytes(0, 16, ctypes.byref(nb)) == -1
    assert L.vb_pack_linear_bytes(16, 16, None) == -1
    need = 112 * 4096 * 4
    assert L.vb_pack_linear(16, 100, 4090, 256, need, None) == -1          # n_in
    assert L.vb_pack_linear(None, 100, 4096, 256, need, None) == -1        # weight NULL
    assert L.vb_pack_linear(16, 100, 4096, None, need, None) == -1         # dst NULL
    assert L.vb_pack_linear(16, 100, 4096, 260, need, None) == -1          # dst misaligned
    assert L.vb_pack_linear(16, 100, 4096, 256, need - 4, None) == -3      # too small


def test_packed_weights_only_on_linear_nodes():
    g, keep = _mlp_graph()
    assert ws_size(g)[0] == 0
    keep[1].weight_packed = 4096                       # a Linear node: accepted
    assert ws_size(g)[0] == 0
    keep[1].weight_packed = 4100                       # misaligned
    assert ws_size(g)[0] == -1
    keep[1].weight_packed = None
    keep[2].weight_packed = 4096                       # a ReLU node
    assert ws_size(g)[0] == -1
