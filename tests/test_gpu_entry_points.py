"""GPU parity of the stand-alone C-ABI calls (vb_concretize, vb_crown_backward,
vb_alpha_init) and of the whole pipeline on degenerate cases, against the float64
oracle.

vb_crown_backward is given node bounds from the oracle's IBP rounded to fp32, and
the oracle runs on the same rounded bounds, so both sides take the same
relaxation decisions."""
import numpy as np
import pytest
import torch

import workloads as wk
from helpers import assert_close, compare_workload, ensure_built, nhwc
from oracle import Oracle, backward, concretize, crown_bounds, ibp as oracle_ibp
from oracle.alpha import alpha_init as oracle_alpha_init, compact_columns

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lbp():
    ensure_built()
    import linear_bound_propagation_amd as m
    return m


def _f64(a):
    return torch.as_tensor(np.asarray(a, np.float64))


# ---------------------------------------------------------------------------
# vb_concretize

@pytest.mark.parametrize("n", [1001, 1024])       # scalar and float4 paths
@pytest.mark.parametrize("radius_array", [False, True])
def test_concretize(lbp, n, radius_array):
    rng = np.random.default_rng([7, n, int(radius_array)])
    batch, rpb = 3, 37
    A = rng.standard_normal((batch * rpb, n)).astype(np.float32)
    bias = rng.standard_normal(batch * rpb).astype(np.float32)
    c = rng.random((batch, n)).astype(np.float32)
    r = (rng.random((batch, n)) * 0.05).astype(np.float32)
    eps = 0.03
    dev = "cuda:0"
    t = lambda a: torch.as_tensor(a, device=dev)
    lb, ub = lbp.concretize(t(A), t(bias), t(c), eps, rpb, radius=t(r) if radius_array else None)
    torch.cuda.synchronize()
    ref_lb = np.zeros(batch * rpb)
    ref_ub = np.zeros(batch * rpb)
    for b in range(batch):
        sl = slice(b * rpb, (b + 1) * rpb)
        rr = _f64(r[b]) if radius_array else torch.full((n,), float(np.float32(eps)), dtype=torch.float64)
        ref_lb[sl] = concretize(_f64(A[sl]), _f64(bias[sl]), _f64(c[b]), rr).numpy()
        ref_ub[sl] = -concretize(-_f64(A[sl]), -_f64(bias[sl]), _f64(c[b]), rr).numpy()
    assert_close(lb, ref_lb, "lb")
    assert_close(ub, ref_ub, "ub")


# ---------------------------------------------------------------------------
# vb_crown_backward

def _fp32_bounds(wl):
    """Oracle IBP bounds rounded to fp32: (oracle lists [B][*shape] float64, device lists)."""
    on = Oracle(wl.nodes)
    lo, hi = oracle_ibp(on, wl.x0, wl.eps)
    lo = [x.float().double() for x in lo]
    hi = [x.float().double() for x in hi]
    return on, lo, hi


def _to_device(lbp, net, wl, lo, hi):
    dlo, dhi = net.alloc_bounds(wl.batch)
    for k, nd in enumerate(wl.nodes):
        if k == 0 or dlo[k] is None:
            continue
        src = k
        while wl.nodes[src].op == "flatten":   # on the device a flatten keeps its producer's [h][w][c] order
            src = wl.nodes[src].inputs[0]
        shape = wl.nodes[src].shape
        dlo[k].copy_(torch.as_tensor(nhwc(lo[src], shape), dtype=torch.float32).reshape(dlo[k].shape))
        dhi[k].copy_(torch.as_tensor(nhwc(hi[src], shape), dtype=torch.float32).reshape(dhi[k].shape))
    return dlo, dhi


def _identity(shape, sign):
    n = int(np.prod(shape))
    return (sign * torch.eye(n, dtype=torch.float64)).reshape((n,) + tuple(shape))


def _oracle_rows(on, lo, hi, wl, b, start, rows, stop, radius=None):
    if stop == 0:
        c = _f64(wl.x0[b])
        r = torch.full_like(c, float(np.float32(wl.eps))) if radius is None else _f64(radius[b])
    else:
        c, r = (lo[stop][b] + hi[stop][b]) / 2, (hi[stop][b] - lo[stop][b]) / 2
    return backward(on, lo, hi, b, start, rows, stop, c, r)


CASES = {
    "mlp": lambda: wk.tiny_mlp([30, 50, 41, 7], 0.08, 21, batch=3),
    "cnn": lambda: wk.cnn(2, 0.02, 22, convs=((8, 1), (16, 2), (16, 1)), fcs=(24, 5), in_shape=(3, 9, 9)),
}


@pytest.mark.parametrize("case", ["mlp", "cnn"])
def test_crown_backward_identity_and_spec_rows(lbp, case):
    wl = CASES[case]()
    on, lo, hi = _fp32_bounds(wl)
    net, x, C = lbp.prepare(wl)
    dlo, dhi = _to_device(lbp, net, wl, lo, hi)
    ws = net.workspace(net.workspace_size(wl.batch, wl.m, "crown"))
    relu_in = [nd.inputs[0] for nd in wl.nodes if nd.op == "relu"]
    L = len(wl.nodes) - 1
    for start in relu_in[1:]:                       # identity rows over a pre-activation node
        print(f"{case}: identity rows over node {start}", flush=True)
        lb, ub = lbp.crown_backward(net, start, 0, dlo, dhi, x, float(wl.eps), ws)
        torch.cuda.synchronize()
        shape = wl.nodes[start].shape
        for b in range(wl.batch):
            rl = _oracle_rows(on, lo, hi, wl, b, start, _identity(shape, 1.0), 0)
            ru = -_oracle_rows(on, lo, hi, wl, b, start, _identity(shape, -1.0), 0)
            assert_close(lb[b], nhwc(rl.reshape((1,) + tuple(shape)), shape)[0], f"lb node {start} input {b}")
            assert_close(ub[b], nhwc(ru.reshape((1,) + tuple(shape)), shape)[0], f"ub node {start} input {b}")
    # spec rows over the last node
    lb, ub = lbp.crown_backward(net, L, 0, dlo, dhi, x, float(wl.eps), ws, C=C)
    torch.cuda.synchronize()
    for b in range(wl.batch):
        Cb = _f64(wl.C[b])
        assert_close(lb[b], _oracle_rows(on, lo, hi, wl, b, L, Cb, 0), f"spec lb input {b}")
        assert_close(ub[b], -_oracle_rows(on, lo, hi, wl, b, L, -Cb, 0), f"spec ub input {b}")


def test_crown_backward_box_domain_and_radius_array(lbp):
    """stop > 0: the domain is the box of a ReLU node's bounds; stop = 0 with a
    per-element input radius."""
    wl = CASES["mlp"]()
    on, lo, hi = _fp32_bounds(wl)
    net, x, C = lbp.prepare(wl)
    dlo, dhi = _to_device(lbp, net, wl, lo, hi)
    relus = [k for k, nd in enumerate(wl.nodes) if nd.op == "relu"]
    L = len(wl.nodes) - 1
    stop = relus[0]
    ws = net.workspace(net.workspace_size(wl.batch, wl.m, "hybrid", stop))
    lb, ub = lbp.crown_backward(net, L, stop, dlo, dhi, x, float(wl.eps), ws, C=C)
    torch.cuda.synchronize()
    for b in range(wl.batch):
        Cb = _f64(wl.C[b])
        assert_close(lb[b], _oracle_rows(on, lo, hi, wl, b, L, Cb, stop), f"box lb input {b}")
        assert_close(ub[b], -_oracle_rows(on, lo, hi, wl, b, L, -Cb, stop), f"box ub input {b}")
    # per-element radius at the input (any box: the oracle takes it as the domain)
    rad = (np.random.default_rng(5).random(wl.x0.shape) * 0.1).astype(np.float32)
    ws = net.workspace(net.workspace_size(wl.batch, wl.m, "crown"))
    lb, ub = lbp.crown_backward(net, L, 0, dlo, dhi, x, 0.0, ws, C=C,
                                x_radius=torch.as_tensor(rad, device=x.device))
    torch.cuda.synchronize()
    for b in range(wl.batch):
        Cb = _f64(wl.C[b])
        assert_close(lb[b], _oracle_rows(on, lo, hi, wl, b, L, Cb, 0, rad), f"radius lb input {b}")
        assert_close(ub[b], -_oracle_rows(on, lo, hi, wl, b, L, -Cb, 0, rad), f"radius ub input {b}")


@pytest.mark.parametrize("case,box", [("mlp", False), ("mlp", True), ("cnn", False)])
def test_crown_backward_linear_bounds(lbp, case, box):
    """A_out / bias_out: the linear bounds over the domain node equal the oracle's
    Lambda there, and the oracle's bound is their concretisation."""
    wl = CASES[case]()
    on, lo, hi = _fp32_bounds(wl)
    net, x, C = lbp.prepare(wl)
    dlo, dhi = _to_device(lbp, net, wl, lo, hi)
    L = len(wl.nodes) - 1
    stop = [k for k, nd in enumerate(wl.nodes) if nd.op == "relu"][0] if box else 0
    method = "hybrid" if box else "crown"
    ws = net.workspace(net.workspace_size(wl.batch, wl.m, method, stop))
    lb, ub, A, bias = lbp.crown_backward(net, L, stop, dlo, dhi, x, float(wl.eps), ws, C=C, linear=True)
    torch.cuda.synchronize()
    shape = wl.nodes[stop].shape
    m = wl.m
    for b in range(wl.batch):
        if stop == 0:
            c = _f64(wl.x0[b])
            r = torch.full_like(c, float(np.float32(wl.eps)))
        else:
            c, r = (lo[stop][b] + hi[stop][b]) / 2, (hi[stop][b] - lo[stop][b]) / 2
        for sgn, sl in ((1.0, slice(0, m)), (-1.0, slice(m, 2 * m))):
            keep = {}
            val = backward(on, lo, hi, b, L, sgn * _f64(wl.C[b]), stop, c, r, keep=keep)
            Lam = keep["domain"]
            beta = val - concretize(Lam, torch.zeros(m, dtype=torch.float64), c, r)
            assert_close(A[b, sl], nhwc(Lam, shape), f"A input {b} sign {sgn}")
            assert_close(bias[b, sl], beta, f"bias input {b} sign {sgn}")
        assert_close(lb[b], _oracle_rows(on, lo, hi, wl, b, L, _f64(wl.C[b]), stop), f"lb input {b}")


@pytest.mark.parametrize("case", ["mlp", "cnn"])
def test_crown_backward_with_alpha_one_sided(lbp, case):
    """Spec rows with given lower slopes (ub NULL: only the rows C are pushed) against
    the oracle's back-substitution with the same slopes; without alpha the one-sided
    call gives the two-sided call's lb."""
    wl = CASES[case]()
    on, lo, hi = _fp32_bounds(wl)
    net, x, C = lbp.prepare(wl)
    dlo, dhi = _to_device(lbp, net, wl, lo, hi)
    L = len(wl.nodes) - 1
    ws = net.workspace(net.workspace_size(wl.batch, wl.m, "crown"))
    lb2, _ = lbp.crown_backward(net, L, 0, dlo, dhi, x, float(wl.eps), ws, C=C)
    lb1, ub1 = lbp.crown_backward(net, L, 0, dlo, dhi, x, float(wl.eps), ws, C=C, lower_only=True)
    torch.cuda.synchronize()
    assert ub1 is None
    assert_close(lb1, lb2.detach().double().cpu().numpy(), "one-sided lb")
    rng = np.random.default_rng(9)
    alpha_dev = [None] * len(wl.nodes)
    alpha_ref = {}
    for r, nd in enumerate(wl.nodes):
        if nd.op != "relu":
            continue
        a = rng.random((wl.batch, wl.m) + tuple(nd.shape)).astype(np.float32)
        alpha_ref[r] = a
        alpha_dev[r] = torch.as_tensor(nhwc(a.reshape((wl.batch * wl.m,) + tuple(nd.shape)), nd.shape)
                                       .reshape(wl.batch, wl.m, -1), dtype=torch.float32, device=x.device)
    lba, uba, A, bias = lbp.crown_backward(net, L, 0, dlo, dhi, x, float(wl.eps), ws, C=C, alpha=alpha_dev,
                                           linear=True)
    torch.cuda.synchronize()
    assert uba is None and A.shape[1] == wl.m
    for b in range(wl.batch):
        c = _f64(wl.x0[b])
        r = torch.full_like(c, float(np.float32(wl.eps)))
        keep = {}
        ref = backward(on, lo, hi, b, L, _f64(wl.C[b]), 0, c, r,
                       alpha={k: _f64(v[b]) for k, v in alpha_ref.items()}, keep=keep)
        assert_close(lba[b], ref, f"alpha lb input {b}")
        assert_close(A[b], nhwc(keep["domain"], wl.nodes[0].shape), f"alpha A input {b}")


# ---------------------------------------------------------------------------
# compact alpha (vb_alpha_layout and the compact layout in the alpha calls)

def _host_columns(wl, lo, hi):
    """Oracle compact columns of every ReLU node from the fp32 bounds in the library's layout."""
    cols = {}
    for r, nd in enumerate(wl.nodes):
        if nd.op == "relu":
            z = nd.inputs[0]
            cols[r] = compact_columns(nhwc(lo[z], wl.nodes[z].shape), nhwc(hi[z], wl.nodes[z].shape))
    return cols


@pytest.mark.parametrize("case", ["mlp", "cnn"])
def test_alpha_layout_matches_oracle(lbp, case):
    wl = CASES[case]()
    on, lo, hi = _fp32_bounds(wl)
    net, x, C = lbp.prepare(wl)
    dlo, dhi = _to_device(lbp, net, wl, lo, hi)
    lay = lbp.alpha_layout(net, dlo, dhi)
    ref = _host_columns(wl, lo, hi)
    for k, nd in enumerate(wl.nodes):
        if nd.op != "relu":
            assert lay.width[k] == 0 and lay.index[k] is None
            continue
        col, width = ref[k]
        assert lay.width[k] == width, (k, lay.width[k], width)
        assert np.array_equal(lay.index[k].cpu().numpy(), col), k
    assert any(w > 0 for w in lay.width)


def _compact_from_dense(dense, col, width):
    """[B][m][n] (library layout) -> [B][m][width]: the unstable neurons' columns."""
    B, m, n = dense.shape
    out = np.zeros((B, m, width), np.float32)
    for b in range(B):
        j = np.nonzero(col[b] >= 0)[0]
        out[b][:, col[b, j]] = dense[b][:, j]
    return out


@pytest.mark.parametrize("case", ["mlp", "cnn"])
def test_crown_backward_with_compact_alpha(lbp, case):
    """Given slopes in the compact layout give the oracle's bound with the same slopes
    (the oracle holds them densely; entries of stable neurons do not enter)."""
    wl = CASES[case]()
    on, lo, hi = _fp32_bounds(wl)
    net, x, C = lbp.prepare(wl)
    dlo, dhi = _to_device(lbp, net, wl, lo, hi)
    L = len(wl.nodes) - 1
    ws = net.workspace(net.workspace_size(wl.batch, wl.m, "crown"))
    lay = lbp.alpha_layout(net, dlo, dhi)
    cols = _host_columns(wl, lo, hi)
    rng = np.random.default_rng(11)
    alpha_dev = [None] * len(wl.nodes)
    alpha_ref = {}
    for r, nd in enumerate(wl.nodes):
        if nd.op != "relu":
            continue
        a = rng.random((wl.batch, wl.m) + tuple(nd.shape)).astype(np.float32)
        alpha_ref[r] = a
        dense = nhwc(a.reshape((wl.batch * wl.m,) + tuple(nd.shape)), nd.shape).reshape(wl.batch, wl.m, -1)
        col, width = cols[r]
        if width > 0:
            alpha_dev[r] = torch.as_tensor(_compact_from_dense(dense, col, width), device=x.device)
    lba, _ = lbp.crown_backward(net, L, 0, dlo, dhi, x, float(wl.eps), ws, C=C, alpha=alpha_dev, layout=lay)
    torch.cuda.synchronize()
    for b in range(wl.batch):
        c = _f64(wl.x0[b])
        r = torch.full_like(c, float(np.float32(wl.eps)))
        ref = backward(on, lo, hi, b, L, _f64(wl.C[b]), 0, c, r, alpha={k: _f64(v[b]) for k, v in alpha_ref.items()})
        assert_close(lba[b], ref, f"compact alpha lb input {b}")


@pytest.mark.parametrize("compact", [False, True])
@pytest.mark.parametrize("case", ["mlp", "cnn"])
def test_crown_backward_alpha_chunked_batch(lbp, case, compact):
    """Given slopes with a workspace for one batch element at a time: the chunks
    address the slopes (and the compact column maps) at their own offsets, so the
    bounds equal the whole-batch call bit for bit."""
    wl = CASES[case]()
    on, lo, hi = _fp32_bounds(wl)
    net, x, C = lbp.prepare(wl)
    dlo, dhi = _to_device(lbp, net, wl, lo, hi)
    L = len(wl.nodes) - 1
    lay = lbp.alpha_layout(net, dlo, dhi) if compact else None
    cols = _host_columns(wl, lo, hi)
    rng = np.random.default_rng(17)
    alpha_dev = [None] * len(wl.nodes)
    for r, nd in enumerate(wl.nodes):
        if nd.op != "relu":
            continue
        a = rng.random((wl.batch * wl.m,) + tuple(nd.shape)).astype(np.float32)
        dense = nhwc(a, nd.shape).reshape(wl.batch, wl.m, -1)
        if compact:
            col, width = cols[r]
            if width > 0:
                alpha_dev[r] = torch.as_tensor(_compact_from_dense(dense, col, width), device=x.device)
        else:
            alpha_dev[r] = torch.as_tensor(dense, device=x.device)
    ws_full = net.workspace(net.workspace_size(wl.batch, wl.m, "crown"))
    full, _ = lbp.crown_backward(net, L, 0, dlo, dhi, x, float(wl.eps), ws_full, C=C, alpha=alpha_dev, layout=lay)
    ws_one = net.workspace(net.workspace_size(1, wl.m, "crown"))
    part, _ = lbp.crown_backward(net, L, 0, dlo, dhi, x, float(wl.eps), ws_one, C=C, alpha=alpha_dev, layout=lay)
    torch.cuda.synchronize()
    assert ws_one.numel() < ws_full.numel()
    assert torch.equal(full, part)


def test_alpha_init_compact(lbp):
    wl = CASES["cnn"]()
    on, lo, hi = _fp32_bounds(wl)
    net, x, C = lbp.prepare(wl)
    dlo, dhi = _to_device(lbp, net, wl, lo, hi)
    lay = lbp.alpha_layout(net, dlo, dhi)
    alpha, am, av = lbp.alpha_state(net, wl.batch, wl.m, lay)
    for t in am + av:
        if t is not None:
            t.fill_(7.0)
    lbp.alpha_init(net, dlo, dhi, alpha, am, av, wl.m, layout=lay)
    torch.cuda.synchronize()
    cols = _host_columns(wl, lo, hi)
    for b in range(wl.batch):
        ref = oracle_alpha_init(on, lo, hi, b, wl.m)
        for r, a in ref.items():
            col, width = cols[r]
            if width == 0:
                assert alpha[r] is None
                continue
            dense = nhwc(a, wl.nodes[r].shape)          # [m][n]
            j = np.nonzero(col[b] >= 0)[0]
            got = alpha[r][b].cpu().numpy()[:, col[b, j]]
            assert np.array_equal(got, dense[:, j].astype(np.float32)), (r, b)
            assert float(np.abs(am[r][b].cpu().numpy()[:, col[b, j]]).max(initial=0)) == 0.0
            assert float(np.abs(av[r][b].cpu().numpy()[:, col[b, j]]).max(initial=0)) == 0.0


# ---------------------------------------------------------------------------
# vb_alpha_init

def test_alpha_init_is_the_adaptive_slope(lbp):
    wl = CASES["cnn"]()
    on, lo, hi = _fp32_bounds(wl)
    net, x, C = lbp.prepare(wl)
    dlo, dhi = _to_device(lbp, net, wl, lo, hi)
    alpha, am, av = lbp.alpha_state(net, wl.batch, wl.m)
    lbp.alpha_init(net, dlo, dhi, alpha, am, av, wl.m)
    torch.cuda.synchronize()
    for b in range(wl.batch):
        ref = oracle_alpha_init(on, lo, hi, b, wl.m)
        for r, a in ref.items():
            shape = wl.nodes[r].shape
            assert_close(alpha[r][b], nhwc(a, shape), f"alpha[{r}] input {b}", atol=0, rtol=0)
            assert float(am[r][b].abs().max()) == 0.0 and float(av[r][b].abs().max()) == 0.0


# ---------------------------------------------------------------------------
# degenerate cases of the whole pipeline

def _run(lbp, wl, method=None):
    net, x, C = lbp.prepare(wl)
    out = lbp.crown(net, x, float(wl.eps), C, method or wl.intermediate, wl.region_start)
    torch.cuda.synchronize()
    return out


def test_zero_radius_gives_the_network_output(lbp):
    """eps = 0: every bound is C f(x0) (lb = ub)."""
    wl = wk.tiny_mlp([20, 33, 17, 6], 0.0, 31, batch=2)
    out = _run(lbp, wl)
    ref = crown_bounds(wl)
    compare_workload(wl, out, ref)
    assert_close(out["lb"], out["ub"].detach().double().cpu().numpy(), "lb = ub")


def test_single_input_single_spec(lbp):
    """batch 1 and a two-class output (one margin spec)."""
    wl = wk.tiny_mlp([12, 19, 2], 0.1, 32, batch=1)
    assert wl.m == 1
    out = _run(lbp, wl)
    compare_workload(wl, out, crown_bounds(wl))


def test_all_inactive_layer(lbp):
    """A hidden layer whose ReLUs are all off: the bounds collapse to the path
    through the biases after it."""
    wl = wk.tiny_mlp([16, 24, 20, 5], 0.05, 33, batch=2)
    k = [i for i, nd in enumerate(wl.nodes) if nd.op == "linear"][1]
    wl.nodes[k].weight = np.zeros_like(wl.nodes[k].weight)
    wl.nodes[k].bias = np.full_like(wl.nodes[k].bias, -1.0)
    out = _run(lbp, wl)
    ref = crown_bounds(wl)
    compare_workload(wl, out, ref)
    assert_close(out["lb"], out["ub"].detach().double().cpu().numpy(), "lb = ub")


# ---------------------------------------------------------------------------
# vb_verify

def test_verify_matches_the_bounds_and_the_oracle(lbp):
    """The per-input verdict: 1 iff every spec lower bound is positive; on the
    784-100-100-10 workload some inputs are proved and some are not, and the
    verdict agrees with the oracle's bounds wherever those are not within the
    parity tolerance of zero.  NaN and zero bounds do not verify."""
    from helpers import ATOL, RTOL
    wl = wk.config(1)
    net, x, C = lbp.prepare(wl)
    out = lbp.crown(net, x, float(wl.eps), C, "crown")
    flags, count = lbp.verify(out["lb"])
    torch.cuda.synchronize()
    lb = out["lb"].cpu()
    want = (lb > 0).all(dim=1).to(torch.int32)
    assert torch.equal(flags.cpu(), want)
    assert int(count.item()) == int(want.sum())
    assert 0 < int(count.item()) < wl.batch
    ref = crown_bounds(wl)["lb"]
    clear = (ref.abs() > ATOL + RTOL * ref.abs()).all(dim=1)
    assert bool(clear.any())
    assert torch.equal(flags.cpu()[clear].bool(), (ref[clear] > 0).all(dim=1))
    odd = torch.tensor([[1.0, 2.0], [1.0, 0.0], [float("nan"), 1.0], [3.0, -1e-30]], device=x.device)
    f2, c2 = lbp.verify(odd)
    torch.cuda.synchronize()
    assert f2.cpu().tolist() == [1, 0, 0, 0] and int(c2.item()) == 1
