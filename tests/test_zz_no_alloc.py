"""vb_crown_noalloc (the library's fixed device scratch instead of a workspace)
against vb_crown (caller workspace) through the C ABI: two calls in a row, the
second with a smaller input, each compared with vb_crown on the same input.
Where both run the whole batch in one chunk the bounds are bitwise equal; a
batch the fixed scratch must chunk is compared at the parity tolerance."""
import numpy as np
import pytest
import torch

import workloads as wk
from helpers import assert_close, ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lbp():
    ensure_built()
    import linear_bound_propagation_amd as m
    return m


def _both(lbp, wl):
    net, x, C = lbp.prepare(wl)
    ref = lbp.crown(net, x, float(wl.eps), C, wl.intermediate, wl.region_start)
    got = lbp.crown_noalloc(net, x, float(wl.eps), C, wl.intermediate, wl.region_start)
    torch.cuda.synchronize()
    return net, ref, got


KEYS = ("lb", "ub", "ibp_lb", "ibp_ub")


@pytest.mark.parametrize("make", [
    lambda b: wk.config(1, batch=b),
    lambda b: wk.cnn(b, 0.01, 71, convs=((8, 1), (16, 2)), fcs=(20, 10), in_shape=(3, 9, 9), intermediate="crown"),
    lambda b: wk.resnet(b, 0.01, 72, widths=(4, 6), blocks=(1, 1), n_out=5, in_shape=(3, 8, 8)),
], ids=["mlp", "cnn", "resnet"])
def test_noalloc_equals_workspace_call_twice_shrinking(lbp, make):
    for batch in (6, 2):                # second call: smaller input on the same scratch
        wl = make(batch)
        print(f"noalloc {wl.name} batch {batch} ({wl.intermediate})", flush=True)
        net, ref, got = _both(lbp, wl)
        for k in KEYS:
            assert torch.equal(got[k], ref[k]), k
        for k in range(1, len(wl.nodes)):
            assert torch.equal(got["lo"][k], ref["lo"][k]), k
            assert torch.equal(got["hi"][k], ref["hi"][k]), k


def test_noalloc_chunks_a_batch_larger_than_the_scratch(lbp):
    """The 3072-wide MLP at 8 inputs needs more than the fixed scratch for the whole
    batch: the call runs in chunks and matches the workspace call; then a smaller call."""
    for batch in (8, 3):
        wl = wk.config(2, batch=batch)
        print(f"noalloc {wl.name} batch {batch}", flush=True)
        net, ref, got = _both(lbp, wl)
        for k in KEYS:
            assert_close(got[k], ref[k].double(), k)


def test_noalloc_rejects_a_graph_beyond_the_scratch(lbp):
    wl = wk.config(5, batch=1)
    net, x, C = lbp.prepare(wl)
    with pytest.raises(lbp.VBError) as e:
        lbp.crown_noalloc(net, x, float(wl.eps), C, wl.intermediate, wl.region_start)
    assert e.value.status == -3 and "fixed scratch" in str(e.value)
