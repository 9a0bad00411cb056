"""The plan entry point for callers that cannot allocate (moonep_plan_noscratch)
against the entry points it is a variant of (moonep_plan, moonep_plan_bounded),
through the C ABI.

The variant keeps the plan kernels' scratch in the library's static device array
and writes only the first persist_bytes of the caller's plan buffer. Its plan
must equal the regular call's bit for bit, call after call on the same GPU (the
static array keeps whatever the previous call left), the later calls smaller
than the first. The plan buffer handed to it is followed by a guard region that
must stay untouched, and the moves read its plan as they read a full one.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_common import assert_plan_equal, read_plan, say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
GUARD = 0x5A


@pytest.fixture(scope="module")
def td():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import token_dispatch_amd as td
    torch.cuda.set_device(DEV)
    return td


def _dims(td, wl):
    return td.Dims(wl.R, wl.E, wl.K, wl.S, wl.B, wl.dtype, wl.H)


def _persist_ws(td, dims, buf):
    """The workspace that later calls read: mat_pre (replicate), xlist and n_x (reduce)."""
    lay = td.moonep_plan_layout(dims)

    def arr(off, n):
        return buf[off:off + 4 * n].view(torch.int32).cpu().numpy()

    n_x = int(arr(lay.ws_n_x, 1)[0])
    return arr(lay.ws_mat_pre, dims.R + 1), n_x, arr(lay.ws_xlist, dims.E)[:n_x]


def _moves_agree(td, dims, wl, pb_full, pb_small):
    """dispatch, replicate and reduce driven by either plan buffer give the same bytes
    (small 4 KiB weight blocks and 1024-element gradient blocks)."""
    hid = W.make_hidden(wl, 0, DEV)
    outs = []
    blk_elems = 1024
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)
    ew = torch.randn((wl.E, blk_elems), generator=gen, device=DEV)
    dg = torch.randn((wl.R, wl.B, blk_elems), generator=gen, device=DEV)
    hg0 = torch.randn((wl.E, blk_elems), generator=gen, device=DEV)
    for pb in (pb_full, pb_small):
        recv = torch.zeros((wl.R, wl.SK, wl.H), dtype=hid.dtype, device=DEV)
        td.moonep_dispatch(dims, pb, hid, recv)
        dup_w = torch.zeros((wl.R, wl.B, blk_elems), device=DEV)
        td.moonep_replicate(dims, pb, ew, dup_w, 4 * blk_elems)
        hg = hg0.clone()
        td.moonep_reduce_dup_grads(dims, pb, dg, hg, blk_elems)
        torch.cuda.synchronize()
        outs.append((recv, dup_w, hg))
    (r0, w0, h0), (r1, w1, h1) = outs
    assert torch.equal(r0.view(torch.int16) if r0.dtype == torch.bfloat16 else r0.view(torch.int32),
                       r1.view(torch.int16) if r1.dtype == torch.bfloat16 else r1.view(torch.int32))
    assert torch.equal(w0.view(torch.int32), w1.view(torch.int32))
    assert torch.equal(h0.view(torch.int32), h1.view(torch.int32))


@pytest.mark.parametrize("bounded", [False, True], ids=["waterfill", "bounded"])
def test_noscratch_plan_equals_plan_calls_in_a_row(td, bounded):
    # the first call the largest, each later one smaller, all on the same static array
    for name, seed in (("k3", 1), ("decode", 2), ("tiny", 0)):
        wl = W.WORKLOADS[name]
        dims = _dims(td, wl)
        lay = td.moonep_plan_layout(dims)
        say(f"noscratch {name} bounded={bounded}: {dims}; persist {lay.persist_bytes} of "
            f"{lay.bytes} bytes, scratch {lay.bytes - lay.persist_bytes}")
        assert lay.bytes - lay.persist_bytes <= td.STATIC_SCRATCH_BYTES
        ids, _ = W.make_routing(wl, seed)
        ids_d = torch.from_numpy(ids).to(DEV)
        full = torch.full((lay.bytes,), 0xA5, dtype=torch.uint8, device=DEV)
        # the variant's buffer is the first persist_bytes of an allocation whose rest
        # is a guard: no byte of it may change
        span = torch.full((lay.bytes,), GUARD, dtype=torch.uint8, device=DEV)
        small = span[:lay.persist_bytes]
        small.fill_(0xA5)
        guard = span[lay.persist_bytes:]
        (td.moonep_plan_bounded if bounded else td.moonep_plan)(dims, ids_d, full)
        td.moonep_plan_noscratch(dims, ids_d, small, bounded)
        torch.cuda.synchronize()
        assert bool((guard == GUARD).all()), "a write landed past persist_bytes"
        g_full = read_plan(td, dims, full)
        g_small = read_plan(td, dims, small)
        assert_plan_equal(g_small, g_full)
        m0, n0, x0 = _persist_ws(td, dims, full)
        m1, n1, x1 = _persist_ws(td, dims, small)
        assert np.array_equal(m0, m1) and n0 == n1 and np.array_equal(x0, x1)
        # every rank holds exactly S*K rows in both
        assert np.all(g_small["seg_ptr"][np.arange(wl.R), wl.G + g_small["n_dup"]] == wl.SK)
        if name != "k3":
            _moves_agree(td, dims, wl, full, small)
        say(f"  equal (dups per rank max {int(g_small['n_dup'].max())}, "
            f"status {int(g_small['status'][0])})")
        del full, span, small, guard


def test_noscratch_random_shapes_in_a_row(td):
    """Seeded random shapes one after another through the same static array, both
    plans alternating: each plan equals the regular call's."""
    from tests.test_gpu_parity import RANDOM
    for i, wl in enumerate(RANDOM[:24]):
        bounded = bool(i & 1)
        dims = _dims(td, wl)
        lay = td.moonep_plan_layout(dims)
        assert lay.bytes - lay.persist_bytes <= td.STATIC_SCRATCH_BYTES
        say(f"noscratch {wl.name} bounded={bounded}: {dims}")
        ids, _ = W.make_routing(wl, 100 + i)
        ids_d = torch.from_numpy(ids).to(DEV)
        full = torch.full((lay.bytes,), 0xA5, dtype=torch.uint8, device=DEV)
        small = torch.full((lay.persist_bytes,), 0xA5, dtype=torch.uint8, device=DEV)
        (td.moonep_plan_bounded if bounded else td.moonep_plan)(dims, ids_d, full)
        td.moonep_plan_noscratch(dims, ids_d, small, bounded)
        torch.cuda.synchronize()
        assert_plan_equal(read_plan(td, dims, small), read_plan(td, dims, full))
        m0, n0, x0 = _persist_ws(td, dims, full)
        m1, n1, x1 = _persist_ws(td, dims, small)
        assert np.array_equal(m0, m1) and n0 == n1 and np.array_equal(x0, x1)
