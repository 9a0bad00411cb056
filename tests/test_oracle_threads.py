"""The oracle's data moves give the same bits on one thread and on many (CPU only).

The moves spread their outer loop over OpenMP threads so that the CPU baseline
uses the host's cores. Every output element has one writer (a slot holds one
entry; a token row, an expert element and a grad_w entry belong to one loop
iteration) and keeps its own order of operations, so the result may not depend
on the thread count. Each move runs on one thread and on eight, and the outputs
are compared byte for byte, on a skewed plan with dropped entries and
duplicates beyond B.
"""
import numpy as np
import pytest

import oracle
import workloads as W

THREADS = 8


@pytest.fixture(scope="module")
def case():
    R, E, K, S, B, H = 8, 64, 4, 700, 2, 72
    wl = W.Workload("threads", R=R, E=E, K=K, S=S, H=H, dtype=W.BF16, B=B, block_shape=(40,),
                    block_dtype=W.F32, routing="bias", bias_std=2.5)
    ids, w = W.make_routing(wl, seed=4)
    ids = ids.reshape(-1).copy()
    rng = np.random.default_rng(4)
    ids[rng.choice(ids.size, 30, replace=False)] = -1
    p = oracle.plan(R, E, K, S, B, ids)
    assert int(p["n_dup"].max()) > B  # some duplicates have no slot
    hid = rng.integers(0, 1 << 16, size=(R * S, H), dtype=np.uint16)
    y = rng.standard_normal((R * S * K, H)).astype(np.float32)
    yb = (y.view(np.uint32) >> 16).astype(np.uint16)
    ew = rng.standard_normal((E, 40)).astype(np.float32)
    dg = rng.standard_normal((R, B, 40)).astype(np.float32)
    hg = rng.standard_normal((E, 40)).astype(np.float32)
    gout = rng.standard_normal((R * S, H)).astype(np.float32)
    return dict(R=R, E=E, K=K, S=S, B=B, H=H, p=p, w=w.reshape(-1), hid=hid, y=y, yb=yb,
                ew=ew, dg=dg, hg=hg, gout=gout)


def _moves(c):
    p, K = c["p"], c["K"]
    dst = p["dst"]
    y_rows = c["yb"][np.maximum(dst, 0)]
    return {
        "dispatch": oracle.dispatch(p, K, c["hid"]),
        "dispatch_window": oracle.dispatch(p, K, c["hid"], 1000, 5000),
        "replicate": oracle.replicate(p, c["B"], c["ew"]),
        "combine_bf16": oracle.combine(dst, K, c["yb"], c["w"], oracle.BF16, oracle.BF16),
        "combine_f32": oracle.combine(dst, K, c["y"], c["w"], oracle.F32, oracle.F32),
        "reduce": oracle.reduce_dup_grads(p, c["B"], c["dg"], c["hg"]),
        "combine_backward_y": oracle.combine_backward_y(dst, K, c["gout"], c["w"], oracle.F32,
                                                        oracle.BF16),
        "combine_backward_w": oracle.combine_backward_w(dst, K, c["gout"], y_rows, oracle.F32,
                                                        oracle.BF16),
        "dispatch_backward": oracle.dispatch_backward(dst, K, c["yb"], oracle.BF16, oracle.F32),
    }


def test_moves_do_not_depend_on_thread_count(case):
    before = oracle.max_threads()
    try:
        oracle.set_threads(1)
        assert oracle.max_threads() == 1
        one = _moves(case)
        oracle.set_threads(THREADS)
        assert oracle.max_threads() == THREADS
        many = _moves(case)
    finally:
        oracle.set_threads(before)
    for k in one:
        assert one[k].dtype == many[k].dtype and one[k].shape == many[k].shape, k
        assert np.array_equal(one[k].view(np.uint8), many[k].view(np.uint8)), k


def test_dispatch_into_a_given_buffer(case):
    """out= writes the filled slots and leaves the others as they were."""
    p, K = case["p"], case["K"]
    want = oracle.dispatch(p, K, case["hid"])
    buf = np.full_like(want, 0xBEEF)
    got = oracle.dispatch(p, K, case["hid"], out=buf)
    assert got is buf
    filled = p["src"] >= 0
    assert not filled.all()
    assert np.array_equal(got[filled], want[filled])
    assert np.all(got[~filled] == 0xBEEF)
    with pytest.raises(ValueError):
        oracle.dispatch(p, K, case["hid"], out=np.zeros((3, case["H"]), np.uint16))
