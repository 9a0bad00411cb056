"""GPU parity of the backward moves: the HIP path (through the C ABI) against the
CPU oracle.

- grad_y of combine and the backward of dispatch are compared bit for bit (both
  sides perform the same binary32 operations in the same order and round the
  same way).
- grad_w of combine is a binary32 dot product over H; it is held against the
  oracle's binary64 value within gamma_H * sum_i |grad_out_i * y_i|, the bound of
  any binary32 summation order (gamma_n = n u / (1 - n u), u = 2^-24).

Small shapes are compared element by element; the workloads run at full size in
the launch configuration the benchmark uses, seeds 0, 1 and 2, every slot of
grad_y and every token of grad_w and grad_hidden through the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_common import (HostStage, bf16_bits, local_dst, read_plan, run_plan, say,
                              token_batches)
from tests.test_gpu_parity import RANDOM_ROWS, SMALL, _dims, _host_rows, _wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
U32 = 2.0 ** -24


@pytest.fixture(scope="module")
def td():
    if not torch.cuda.is_available():
        pytest.fail("GPU parity tests need a GPU")
    import token_dispatch_amd as td
    torch.cuda.set_device(DEV)
    return td


def _as_f32(rows, dt):
    if dt == W.BF16:
        return (rows.astype(np.uint32) << 16).view(np.float32)
    return rows


def _gamma(n):
    return n * U32 / (1 - n * U32)


def _check_grad_w(got, want64, gout_h, y_rows_h, g_dt, y_dt, K, H, what):
    mag = (np.abs(_as_f32(gout_h, g_dt).astype(np.float64)).repeat(K, axis=0) *
           np.abs(_as_f32(y_rows_h, y_dt).astype(np.float64))).sum(1)
    err = np.abs(got.astype(np.float64) - want64)
    bad = np.nonzero(err > _gamma(H) * mag)[0]
    assert bad.size == 0, f"{what}: grad_w off at {bad[:8].tolist()}: {got[bad[:8]]} vs {want64[bad[:8]]}"


def _small_case(td, wl, ids, w, seed):
    dims = _dims(td, wl)
    say(f"backward case {wl.name}: {dims}")
    plan_buf, _ = run_plan(td, dims, ids, DEV)
    p = oracle.plan(wl.R, wl.E, wl.K, wl.S, wl.B, ids)
    g = read_plan(td, dims, plan_buf)
    assert np.array_equal(g["dst"], p["dst"])
    filled = p["src"] >= 0
    y = W.make_expert_out(wl, seed)
    y_d = y.to(DEV)
    y_h = _host_rows(y).reshape(-1, wl.H)
    w_d = torch.from_numpy(w).to(DEV)
    y_rows_h = y_h[np.maximum(p["dst"], 0)]
    for g_dt in (W.F32, W.BF16):
        gout = W.dense((wl.R, wl.S, wl.H), g_dt, 1.0, seed + 7, "hidden", "cpu")
        gout_d = gout.to(DEV)
        gout_h = _host_rows(gout).reshape(wl.n_tok, wl.H)
        grad_y = torch.full((wl.R, wl.SK, wl.H), 3.0, dtype=y.dtype, device=DEV)
        grad_w = torch.full((wl.R, wl.S, wl.K), 5.0, dtype=torch.float32, device=DEV)
        if wl.H * (2 if g_dt == W.BF16 else 4) % 16:
            # grad_out rows must be whole 16-byte chunks: rejected, nothing written
            with pytest.raises(td.MoonEPError) as err:
                td.moonep_combine_backward(dims, plan_buf, gout_d, w_d, y_d, grad_y, grad_w)
            assert err.value.rc == td.ERR_DIMS
            torch.cuda.synchronize()
            assert bool((grad_w == 5.0).all()) and bool((grad_y == 3.0).all())
            continue
        td.moonep_combine_backward(dims, plan_buf, gout_d, w_d, y_d, grad_y, grad_w)
        torch.cuda.synchronize()
        want_y = oracle.combine_backward_y(p["dst"], wl.K, gout_h, w, g_dt, wl.dtype)
        got_y = _host_rows(grad_y).reshape(-1, wl.H)
        assert np.array_equal(got_y[filled].view(np.uint8), want_y[filled].view(np.uint8)), \
            f"grad_y gout_dtype={g_dt}"
        sentinel = _host_rows(torch.full((1, wl.H), 3.0, dtype=y.dtype)).reshape(-1)
        assert np.all(got_y[~filled] == sentinel), "a slot without an entry was written"
        want_w = oracle.combine_backward_w(p["dst"], wl.K, gout_h, y_rows_h, g_dt, wl.dtype)
        got_w = grad_w.cpu().numpy().reshape(-1)
        _check_grad_w(got_w, want_w, gout_h, y_rows_h, g_dt, wl.dtype, wl.K, wl.H,
                      f"{wl.name} gout_dtype={g_dt}")
        assert np.all(got_w[p["dst"] < 0] == 0.0)
        # each output alone gives the same values
        gy2 = torch.zeros_like(grad_y)
        td.moonep_combine_backward(dims, plan_buf, gout_d, w_d, None, gy2, None)
        gw2 = torch.zeros_like(grad_w)
        td.moonep_combine_backward(dims, plan_buf, gout_d, None, y_d, None, gw2)
        torch.cuda.synchronize()
        fm = torch.from_numpy(filled).to(DEV)
        assert torch.equal(gy2.reshape(-1, wl.H).view(torch.int8)[fm],
                           grad_y.reshape(-1, wl.H).view(torch.int8)[fm])
        assert torch.equal(gw2, grad_w)
    # backward of dispatch
    grec = W.make_expert_out(wl, seed + 1)
    grec_h = _host_rows(grec).reshape(-1, wl.H)
    for od in (W.F32, W.BF16):
        gh = torch.empty((wl.R, wl.S, wl.H), dtype=W.torch_dtype(od), device=DEV)
        td.moonep_dispatch_backward(dims, plan_buf, grec.to(DEV), gh, od)
        torch.cuda.synchronize()
        want = oracle.dispatch_backward(p["dst"], wl.K, grec_h, wl.dtype, od)
        got = _host_rows(gh).reshape(-1, wl.H)
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), f"dispatch backward od={od}"


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_backward_small_shapes_elementwise(td, wl):
    ids, w = W.make_routing(wl, seed=8)
    _small_case(td, wl, ids.reshape(-1), w.reshape(-1), 8)


@pytest.mark.parametrize("wl", RANDOM_ROWS, ids=[w.name for w in RANDOM_ROWS])
def test_backward_random_row_widths(td, wl):
    """The backward moves at seeded random row widths and K."""
    ids, w = W.make_routing(wl, 300 + int(wl.name[4:]))
    _small_case(td, wl, ids.reshape(-1), w.reshape(-1), 9)


def test_backward_with_dropped_entries(td):
    wl = _wl("bwd_bad_ids", 4, 32, 4, 1500, 4, 64, W.BF16, 2.0)
    rng = np.random.default_rng(23)
    ids, w = W.make_routing(wl, seed=9)
    ids = ids.reshape(-1).copy()
    ids[rng.choice(ids.size, 50, replace=False)] = -1
    _small_case(td, wl, ids, w.reshape(-1), 9)


def test_dispatch_backward_of_dispatch_is_k_times_hidden(td):
    """Each token's K slots hold copies of its bf16 row; with K a power of two the
    binary32 sum K * x is exact and a bf16 value."""
    wl = _wl("bwd_identity", 8, 64, 8, 900, 8, 512, W.BF16, 2.0)
    dims = _dims(td, wl)
    ids, _ = W.make_routing(wl, seed=2)
    plan_buf, _ = run_plan(td, dims, ids, DEV)
    hid = W.make_hidden(wl, 2).to(DEV)
    recv = torch.empty((wl.R, wl.SK, wl.H), dtype=hid.dtype, device=DEV)
    back = torch.empty_like(hid)
    td.moonep_dispatch(dims, plan_buf, hid, recv)
    td.moonep_dispatch_backward(dims, plan_buf, recv, back)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16), (hid.float() * wl.K).to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("name", ["uniform", "zipf", "k3", "decode"])
def test_backward_full_size(td, name, seed):
    """Every output element of both backward moves at full size, in the launch
    configuration the benchmark uses, against the oracle: grad_y slot by slot in
    destination-rank windows, grad_w and the backward of dispatch token by token
    in batches of gathered rows. grad_w is held to the binary32 summation bound
    around the oracle's binary64 value; the bound's magnitude sum_i |grad_out_i *
    y_i| is taken on the GPU in binary64."""
    wl = W.WORKLOADS[name]
    dims = _dims(td, wl)
    say(f"full-size backward {name} seed={seed}: {dims}")
    ids, w = W.make_routing(wl, seed)
    p = oracle.plan(wl.R, wl.E, wl.K, wl.S, wl.B, ids)
    pb, _ = run_plan(td, dims, ids, DEV)
    assert np.array_equal(read_plan(td, dims, pb)["dst"], p["dst"])
    w_d = torch.from_numpy(w).to(DEV)
    gout = W.dense((wl.R, wl.S, wl.H), W.BF16, 1.0, seed + 7, "hidden", DEV)
    y = torch.empty((wl.R, wl.SK, wl.H), dtype=torch.bfloat16, device=DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(4321 + seed)
    for r in range(wl.R):
        y[r].copy_(torch.randn((wl.SK, wl.H), generator=gen, device=DEV, dtype=torch.float32))
    grad_y = torch.empty_like(y)
    grad_w = torch.empty((wl.R, wl.S, wl.K), dtype=torch.float32, device=DEV)
    say("  combine backward")
    td.moonep_combine_backward(dims, pb, gout, w_d, y, grad_y, grad_w)
    torch.cuda.synchronize()
    gout_h = bf16_bits(gout).reshape(wl.n_tok, wl.H)
    # grad_y: every slot that holds an entry, one destination rank at a time
    stage = HostStage(wl.SK * wl.row_bytes)
    gyflat = grad_y.view(-1, wl.H)
    for r in range(wl.R):
        lo, hi = r * wl.SK, (r + 1) * wl.SK
        want = oracle.combine_backward_y(p["dst"], wl.K, gout_h, w, W.BF16, W.BF16, lo, hi)
        got = stage.fetch(gyflat[lo:hi])
        filled = p["src"][lo:hi] >= 0
        if not np.array_equal(got[filled], want[filled]):
            bad = np.nonzero((got != want).any(axis=1) & filled)[0]
            raise AssertionError(f"grad_y differs at slots {(lo + bad[:8]).tolist()}")
    say(f"  grad_y: all {wl.n_ent} slots equal")
    del grad_y, stage
    # backward of dispatch with grad_recv = y
    say("  dispatch backward")
    gh = torch.empty((wl.R, wl.S, wl.H), dtype=torch.bfloat16, device=DEV)
    td.moonep_dispatch_backward(dims, pb, y, gh)
    torch.cuda.synchronize()
    # grad_w and grad_hidden, token batch by token batch
    dst_tok = p["dst"].reshape(wl.n_tok, wl.K)
    dst_d = torch.from_numpy(np.maximum(p["dst"], 0).astype(np.int64)).to(DEV)
    yflat, ghflat = y.view(-1, wl.H), gh.view(wl.n_tok, wl.H)
    goflat = gout.view(wl.n_tok, wl.H)
    gwflat = grad_w.view(-1)
    budget = 1 << 29
    stage_y = HostStage(budget)
    stage_h = HostStage(budget // wl.K + wl.row_bytes)
    for t0, n in token_batches(wl.n_tok, wl.K, wl.row_bytes, budget):
        a0, a1 = t0 * wl.K, (t0 + n) * wl.K
        rows_d = yflat.index_select(0, dst_d[a0:a1])
        mag = (goflat[t0:t0 + n].double().abs().repeat_interleave(wl.K, 0) *
               rows_d.double().abs()).sum(1).cpu().numpy()
        y_rows = stage_y.fetch(rows_d)
        loc = local_dst(dst_tok[t0:t0 + n])
        want_w = oracle.combine_backward_w(loc, wl.K, gout_h[t0:t0 + n], y_rows, W.BF16, W.BF16)
        got_w = gwflat[a0:a1].cpu().numpy()
        err = np.abs(got_w.astype(np.float64) - want_w)
        bad = np.nonzero(err > _gamma(wl.H) * mag)[0]
        assert bad.size == 0, f"grad_w off at entries {(a0 + bad[:8]).tolist()}"
        want_h = oracle.dispatch_backward(loc, wl.K, y_rows, W.BF16, W.BF16)
        got_h = stage_h.fetch(ghflat[t0:t0 + n])
        if not np.array_equal(got_h, want_h):
            bad = np.nonzero((got_h != want_h).any(axis=1))[0]
            raise AssertionError(f"dispatch backward differs at tokens {(t0 + bad[:8]).tolist()}")
        del rows_d
    say(f"  ok (grad_w and grad_hidden of all {wl.n_tok} tokens)")
