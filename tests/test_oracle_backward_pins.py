"""Pins of the oracle's backward moves to things other than itself (CPU only).

combine (out[g] = sum_k w[g,k] * y[dst(g,k)]) and dispatch (recv[dst(a)] =
hidden[a / K]) are linear maps; their gradients are fixed by the forward
definitions alone. The pins:
- torch autograd in binary64 of the plain forward definitions (a gather and a
  weighted sum written with torch ops), which yields the exact products and
  near-exact sums the oracle's binary32 / binary64 results are held against
- numpy's nearest-even float64 -> float32 cast and torch's bf16 rounding for the
  one rounding of each grad_y element
- closed forms: unit weights with K = 1 pass grad_out through bit for bit; the
  backward of dispatch applied to the dispatch of bf16 rows sums K equal values
  exactly, giving K * hidden
- binary64 error bounds for the binary32 sums
"""
import numpy as np
import pytest
import torch

import oracle
from tests.test_oracle_pins import _bf16_bits, _routing, _skewed_ids

U32 = 2.0 ** -24


def _as_f32(bits_or_f32, dtype):
    if dtype == oracle.BF16:
        return (bits_or_f32.astype(np.uint32) << 16).view(np.float32)
    return bits_or_f32


def _rows(rng, n, H, dtype):
    x = rng.normal(size=(n, H)).astype(np.float32)
    return _bf16_bits(x) if dtype == oracle.BF16 else x


def _case(seed, drop=False):
    rng = np.random.default_rng(seed)
    R, E, K, S, H = 4, 16, 4, 30, 40
    ids, w = _routing(rng, R, E, K, S)
    if drop:
        ids = ids.copy()
        ids[rng.choice(ids.size, 7, replace=False)] = -1
    p = oracle.plan(R, E, K, S, 4, ids)
    return rng, R, K, S, H, p, w


@pytest.mark.parametrize("y_dt", [oracle.F32, oracle.BF16])
@pytest.mark.parametrize("g_dt", [oracle.F32, oracle.BF16])
@pytest.mark.parametrize("drop", [False, True])
def test_combine_backward_against_autograd(y_dt, g_dt, drop):
    rng, R, K, S, H, p, w = _case(11 + 2 * y_dt + g_dt, drop)
    n_tok, n_slots = R * S, R * S * K
    dst = p["dst"]
    y = _rows(rng, n_slots, H, y_dt)
    gout = _rows(rng, n_tok, H, g_dt)

    # autograd of the plain forward definition, binary64
    valid = torch.from_numpy(dst >= 0)
    y64 = torch.from_numpy(_as_f32(y, y_dt).astype(np.float64)).requires_grad_(True)
    w64 = torch.from_numpy(w.astype(np.float64)).requires_grad_(True)
    rows = y64[torch.from_numpy(np.maximum(dst, 0).astype(np.int64))]
    rows = rows * valid[:, None].to(torch.float64)
    out = (w64[:, None] * rows).view(n_tok, K, H).sum(1)
    (out * torch.from_numpy(_as_f32(gout, g_dt).astype(np.float64))).sum().backward()
    gy_exact = y64.grad.numpy()
    gw_exact = w64.grad.numpy()

    # grad_y: the binary32 product is the nearest-even rounding of the exact one
    fill = 7 if y_dt == oracle.BF16 else np.float32(7.0)
    gy = oracle.combine_backward_y(dst, K, gout, w, g_dt, y_dt, fill=fill)
    want32 = gy_exact.astype(np.float32)
    filled = p["src"] >= 0
    if y_dt == oracle.F32:
        assert np.array_equal(gy[filled].view(np.uint32), want32[filled].view(np.uint32))
    else:
        assert np.array_equal(gy[filled], _bf16_bits(want32[filled]))
    assert np.all(gy[~filled] == fill), "a slot without an entry was written"

    # grad_w in binary64 agrees with autograd to binary64 rounding
    y_rows = y[np.maximum(dst, 0)]
    gw = oracle.combine_backward_w(dst, K, gout, y_rows, g_dt, y_dt)
    mag = np.abs(_as_f32(gout, g_dt).astype(np.float64)).repeat(K, axis=0) * \
        np.abs(_as_f32(y_rows, y_dt).astype(np.float64))
    bound = 2 * H * 2.0 ** -53 * mag.sum(1)
    assert np.all(np.abs(gw - gw_exact) <= bound)
    assert np.all(gw[dst < 0] == 0.0)


def test_combine_backward_unit_weight_k1_passes_grad_through():
    rng = np.random.default_rng(5)
    R, E, K, S, H = 2, 8, 1, 16, 24
    ids = _skewed_ids(rng, R, E, K, S, 2.0)
    p = oracle.plan(R, E, K, S, 2, ids)
    for dt in (oracle.F32, oracle.BF16):
        gout = _rows(rng, R * S, H, dt)
        gy = oracle.combine_backward_y(p["dst"], K, gout, np.ones(R * S, np.float32), dt, dt)
        assert np.array_equal(gy[p["dst"]].view(np.uint8), gout.view(np.uint8))


@pytest.mark.parametrize("in_dt", [oracle.F32, oracle.BF16])
@pytest.mark.parametrize("drop", [False, True])
def test_dispatch_backward_against_autograd(in_dt, drop):
    rng, R, K, S, H, p, _ = _case(21 + in_dt, drop)
    n_tok, n_slots = R * S, R * S * K
    dst, src = p["dst"], p["src"]
    grec = _rows(rng, n_slots, H, in_dt)
    # autograd of the gather recv[slot] = hidden[src(slot) / K], binary64
    h64 = torch.zeros((n_tok, H), dtype=torch.float64, requires_grad=True)
    filled = torch.from_numpy(src >= 0)
    recv = h64[torch.from_numpy(np.maximum(src, 0).astype(np.int64) // K)]
    recv = recv * filled[:, None].to(torch.float64)
    (recv * torch.from_numpy(_as_f32(grec, in_dt).astype(np.float64))).sum().backward()
    exact = h64.grad.numpy()
    gh = oracle.dispatch_backward(dst, K, grec, in_dt, oracle.F32)
    # binary32 sums of at most K terms: within gamma_K of the binary64 sum
    terms = np.abs(_as_f32(grec, in_dt).astype(np.float64))[np.maximum(dst, 0)] * \
        (dst >= 0)[:, None]
    mag = terms.reshape(n_tok, K, H).sum(1)
    gamma = K * U32 / (1 - K * U32)
    assert np.all(np.abs(gh.astype(np.float64) - exact) <= gamma * mag)
    # integer-valued gradients sum exactly, in any order
    gi = rng.integers(-500, 500, size=(n_slots, H)).astype(np.float32)
    gh_i = oracle.dispatch_backward(dst, K, gi, oracle.F32, oracle.F32)
    want = np.zeros((n_tok, H))
    for a in range(dst.size):
        if dst[a] >= 0:
            want[a // K] += gi[dst[a]]
    assert np.array_equal(gh_i, want.astype(np.float32))
    # the bf16 output is the nearest-even rounding of the binary32 sum
    assert np.array_equal(oracle.dispatch_backward(dst, K, grec, in_dt, oracle.BF16),
                          _bf16_bits(gh))


@pytest.mark.parametrize("K", [1, 2, 4, 8])
def test_dispatch_backward_of_dispatch_is_k_times_hidden(K):
    """Each token's K slots hold copies of its bf16 row; summing K equal bf16
    values needs at most 8 + 3 significant bits, so the binary32 sum is exact and
    K * x is a bf16 value when K is a power of two."""
    rng = np.random.default_rng(30 + K)
    R, E, S, H = 4, 16, 25, 32
    ids, _ = _routing(rng, R, E, K, S)
    p = oracle.plan(R, E, K, S, 4, ids)
    hidden = _rows(rng, R * S, H, oracle.BF16)
    recv = oracle.dispatch(p, K, hidden)
    back = oracle.dispatch_backward(p["dst"], K, recv, oracle.BF16, oracle.BF16)
    assert np.array_equal(back, _bf16_bits(K * _as_f32(hidden, oracle.BF16)))


@pytest.mark.parametrize("out_dt", [oracle.F32, oracle.BF16])
def test_dispatch_backward_sum_starts_from_positive_zero(out_dt):
    """The backward of dispatch adds from +0.0 (the reading of its definition).
    A token whose K entries are all dropped then gets +0.0, and so does a token
    whose every slot gradient is -0.0, because (+0) + (-0) = +0 when rounding to
    nearest; a -0.0 start would give -0.0 in both cases."""
    K, H = 2, 4
    dst = np.array([-1, -1, 0, 1], dtype=np.int32)  # token 0 dropped, token 1 in slots 0 and 1
    grec = np.full((2, H), -0.0, dtype=np.float32)
    gh = oracle.dispatch_backward(dst, K, grec, oracle.F32, out_dt)
    bits = gh.view(np.uint32) if out_dt == oracle.F32 else gh.view(np.uint16)
    assert not np.any(bits)
