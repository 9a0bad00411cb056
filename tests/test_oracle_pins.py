"""Pins of the CPU oracle to things other than itself (CPU only).

- hand-worked examples under tests/golden/ (each file names the passage it follows)
- library routines: numpy bincount for the histogram, numpy stable argsort in an
  independent sort-and-slice formulation of the plan, torch's bf16 rounding
- brute force: every routing of several tiny shapes against the sort-and-slice plan
- closed forms: balanced routing gives maxvio = 0 and a plain stable counting
  sort; all tokens on the same K experts give maxvio = E/K - 1; identity
  experts with weights 1/K give back the hidden rows bit for bit
- error bounds: the binary32 combine and reduce against binary64 sums
- invariants of any balanced plan (tests/invariants.py)
"""
import glob
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from tests.invariants import check_plan
from tests.plan_by_sorting import plan_by_sorting

GOLDEN = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "plan_example*.json")))


def _compare_to_sorting(R, E, K, S, ids, p):
    q = plan_by_sorting(R, E, K, S, ids)
    assert np.array_equal(p["T"], q["T"])
    assert np.array_equal(p["dst"], q["dst"])
    assert np.array_equal(p["src"], q["src"])
    assert np.array_equal(p["n_dup"], q["n_dup"])
    for (r, b, e, s0, n) in q["dups"]:
        assert (p["dup_expert"][r, b], p["dup_start"][r, b], p["dup_count"][r, b]) == (e, s0, n)
    nl = int(p["n_list"][0])
    got = list(zip(p["list_expert"][:nl].tolist(), p["list_rank"][:nl].tolist(),
                   p["list_b"][:nl].tolist()))
    assert got == [tuple(x) for x in q["list"]]
    assert np.array_equal(p["dup_ptr"], q["dup_ptr"])


@pytest.mark.parametrize("path", GOLDEN, ids=[os.path.basename(g) for g in GOLDEN])
def test_hand_worked_examples(path):
    ex = json.load(open(path))
    R, E, K, S, B = ex["R"], ex["E"], ex["K"], ex["S"], ex["B"]
    G, SK = E // R, S * K
    ids = np.array(ex["ids"], dtype=np.int32)
    p = oracle.plan(R, E, K, S, B, ids)
    x = ex["expect"]
    assert int(p["status"][0]) == x["status"]
    assert int(p["maxT"][0]) == x["maxT"]
    assert float(p["maxvio"][0]) == x["maxvio"]
    for k in ("T", "hoff", "L", "keep", "O", "D", "Opre", "Dpre", "n_dup", "dup_ptr"):
        assert p[k].tolist() == x[k], k
    assert [[d // SK, d % SK] for d in p["dst"].tolist()] == x["dst_rank_slot"]
    got_dups = [[r, b, int(p["dup_expert"][r, b]), int(p["dup_start"][r, b]),
                 int(p["dup_count"][r, b])] for r in range(R) for b in range(int(p["n_dup"][r]))]
    assert got_dups == x["dups"]
    for r in range(R):
        ns = G + int(p["n_dup"][r])
        assert p["seg_ptr"][r, :ns + 1].tolist() == x["seg_ptr"][r]
        assert p["seg_expert"][r, :ns].tolist() == x["seg_expert"][r]
    nl = int(p["n_list"][0])
    assert [[int(p["list_expert"][i]), int(p["list_rank"][i]), int(p["list_b"][i])]
            for i in range(nl)] == x["list"]
    # dispatch: rows carry their token index, so recv shows which token each slot got
    hidden = np.arange(R * S, dtype=np.int32).reshape(R * S, 1)
    recv = oracle.dispatch(p, K, hidden)
    assert recv.reshape(R, SK).tolist() == x["recv_tokens"]
    # replicate: blocks carry their expert id
    expert_w = np.repeat(np.arange(E, dtype=np.int64)[:, None], 4, axis=1)
    dup_w = oracle.replicate(p, B, expert_w)
    want = np.zeros((R, B, 4), dtype=np.int64)
    for r, b, e in x["replicated"]:
        want[r, b, :] = e
    assert np.array_equal(dup_w, want)
    if "reduce" in ex:
        rd = ex["reduce"]
        home = np.array(rd["home_before"], dtype=np.float32)
        dup = np.array(rd["dup_grads"], dtype=np.float32)
        out = oracle.reduce_dup_grads(p, B, dup, home)
        assert out.tolist() == rd["home_after"]
    if "combine" in ex:
        cb = ex["combine"]
        y = np.arange(R * SK, dtype=np.float32).reshape(R * SK, 1)
        out = oracle.combine(p["dst"], K, y, np.array(cb["w"], np.float32), oracle.F32, oracle.F32)
        assert out.reshape(-1).tolist() == cb["out"]
    check_plan(R, E, K, S, B, ids, p)


def test_combine_is_fused_multiply_add():
    ex = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "combine_fma.json")))
    y = np.array(ex["y"], np.float32).reshape(-1, 1)
    dst = np.array(ex["dst"], np.int32)
    w = np.array(ex["w"], np.float32)
    out = oracle.combine(dst, ex["K"], y, w, oracle.F32, oracle.F32)
    assert out.reshape(-1).tolist() == [ex["out_f32"]]
    outb = oracle.combine(dst, ex["K"], y, w, oracle.F32, oracle.BF16)
    assert outb.reshape(-1).tolist() == [ex["out_bf16_bits"]]


def test_combine_starts_from_positive_zero():
    ex = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "combine_zero_sign.json")))
    y = np.array(ex["y"], np.float32).reshape(-1, 1)
    dst = np.array(ex["dst"], np.int32)
    w = np.array(ex["w"], np.float32)
    out = oracle.combine(dst, ex["K"], y, w, oracle.F32, oracle.F32)
    assert int(out.view(np.uint32).reshape(-1)[0]) == ex["out_f32_bits"]
    outb = oracle.combine(dst, ex["K"], y, w, oracle.F32, oracle.BF16)
    assert outb.reshape(-1).tolist() == [ex["out_bf16_bits"]]


def test_histogram_is_bincount():
    rng = np.random.default_rng(5)
    for R, E, K, S in [(4, 32, 4, 100), (8, 64, 8, 33), (3, 9, 2, 7)]:
        ids = np.stack([rng.permutation(E)[:K] for _ in range(R * S)]).astype(np.int32)
        p = oracle.plan(R, E, K, S, 4, ids)
        assert np.array_equal(p["T"], np.bincount(ids.ravel(), minlength=E))


def test_maxvio_closed_forms():
    # perfectly balanced: token g takes experts (g*K + k) mod E; R*S*K divisible by E
    R, E, K, S = 4, 16, 4, 8
    ids = (np.arange(R * S * K) % E).astype(np.int32)
    p = oracle.plan(R, E, K, S, 1, ids)
    assert float(p["maxvio"][0]) == 0.0
    assert np.all(p["T"] == R * S * K // E)
    assert int(p["n_dup"].sum()) == 0 and np.all(p["O"] == 0) and np.all(p["D"] == 0)
    # all tokens routed to the same K experts: T = R*S on those, maxvio = E/K - 1
    for (R, E, K, S) in [(4, 16, 2, 8), (2, 8, 4, 3), (8, 64, 8, 5)]:
        ids = np.tile(np.arange(K, dtype=np.int32)[::-1], R * S)
        p = oracle.plan(R, E, K, S, E // R, ids)
        assert float(p["maxvio"][0]) == E / K - 1.0
        check_plan(R, E, K, S, E // R, ids, p)


def test_balanced_is_stable_counting_sort():
    """With every L_r = S*K nothing moves; each rank is a stable sort by expert."""
    rng = np.random.default_rng(11)
    R, E, K, S = 4, 16, 2, 24
    G, SK = E // R, S * K
    for _ in range(20):
        # route so that each rank's home load is exactly S*K: shuffle a multiset
        # holding S*K assignments per home rank, then pair them into tokens
        pool = np.concatenate([rng.integers(r * G, (r + 1) * G, size=SK) for r in range(R)])
        ids = rng.permutation(pool).astype(np.int32)
        p = oracle.plan(R, E, K, S, 2, ids)
        assert np.all(p["L"] == SK) and int(p["n_dup"].sum()) == 0
        for r in range(R):
            mine = np.nonzero(ids // G == r)[0]
            order = mine[np.argsort(ids[mine], kind="stable")]
            assert np.array_equal(p["src"][r * SK:(r + 1) * SK], order)


def _enumerate(R, E, K, S, allow_repeat=False):
    if allow_repeat:
        token_choices = list(itertools.product(range(E), repeat=K))
    else:
        token_choices = list(itertools.permutations(range(E), K))
    for combo in itertools.product(token_choices, repeat=R * S):
        yield np.array(combo, dtype=np.int32).reshape(-1)


@pytest.mark.parametrize("R,E,K,S,rep", [
    (2, 4, 1, 1, False), (2, 4, 1, 2, False), (2, 4, 1, 3, False),
    (2, 4, 2, 1, False), (2, 4, 2, 2, False), (3, 3, 1, 2, False),
    (2, 2, 2, 2, True), (4, 4, 1, 2, False),
])
def test_bruteforce_against_sorting(R, E, K, S, rep):
    n = 0
    for i, ids in enumerate(_enumerate(R, E, K, S, rep)):
        B = 2
        p = oracle.plan(R, E, K, S, B, ids)
        _compare_to_sorting(R, E, K, S, ids, p)
        if i % 97 == 0:
            check_plan(R, E, K, S, B, ids, p)
        n += 1
    assert n == (E ** K if rep else int(np.prod(range(E - K + 1, E + 1)))) ** (R * S)


def _skewed_ids(rng, R, E, K, S, skew):
    bias = rng.normal(0.0, skew, size=E)
    scores = rng.normal(size=(R * S, E)) + bias
    return np.argsort(-scores, axis=1, kind="stable")[:, :K].astype(np.int32).reshape(-1)


@pytest.mark.parametrize("seed", range(12))
def test_random_skewed_against_sorting(seed):
    rng = np.random.default_rng(100 + seed)
    R = int(rng.choice([1, 2, 3, 4, 8]))
    G = int(rng.integers(1, 6))
    E = R * G
    K = int(rng.integers(1, min(E, 6) + 1))
    S = int(rng.integers(1, 40))
    ids = _skewed_ids(rng, R, E, K, S, skew=float(rng.choice([0.0, 1.0, 3.0])))
    B = int(rng.integers(0, 4))
    p = oracle.plan(R, E, K, S, B, ids)
    _compare_to_sorting(R, E, K, S, ids, p)
    check_plan(R, E, K, S, B, ids, p)


def test_invalid_and_repeated_ids():
    rng = np.random.default_rng(7)
    R, E, K, S = 4, 12, 3, 20
    for trial in range(10):
        ids = _skewed_ids(rng, R, E, K, S, 2.0)
        if trial % 2 == 0:
            ids[rng.integers(0, ids.size, 5)] = rng.choice([-1, E, E + 3, -7], 5)
        else:
            t = rng.integers(0, R * S, 3)
            ids[t * K + 1] = ids[t * K]
        p = oracle.plan(R, E, K, S, 8, ids)
        _compare_to_sorting(R, E, K, S, ids, p)
        check_plan(R, E, K, S, 8, ids, p, valid_input=(trial % 2 == 1))
        st = int(p["status"][0])
        assert (st & oracle.ST_BAD_ID) == (oracle.ST_BAD_ID if trial % 2 == 0 else 0)
        assert bool(st & oracle.ST_REPEAT_ID) == (trial % 2 == 1)


@pytest.mark.parametrize("bounded", [False, True])
def test_every_id_dropped_closed_form(bounded):
    """No valid assignment at all: T = 0, maxvio = 0 * E / (R*S*K) - 1 = -1, every
    rank keeps nothing and has a deficit of S*K, nothing overflows, every entry
    and every slot is empty, and the bad-id bit is set."""
    R, E, K, S = 3, 9, 2, 7
    for fill in (-1, E, -5):
        ids = np.full(R * S * K, fill, dtype=np.int32)
        p = oracle.plan(R, E, K, S, 2, ids, bounded=bounded)
        assert not np.any(p["T"]) and float(p["maxvio"][0]) == -1.0
        assert not np.any(p["L"]) and not np.any(p["keep"]) and not np.any(p["O"])
        assert np.all(p["D"] == S * K) and p["Dpre"].tolist() == [r * S * K for r in range(R + 1)]
        assert np.all(p["dst"] == -1) and np.all(p["src"] == -1)
        assert not np.any(p["n_dup"]) and int(p["n_list"][0]) == 0
        assert int(p["status"][0]) == oracle.ST_BAD_ID


# ------------------------------------------------------------------ data moves

def _bf16_bits(x):
    import torch
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def test_bf16_rounding_is_torch_rne():
    import torch
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.normal(size=20000).astype(np.float32),
        (rng.normal(size=2000) * 1e-39).astype(np.float32),          # subnormals
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1.0, 1.00390625,
                  1.005859375, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], np.float32),
    ])
    # exact ties: bf16 values +/- half an ulp
    base = rng.normal(size=4000).astype(np.float32)
    bits = base.view(np.uint32) & np.uint32(0xFFFF0000)
    ties = (bits | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties])
    assert np.array_equal(oracle.f32_to_bf16(x), _bf16_bits(x))
    nan = oracle.f32_to_bf16(np.array([np.nan], np.float32))
    back = torch.from_numpy(nan.view(np.int16)).view(torch.bfloat16).float()
    assert torch.isnan(back).all()


def _routing(rng, R, E, K, S):
    ids = _skewed_ids(rng, R, E, K, S, 1.5)
    logit = rng.normal(size=(R * S, K))
    w = np.exp(logit) / np.exp(logit).sum(1, keepdims=True)
    return ids, w.astype(np.float32).reshape(-1)


def test_combine_k1_unit_weight_is_gather():
    rng = np.random.default_rng(1)
    R, E, K, S, H = 2, 8, 1, 16, 24
    ids, _ = _routing(rng, R, E, K, S)
    p = oracle.plan(R, E, K, S, 4, ids)
    y = rng.normal(size=(R * S * K, H)).astype(np.float32)
    out = oracle.combine(p["dst"], K, y, np.ones(R * S * K, np.float32), oracle.F32, oracle.F32)
    assert np.array_equal(out, y[p["dst"]])


@pytest.mark.parametrize("K", [1, 2, 4, 8])
def test_combine_identity_expert_mean_is_exact(K):
    """y = recv (identity expert), w = 1/K: every partial sum m*x/K needs at most
    8 + 3 significant bits, so the bf16 result is the hidden row bit for bit."""
    rng = np.random.default_rng(K)
    R, E, S, H = 4, 16, 20, 40
    ids, _ = _routing(rng, R, E, K, S)
    p = oracle.plan(R, E, K, S, 4, ids)
    hidden = _bf16_bits(rng.normal(size=(R * S, H)))
    recv = oracle.dispatch(p, K, hidden)
    w = np.full(R * S * K, 1.0 / K, np.float32)
    out = oracle.combine(p["dst"], K, recv, w, oracle.BF16, oracle.BF16)
    assert np.array_equal(out, hidden)


@pytest.mark.parametrize("dt", [oracle.F32, oracle.BF16])
def test_combine_within_binary64_error_bound(dt):
    rng = np.random.default_rng(9)
    R, E, K, S, H = 4, 32, 8, 30, 64
    ids, w = _routing(rng, R, E, K, S)
    p = oracle.plan(R, E, K, S, 8, ids)
    yf = rng.normal(size=(R * S * K, H)).astype(np.float32)
    y = _bf16_bits(yf) if dt == oracle.BF16 else yf
    yv = (y.astype(np.uint32) << 16).view(np.float32) if dt == oracle.BF16 else y
    out = oracle.combine(p["dst"], K, y, w, dt, oracle.F32)
    prod = w.astype(np.float64).reshape(-1, K, 1) * yv[p["dst"]].astype(np.float64).reshape(-1, K, H)
    exact = prod.sum(axis=1)
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    bound = gamma * np.abs(prod).sum(axis=1)
    assert np.all(np.abs(out.astype(np.float64) - exact) <= bound)
    # and the bf16 output is the nearest-even rounding of that accumulator
    outb = oracle.combine(p["dst"], K, y, w, dt, oracle.BF16)
    assert np.array_equal(outb, _bf16_bits(out))


def test_reduce_integer_grads_and_error_bound():
    rng = np.random.default_rng(4)
    R, E, K, S, n = 4, 16, 4, 64, 33
    ids = _skewed_ids(rng, R, E, K, S, 3.0)
    B = 6
    p = oracle.plan(R, E, K, S, B, ids)
    assert int(p["n_dup"].sum()) > 0
    for integer in (True, False):
        if integer:
            dup = rng.integers(-1000, 1000, size=(R, B, n)).astype(np.float32)
            home = rng.integers(-1000, 1000, size=(E, n)).astype(np.float32)
        else:
            dup = rng.normal(size=(R, B, n)).astype(np.float32)
            home = rng.normal(size=(E, n)).astype(np.float32)
        out = oracle.reduce_dup_grads(p, B, dup, home)
        exact = home.astype(np.float64).copy()
        mag = np.abs(home).astype(np.float64)
        cnt = np.zeros(E)
        for r in range(R):
            for b in range(min(int(p["n_dup"][r]), B)):
                e = int(p["dup_expert"][r, b])
                exact[e] += dup[r, b]
                mag[e] += np.abs(dup[r, b])
                cnt[e] += 1
        if integer:
            assert np.array_equal(out, exact.astype(np.float32))
        else:
            u = 2.0 ** -24
            gamma = (cnt * u / (1 - cnt * u))[:, None]
            assert np.all(np.abs(out - exact) <= gamma * mag)
        untouched = cnt == 0
        assert np.array_equal(out[untouched], home[untouched])


def test_dispatch_covers_every_slot_once():
    rng = np.random.default_rng(2)
    R, E, K, S, H = 4, 16, 4, 50, 8
    ids = _skewed_ids(rng, R, E, K, S, 2.0)
    p = oracle.plan(R, E, K, S, 4, ids)
    hidden = np.arange(R * S, dtype=np.int64)[:, None] * 1000 + np.arange(H)
    recv = oracle.dispatch(p, K, hidden)
    tok = recv[:, 0] // 1000
    assert np.array_equal(np.sort(np.bincount(tok, minlength=R * S)), np.full(R * S, K))
    assert np.array_equal(tok, p["src"] // K)
    # streaming by window gives the same rows
    SK = S * K
    for r in range(R):
        part = oracle.dispatch(p, K, hidden, r * SK, (r + 1) * SK)
        assert np.array_equal(part, recv[r * SK:(r + 1) * SK])
