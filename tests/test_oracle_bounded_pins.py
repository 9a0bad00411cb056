"""Pins of the oracle's bounded plan (at most B duplicates per rank where it can)
to things other than itself (CPU only).

- hand-worked examples under tests/golden/bounded_example*.json (each names the
  passage it follows and how it was derived)
- the invariants every balanced plan has (tests/invariants.py): exactly S*K rows
  per rank, dst/src a bijection, each entry on its home rank or on a rank that
  holds a duplicate of its expert, contiguous experts, the minimum number of
  moved rows, the merge bound on pieces, the list order and the status bits
- brute force: the experts an overloaded rank overflows are as few as any
  choice of its home experts allows (every subset is tried on small ranks)
- structure: those experts are the largest by (T descending, id), all but the
  last move whole, and every expert keeps its first entries at home
- closed forms: balanced routing moves nothing and gives the water-fill's plan;
  one overloaded rank with one dominant expert gives one duplicate per
  receiving rank
"""
import glob
import itertools
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W
from tests.invariants import check_plan
from tests.test_oracle_pins import _skewed_ids

GOLDEN = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "bounded_example*.json")))


@pytest.mark.parametrize("path", GOLDEN, ids=[os.path.basename(g) for g in GOLDEN])
def test_bounded_hand_worked_examples(path):
    ex = json.load(open(path))
    R, E, K, S, B = ex["R"], ex["E"], ex["K"], ex["S"], ex["B"]
    G, SK = E // R, S * K
    ids = np.array(ex["ids"], dtype=np.int32)
    p = oracle.plan(R, E, K, S, B, ids, bounded=True)
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
    hidden = np.arange(R * S, dtype=np.int32).reshape(R * S, 1)
    assert oracle.dispatch(p, K, hidden).reshape(R, SK).tolist() == x["recv_tokens"]
    expert_w = np.repeat(np.arange(E, dtype=np.int64)[:, None], 4, axis=1)
    want = np.zeros((R, B, 4), dtype=np.int64)
    for r, b, e in x["replicated"]:
        want[r, b, :] = e
    assert np.array_equal(oracle.replicate(p, B, expert_w), want)
    check_plan(R, E, K, S, B, ids, p)


def _overflow_rows(p, ids, R, E, K, S):
    """Per expert: how many of its entries left the home rank (from dst)."""
    G, SK = E // R, S * K
    ids = np.asarray(ids).reshape(-1)
    ok = (ids >= 0) & (ids < E)
    away = (p["dst"] // SK) != (ids // G)
    return np.bincount(ids[ok & away], minlength=E)


def _check_structure(R, E, K, S, ids, p):
    G, SK = E // R, S * K
    ids = np.asarray(ids).reshape(-1)
    T = p["T"].astype(np.int64)
    ov = _overflow_rows(p, ids, R, E, K, S)
    for r in range(R):
        home = np.arange(r * G, (r + 1) * G)
        O = int(p["O"][r])
        assert int(ov[home].sum()) == O
        order = sorted(home.tolist(), key=lambda e: (-int(T[e]), e))
        moved = [e for e in order if ov[e] > 0]
        assert moved == order[:len(moved)], "overflow is not taken from the largest experts"
        for e in moved[:-1]:
            assert ov[e] == T[e], "an expert before the last one in the order did not move whole"
    # every expert keeps its first entries at home, in entry order
    for e in range(E):
        where = np.nonzero(ids == e)[0]
        at_home = (p["dst"][where] // SK) == e // G
        k = int(at_home.sum())
        assert np.all(at_home[:k]) and not np.any(at_home[k:]), "kept entries are not a prefix"


def _min_experts_to_cover(Ts, O):
    for m in range(len(Ts) + 1):
        if any(sum(c) >= O for c in itertools.combinations(Ts, m)):
            return m
    return len(Ts)


@pytest.mark.parametrize("seed", range(16))
def test_bounded_random_invariants_and_structure(seed):
    rng = np.random.default_rng(300 + seed)
    R = int(rng.choice([1, 2, 3, 4, 6, 8]))
    G = int(rng.integers(1, 7))
    E = R * G
    K = int(rng.integers(1, min(E, 6) + 1))
    S = int(rng.integers(1, 50))
    B = int(rng.integers(0, 5))
    ids = _skewed_ids(rng, R, E, K, S, skew=float(rng.choice([0.0, 1.0, 2.5, 4.0])))
    p = oracle.plan(R, E, K, S, B, ids, bounded=True)
    check_plan(R, E, K, S, B, ids, p)
    _check_structure(R, E, K, S, ids, p)
    # as few overflowing experts per rank as any subset of its home experts allows
    T = p["T"].astype(np.int64)
    ov = _overflow_rows(p, ids, R, E, K, S)
    for r in range(R):
        home = list(range(r * G, (r + 1) * G))
        n_moved = int(np.sum(ov[home] > 0))
        assert n_moved == _min_experts_to_cover([int(T[e]) for e in home], int(p["O"][r]))


def test_bounded_with_dropped_and_repeated_ids():
    rng = np.random.default_rng(41)
    R, E, K, S = 4, 12, 3, 25
    for trial in range(8):
        ids = _skewed_ids(rng, R, E, K, S, 2.5)
        if trial % 2 == 0:
            ids[rng.integers(0, ids.size, 6)] = rng.choice([-1, E, E + 2], 6)
        else:
            t = rng.integers(0, R * S, 3)
            ids[t * K + 2] = ids[t * K]
        p = oracle.plan(R, E, K, S, 3, ids, bounded=True)
        check_plan(R, E, K, S, 3, ids, p, valid_input=(trial % 2 == 1))


def test_bounded_equals_water_fill_when_balanced():
    """No rank is overloaded: nothing moves, and both plans are the stable
    counting sort of the entries by expert."""
    R, E, K, S = 4, 16, 4, 32
    ids = (np.arange(R * S * K) % E).astype(np.int32)
    a = oracle.plan(R, E, K, S, 2, ids, bounded=True)
    b = oracle.plan(R, E, K, S, 2, ids)
    for k in ("dst", "src", "n_dup", "seg_ptr", "dup_ptr", "status"):
        assert np.array_equal(a[k], b[k]), k
    assert int(a["n_dup"].sum()) == 0
    assert np.array_equal(a["dst"], np.argsort(np.argsort(ids, kind="stable"), kind="stable")
                          .astype(np.int32))


def test_bounded_one_dominant_expert():
    """Rank 0 holds 40 rows of expert 0 and 4 of expert 1 (S*K = 16, so 28 must
    leave); ranks 1-3 have room 12, 8 and 8. The 28 rows leave through expert 0
    alone, and each receiving rank gets exactly one duplicate, of expert 0."""
    R, E, K, S = 4, 8, 1, 16
    ids = np.array([0] * 40 + [1] * 4 + [3] * 4 + [4] * 8 + [6] * 8, dtype=np.int32)
    p = oracle.plan(R, E, K, S, 4, ids, bounded=True)
    check_plan(R, E, K, S, 4, ids, p)
    assert p["O"].tolist() == [28, 0, 0, 0] and p["D"].tolist() == [0, 12, 8, 8]
    ov = _overflow_rows(p, ids, R, E, K, S)
    assert int(ov[0]) == 28 and int(ov[1]) == 0
    assert p["n_dup"].tolist() == [0, 1, 1, 1]
    assert p["dup_expert"][1:, 0].tolist() == [0, 0, 0]
    assert p["dup_count"][1:, 0].tolist() == [12, 8, 8]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bounded_decode_workload_within_b(seed):
    """On the decode-shaped workload (B = 4) the bounded plan needs no rank above
    B, where the water-fill needs 10 to 23 on its worst rank."""
    wl = W.WORKLOADS["decode"]
    ids, _ = W.make_routing(wl, seed)
    p = oracle.plan(wl.R, wl.E, wl.K, wl.S, wl.B, ids, bounded=True)
    assert int(p["n_dup"].max()) <= wl.B and int(p["status"][0]) == 0
    q = oracle.plan(wl.R, wl.E, wl.K, wl.S, wl.B, ids)
    assert int(q["n_dup"].max()) > wl.B
    # the same rows move: only the choice of which rows, and where, differs
    assert np.array_equal(p["O"], q["O"]) and np.array_equal(p["D"], q["D"])
