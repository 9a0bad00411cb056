"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Plan arrays, dispatch and replicate bytes are compared bit for bit. Combine and
reduce accumulate in binary32 in the same fixed order as the oracle, so they are
compared bit for bit too, which is stricter than the 1e-5 relative bound the
path promises (that bound is also asserted on the fp32 combine output).

Both plans are covered: the water-fill (moonep_plan) and the plan bounded by B
duplicates per rank (moonep_plan_bounded), each against its oracle.

Small shapes are compared element by element; they span several plan tiles with
a ragged last tile and rows whose 16-byte chunk count does not fill the lanes.
The five workload shapes are run at full size in the launch configuration the
benchmark times, for seeds 0, 1 and 2: the whole plan is compared, dispatch and
replicate are checked everywhere against the oracle's plan tables, combine on
every token and reduce on every expert with duplicates through the oracle
(batches of rows streamed to the host), the other experts checked untouched.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_common import (PLAN_INT_KEYS, HostStage, assert_plan_equal, bf16_bits, f32_bits,
                              local_dst, other_form, read_plan, run_plan, say, token_batches)
from tests.invariants import check_plan

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def td():
    if not torch.cuda.is_available():
        pytest.fail("GPU parity tests need a GPU")
    import token_dispatch_amd as td
    torch.cuda.set_device(DEV)
    return td


def _wl(name, R, E, K, S, B, H, dtype, skew, block=(8, 36)):
    return W.Workload(name, R=R, E=E, K=K, S=S, H=H, dtype=dtype, B=B, block_shape=block,
                      block_dtype=W.BF16, routing="bias", bias_std=skew)


SMALL = [
    # several tiles with a ragged tail; fp32 rows of 18 chunks (ragged lanes)
    _wl("tiles_ragged", 4, 32, 4, 3001, 4, 72, W.F32, 2.0),
    # bf16 rows of 125 chunks: two chunks per lane, ragged
    _wl("bf16_ragged_row", 8, 64, 8, 700, 8, 1000, W.BF16, 1.5),
    _wl("k1", 2, 8, 1, 5000, 2, 64, W.BF16, 3.0),
    # one home expert per rank, 16-byte rows
    _wl("g1", 6, 6, 2, 333, 3, 8, W.BF16, 2.0),
    # a single rank: nothing can overflow; no duplicate slots
    _wl("r1", 1, 16, 4, 2000, 0, 32, W.F32, 1.0),
    _wl("k64", 2, 128, 64, 300, 64, 256, W.BF16, 1.0),
    _wl("s1", 16, 64, 8, 1, 4, 128, W.BF16, 3.0),
    # rows longer than one 16-chunk-per-lane segment (two segments)
    _wl("long_row", 2, 16, 2, 200, 2, 12288, W.BF16, 2.0),
    _wl("e1024", 8, 1024, 8, 600, 128, 64, W.BF16, 2.0),
    # the largest rank and expert counts: one home expert per rank, 1024 ranks
    _wl("r1024", 1024, 1024, 2, 4, 2, 8, W.BF16, 2.0),
    # fp32 rows and a larger fp32 weight block
    _wl("f32_wide", 4, 16, 2, 1000, 4, 1024, W.F32, 2.5, block=(3, 64, 64)),
    # K that is not a power of two: tokens straddle 64-entry chunks, tiles hold
    # 4096 // K whole tokens, and the count kernel takes scalar id loads
    _wl("k3_r3", 3, 27, 3, 1001, 3, 16, W.BF16, 2.5),
    _wl("k6", 4, 48, 6, 777, 4, 64, W.BF16, 2.0),
    _wl("k12_f32", 8, 96, 12, 300, 6, 40, W.F32, 1.5),
    _wl("k40", 2, 80, 40, 120, 8, 64, W.BF16, 1.0),
    # four launches with 2048-entry plan tiles (two 64-entry chunks per assign
    # wave), ragged last tile
    _wl("tiles_2048", 8, 1024, 8, 8200, 8, 64, W.BF16, 2.0),
    # two launches with 2048- and 4096-entry tiles (n_tiles * E just within the
    # fused kernel's count budget)
    _wl("fused_2048", 8, 1024, 8, 1500, 8, 64, W.BF16, 2.0),
    _wl("fused_4096", 8, 1024, 8, 3000, 8, 64, W.BF16, 2.0),
    # the tiny workload as given: fp32 rows, fp32 [128, 256] weight blocks
    W.WORKLOADS["tiny"],
    # 7 and 16 chunks per lane (rows of 425 or 426 and 1000 16-byte chunks,
    # ragged), in bf16 and fp32 rows
    _wl("cpl7_bf16", 4, 16, 4, 300, 4, 3400, W.BF16, 2.0),
    _wl("cpl7_f32", 2, 8, 2, 400, 2, 1704, W.F32, 2.0),
    _wl("cpl16_bf16", 2, 8, 4, 250, 2, 8000, W.BF16, 1.5),
    _wl("cpl16_f32", 2, 8, 2, 500, 2, 4000, W.F32, 2.0),
    # an expert with more than 2^21 entries (2 387 355 at seed 0): the bounded
    # placement's (rows, id) keys no longer pack into one word, and it takes its
    # three-reduction path; two overflowing experts, pieces on three ranks
    _wl("big_counts", 4, 8, 2, 600_000, 2, 8, W.BF16, 5.0),
    # more than 64 overflowing experts (103, 206 and 408 at seed 3): the bounded
    # placement holds them in 2, 4 and 8 registers per lane and searches them
    # with reductions; up to 64 it keeps them sorted across one wave instead
    _wl("over_103", 512, 1024, 4, 8, 2, 64, W.BF16, 1.0),
    _wl("over_206", 512, 1024, 8, 8, 2, 64, W.BF16, 0.3),
    _wl("over_408", 1024, 1024, 2, 4, 2, 64, W.BF16, 0.0),
]


def _dims(td, wl):
    return td.Dims(wl.R, wl.E, wl.K, wl.S, wl.B, wl.dtype, wl.H)


def _host_rows(t):
    """Bits of a row tensor as numpy (uint16 for bf16, float32 for fp32)."""
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.detach().contiguous().cpu().numpy()


def _full_case(td, wl, ids, w, seed, bounded=False):
    """Everything compared element by element (small shapes only)."""
    dims = _dims(td, wl)
    say(f"case {wl.name} bounded={bounded}: {dims}")
    plan_buf, _ = run_plan(td, dims, ids, DEV, bounded=bounded)
    g = read_plan(td, dims, plan_buf)
    p = oracle.plan(wl.R, wl.E, wl.K, wl.S, wl.B, ids, bounded=bounded)
    assert_plan_equal(g, p)
    valid = bool(np.all((ids >= 0) & (ids < wl.E)))
    check_plan(wl.R, wl.E, wl.K, wl.S, wl.B, ids, g, valid_input=valid)
    # the other launch form gives the same plan
    form = other_form(td, dims)
    buf2, _ = run_plan(td, dims, ids, DEV, bounded=bounded, form=form)
    assert_plan_equal(read_plan(td, dims, buf2), p)
    del buf2

    hidden = W.make_hidden(wl, seed)
    hid_d = hidden.to(DEV)
    recv = torch.full((wl.R, wl.SK, wl.H), 7.0, dtype=hid_d.dtype, device=DEV)
    td.moonep_dispatch(dims, plan_buf, hid_d, recv)
    torch.cuda.synchronize()
    hid_h = _host_rows(hidden).reshape(wl.n_tok, wl.H)
    want = oracle.dispatch(p, wl.K, hid_h)
    got = _host_rows(recv).reshape(-1, wl.H)
    filled = p["src"] >= 0
    assert np.array_equal(got[filled].view(np.uint8), want[filled].view(np.uint8)), "dispatch"

    # combine reads expert outputs y; here y = a fresh seeded tensor in recv layout
    y = W.make_expert_out(wl, seed)
    y_d = y.to(DEV)
    w_d = torch.from_numpy(w).to(DEV)
    y_h = _host_rows(y).reshape(-1, wl.H)
    for od in (W.F32, W.BF16):
        out = torch.empty((wl.R, wl.S, wl.H), dtype=W.torch_dtype(od), device=DEV)
        td.moonep_combine(dims, plan_buf, y_d, w_d, out, od)
        torch.cuda.synchronize()
        want = oracle.combine(p["dst"], wl.K, y_h, w, wl.dtype, od)
        got = _host_rows(out).reshape(-1, wl.H)
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), f"combine out_dtype={od}"
        if od == W.F32:
            rel = np.abs(got.astype(np.float64) - want) / np.maximum(np.abs(want), 1e-30)
            assert np.all(rel <= 1e-5)

    # replicate and reduce
    ew = W.make_expert_weights(wl, seed)
    ew_d = ew.to(DEV)
    dup_w = torch.zeros((wl.R, wl.B) + tuple(wl.block_shape), dtype=ew.dtype, device=DEV)
    td.moonep_replicate(dims, plan_buf, ew_d, dup_w, wl.block_bytes)
    dg, hg = W.make_grads(wl, seed)
    hg_d = hg.to(DEV)
    td.moonep_reduce_dup_grads(dims, plan_buf, dg.to(DEV), hg_d, wl.block_elems)
    torch.cuda.synchronize()
    want_w = oracle.replicate(p, wl.B, bf16_bits(ew) if ew.dtype == torch.bfloat16 else ew.numpy())
    got_w = _host_rows(dup_w)
    for r in range(wl.R):
        for b in range(wl.B):
            if b < int(p["n_dup"][r]):
                assert np.array_equal(got_w[r, b].view(np.uint8), want_w[r, b].view(np.uint8))
            else:
                assert not np.any(got_w[r, b].view(np.uint8)), "an unused slot was written"
    want_h = oracle.reduce_dup_grads(p, wl.B, dg.numpy(), hg.numpy())
    assert np.array_equal(f32_bits(hg_d), want_h.view(np.uint32)), "reduce"
    return g


PLANS = pytest.mark.parametrize("bounded", [False, True], ids=["waterfill", "bounded"])


@PLANS
@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_small_shapes_elementwise(td, wl, bounded):
    ids, w = W.make_routing(wl, seed=3)
    _full_case(td, wl, ids.reshape(-1), w.reshape(-1), 3, bounded)


def test_hand_worked_examples_on_gpu(td):
    import glob
    import json
    import os
    for path in sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden",
                                              "plan_example*.json"))):
        ex = json.load(open(path))
        dims = td.Dims(ex["R"], ex["E"], ex["K"], ex["S"], ex["B"], W.F32, 4)
        say(f"golden {os.path.basename(path)}")
        ids = np.array(ex["ids"], np.int32)
        for form in ("two", "four"):
            plan_buf, _ = run_plan(td, dims, ids, DEV, form=form)
            g = read_plan(td, dims, plan_buf)
            SK = ex["S"] * ex["K"]
            x = ex["expect"]
            assert [[d // SK, d % SK] for d in g["dst"].tolist()] == x["dst_rank_slot"]
            assert g["n_dup"].tolist() == x["n_dup"] and int(g["status"][0]) == x["status"]
            assert float(g["maxvio"][0]) == x["maxvio"]
            assert_plan_equal(g, oracle.plan(ex["R"], ex["E"], ex["K"], ex["S"], ex["B"], ids))


def test_bounded_hand_worked_examples_on_gpu(td):
    import glob
    import json
    import os
    paths = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden",
                                          "bounded_example*.json")))
    assert paths
    for path in paths:
        ex = json.load(open(path))
        R, E, K, S, B = ex["R"], ex["E"], ex["K"], ex["S"], ex["B"]
        dims = td.Dims(R, E, K, S, B, W.F32, 4)
        say(f"golden {os.path.basename(path)}")
        ids = np.array(ex["ids"], np.int32)
        for form in ("two", "four"):
            plan_buf, _ = run_plan(td, dims, ids, DEV, bounded=True, form=form)
            _check_bounded_golden(td, dims, ex, ids, plan_buf)


def _check_bounded_golden(td, dims, ex, ids, plan_buf):
    R, E, K, S, B = ex["R"], ex["E"], ex["K"], ex["S"], ex["B"]
    g = read_plan(td, dims, plan_buf)
    SK, G = S * K, E // R
    x = ex["expect"]
    assert [[d // SK, d % SK] for d in g["dst"].tolist()] == x["dst_rank_slot"]
    assert g["n_dup"].tolist() == x["n_dup"] and int(g["status"][0]) == x["status"]
    assert float(g["maxvio"][0]) == x["maxvio"]
    got_dups = [[r, b, int(g["dup_expert"][r, b]), int(g["dup_start"][r, b]),
                 int(g["dup_count"][r, b])] for r in range(R) for b in range(int(g["n_dup"][r]))]
    assert got_dups == x["dups"]
    nl = int(g["n_list"][0])
    assert [[int(g["list_expert"][i]), int(g["list_rank"][i]), int(g["list_b"][i])]
            for i in range(nl)] == x["list"]
    for r in range(R):
        ns = G + int(g["n_dup"][r])
        assert g["seg_ptr"][r, :ns + 1].tolist() == x["seg_ptr"][r]
    assert_plan_equal(g, oracle.plan(R, E, K, S, B, ids, bounded=True))


@PLANS
def test_invalid_and_repeated_ids(td, bounded):
    wl = _wl("bad_ids", 4, 32, 4, 1500, 4, 64, W.BF16, 2.0)
    rng = np.random.default_rng(17)
    ids, w = W.make_routing(wl, seed=5)
    ids = ids.reshape(-1).copy()
    w = w.reshape(-1)
    bad = rng.choice(ids.size, 40, replace=False)
    ids[bad] = rng.choice([-1, -100, wl.E, wl.E + 7], 40)
    g = _full_case(td, wl, ids, w, 5, bounded)
    assert int(g["status"][0]) & 1
    ids2, w2 = W.make_routing(wl, seed=6)
    ids2 = ids2.reshape(-1, wl.K).copy()
    t = rng.choice(wl.n_tok, 25, replace=False)
    ids2[t, 2] = ids2[t, 0]
    g = _full_case(td, wl, ids2.reshape(-1), w2.reshape(-1), 6, bounded)
    assert int(g["status"][0]) & 2


@PLANS
def test_every_id_dropped(td, bounded):
    """The degenerate step with no valid assignment: every id out of range. The
    plan has T = 0, no overflow and no duplicates, every slot stays empty, combine
    gives +0 everywhere, and replicate and reduce touch nothing."""
    wl = _wl("all_dropped", 4, 32, 4, 600, 4, 64, W.BF16, 2.0)
    _, w = W.make_routing(wl, seed=9)
    for fill in (-1, wl.E):
        ids = np.full(wl.n_ent, fill, dtype=np.int32)
        g = _full_case(td, wl, ids, w.reshape(-1), 9, bounded)
        assert int(g["status"][0]) & 1
        assert not np.any(g["T"]) and not np.any(g["n_dup"])
        assert np.all(g["dst"] == -1) and np.all(g["src"] == -1)


@PLANS
def test_repeated_ids_several_tokens_per_thread(td, bounded):
    # K = 2 and 512 tokens per 1024-entry tile: counting thread t takes tokens
    # t and t + 256 of its tile in turn, so its per-token seen set must be
    # cleared between them. Token t + 256 names the ids of token t, swapped (no
    # repeat); then a few tokens repeat one id, first and second tokens alike.
    wl = _wl("rep_k2", 2, 16, 2, 2000, 2, 32, W.BF16, 1.0)
    dims = _dims(td, wl)
    assert td.moonep_plan_layout(dims).tile_tokens == 512
    ids, w = W.make_routing(wl, seed=3)
    ids = ids.reshape(-1, wl.K).copy()
    for t0 in range(0, wl.n_tok, 512):
        n2 = max(0, min(256, wl.n_tok - t0 - 256))
        ids[t0 + 256:t0 + 256 + n2] = ids[t0:t0 + n2][:, ::-1]
    g = _full_case(td, wl, ids.reshape(-1), w.reshape(-1), 3, bounded)
    assert (int(g["status"][0]) & 2) == 0
    ids[[5, 300, 512 + 40, 3000], 1] = ids[[5, 300, 512 + 40, 3000], 0]
    g = _full_case(td, wl, ids.reshape(-1), w.reshape(-1), 3, bounded)
    assert int(g["status"][0]) & 2


@PLANS
def test_extreme_skew_and_balance(td, bounded):
    # every token picks the same K experts, all homed on rank 0
    wl = _wl("one_hot_rank", 8, 64, 8, 1000, 8, 64, W.BF16, 0.0)
    ids = np.tile(np.arange(8, dtype=np.int32), wl.n_tok)
    w = np.full(ids.size, 1.0 / 8, np.float32)
    g = _full_case(td, wl, ids, w, 1, bounded)
    assert int(g["n_dup"].sum()) > 0 and int(g["L"][0]) == wl.n_ent
    # perfectly balanced routing: no overflow, no duplicates
    wl = _wl("balanced", 4, 16, 4, 256, 2, 64, W.BF16, 0.0)
    ids = (np.arange(wl.n_ent) % wl.E).astype(np.int32)
    w = np.full(ids.size, 0.25, np.float32)
    g = _full_case(td, wl, ids, w, 2, bounded)
    assert int(g["n_dup"].sum()) == 0 and float(g["maxvio"][0]) == 0.0


@PLANS
def test_overflows_past_512(td, bounded):
    # one expert per rank; 700 experts get S*K + 1 entries and the other 324
    # make up the total: 700 one-row overflows (16 registers per lane in the
    # bounded placement) onto 324 ranks short by 2 or 3 rows
    wl = _wl("over_700", 1024, 1024, 2, 4, 4, 64, W.BF16, 0.0)
    counts = np.concatenate([np.full(700, wl.SK + 1), np.full(272, wl.SK - 2),
                             np.full(52, wl.SK - 3)]).astype(np.int64)
    assert counts.sum() == wl.n_ent
    flat = np.repeat(np.arange(wl.E, dtype=np.int32), counts)
    # token t takes entries t and t + n_tok of the sorted list: two distinct experts
    ids = np.stack([flat[:wl.n_tok], flat[wl.n_tok:]], axis=1)
    ids = ids[np.random.default_rng(5).permutation(wl.n_tok)].reshape(-1)
    w = np.full(ids.size, 0.5, np.float32)
    g = _full_case(td, wl, ids, w, 4, bounded)
    assert int((g["O"] > 0).sum()) == 700 and int(g["n_list"][0]) >= 700


def _ids_from_counts(T, n_tok, K, seed):
    """Router ids with exactly T[e] entries of expert e and K distinct experts per
    token: the sorted id list is cut into K columns of n_tok (no expert has more
    than n_tok entries, so a token's K ids come from K different runs)."""
    T = np.asarray(T, dtype=np.int64)
    flat = np.repeat(np.arange(T.size, dtype=np.int32), T)
    assert flat.size == n_tok * K and int(T.max()) <= n_tok
    ids = flat.reshape(K, n_tok).T.copy()
    return ids[np.random.default_rng(seed).permutation(n_tok)].reshape(-1)


def _balanced_counts(R, G, SK, over, short, seed):
    """Expert counts for R ranks of G experts: ranks in `over` get extra rows (one
    list of per-expert extras each), ranks in `short` fewer rows; the rest exactly
    S*K. Overflows and deficits are placed on random ranks."""
    T = np.full((R, G), SK // G, dtype=np.int64)
    T[:, : SK % G] += 1
    idx = np.random.default_rng(seed).permutation(R)
    for r, extra in zip(idx[: len(over)], over):
        T[r, : len(extra)] += np.asarray(extra)
    for r, d in zip(idx[len(over): len(over) + len(short)], short):
        left = d
        for g in range(G):
            take = min(left, int(T[r, g]))
            T[r, g] -= take
            left -= take
        assert left == 0
    T = T.reshape(-1)
    assert T.sum() == R * SK
    return T


def _deficits(total, hi, seed):
    rng = np.random.default_rng(seed)
    d = []
    while sum(d) < total:
        d.append(min(1 + int(rng.integers(0, hi)), total - sum(d)))
    return d


# Routings built from per-expert counts for the edges of the bounded placement:
# exactly 64 overflows (every lane of the sorted wave live) and 65 (the register-
# slot search), ties in rows, B = 1 (no fit-whole pieces), overflows cut over many
# deficit ranks, deficits of more than 2^21 rows with every overflow below it,
# more than 64 deficit ranks, and B = 2, 63 and 64.
def _edge_cases():
    def rows(over):
        return sum(sum(x) for x in over)
    out = []
    ov = [[1 + (i % 8)] for i in range(64)]
    out.append(("ov64_unit", 128, 1, 2, 4, 2, [[1]] * 64, [1] * 64))
    out.append(("ov64_ties", 256, 1, 4, 16, 3, ov, _deficits(rows(ov), 12, 1)))
    ov65 = ov + [[5]]
    out.append(("ov65_ties", 256, 1, 4, 16, 3, ov65, _deficits(rows(ov65), 12, 2)))
    out.append(("ov63_fill_only", 256, 1, 4, 16, 1, ov[:63], _deficits(rows(ov[:63]), 9, 3)))
    big = [[300], [280], [280], [150]]
    out.append(("cut_heavy", 256, 1, 4, 64, 4, big, _deficits(rows(big), 9, 4)))
    mixed = [[500]] + [[10]] * 40 + [[1]] * 20
    out.append(("one_big", 256, 1, 4, 64, 2, mixed, _deficits(rows(mixed), 16, 5)))
    SK = (1 << 21) + (1 << 20)
    q = SK // 4
    out.append(("room_past_2p21", 2, 4, 1, SK, 2, [[q - 1000, q, q, q - 1000]], [SK - 2000]))
    # more than 64 deficit ranks with at most 64 overflows: the sorted placement
    # reloads the deficits every 64 ranks and flushes its piece records many times
    few = [[10 + 3 * (i % 5)] for i in range(24)]
    out.append(("ranks_past_64_b4", 256, 1, 2, 64, 4, few, _deficits(rows(few), 5, 6)))
    out.append(("ranks_past_64_b2", 256, 1, 2, 64, 2, few, _deficits(rows(few), 5, 7)))
    # B = 63, the largest the sorted placement takes (a flush before almost every
    # rank), and B = 64, which takes the register-slot search
    many = [[1 + (i % 5)] for i in range(60)]
    out.append(("b63", 256, 1, 4, 16, 63, many, _deficits(rows(many), 40, 8)))
    out.append(("b64", 256, 1, 4, 16, 64, many, _deficits(rows(many), 40, 8)))
    return out


@PLANS
@pytest.mark.parametrize("case", _edge_cases(), ids=lambda c: c[0])
def test_bounded_placement_edges(td, case, bounded):
    name, R, G, K, S, B, over, short = case
    wl = _wl(name, R, R * G, K, S, B, 8, W.BF16, 0.0)
    T = _balanced_counts(R, G, S * K, over, short, 7)
    ids = _ids_from_counts(T, R * S, K, 8)
    w = np.full(ids.size, 1.0 / K, np.float32)
    g = _full_case(td, wl, ids, w, 5, bounded)
    n_over = len(over) if G == 1 else int((g["O"] > 0).sum())
    assert int((g["O"] > 0).sum()) == n_over


def _random_shapes(n, seed):
    """Seeded random shapes of up to about 60 000 entries: 1 to 512 ranks of 1 to 8
    experts, K from 1 to 16, B from 0 to 200, router skew from none to strong, bf16
    and fp32 rows of one 16-byte chunk. They reach both launch forms, both
    placement paths of the bounded plan (up to 64 overflowing experts and more),
    ranks that take several duplicates, and B of 0, 1 and past every rank's need."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        R = int(rng.choice([1, 2, 3, 5, 8, 16, 24, 32, 64, 96, 128, 256, 512]))
        G = int(rng.integers(1, max(2, min(8, 1024 // R) + 1)))
        K = int(rng.integers(1, min(R * G, 16) + 1))
        S = int(rng.integers(1, max(1, 60000 // (R * K)) + 1))
        B = int(rng.choice([0, 1, 2, 3, 4, 6, 8, 16, 31, 63, 64, 200]))
        skew = float(rng.choice([0.0, 0.5, 1.0, 2.0, 3.0, 5.0]))
        dt = W.BF16 if rng.random() < 0.5 else W.F32
        out.append(_wl(f"rand{i}", R, R * G, K, S, B, 8 if dt == W.BF16 else 4, dt, skew))
    return out


RANDOM = _random_shapes(64, 11)


@PLANS
@pytest.mark.parametrize("wl", RANDOM, ids=[w.name for w in RANDOM])
def test_random_shapes(td, wl, bounded):
    """Every plan array, dispatch, combine, replicate and reduce against the oracle,
    and the plan invariants, on seeded random shapes and routings."""
    ids, w = W.make_routing(wl, 100 + int(wl.name[4:]))
    _full_case(td, wl, ids.reshape(-1), w.reshape(-1), 6, bounded)


def _random_rows(n, seed):
    """Seeded random row widths for the moves: any multiple of 16 bytes from 16 B
    to 40 KiB in bf16 and fp32 (every chunks-per-lane width, ragged lanes, rows of
    several segments), K from 1 to 64, about 2 to 60 MiB of rows, and weight
    blocks of random 16-byte multiples."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt = W.BF16 if rng.random() < 0.5 else W.F32
        chunks = int(rng.choice([int(rng.integers(1, 65)), int(rng.integers(65, 2561))]))
        H = chunks * (8 if dt == W.BF16 else 4)
        R = int(rng.choice([1, 2, 3, 4, 8, 16]))
        G = int(rng.integers(1, 9))
        K = int(rng.integers(1, min(R * G, 64) + 1))
        S = max(1, int(rng.integers(1 << 21, 60 << 20)) // (R * K * chunks * 16))
        B = int(rng.choice([0, 1, 2, 4, 8]))
        blk = (int(rng.integers(1, 9)), 8 * int(rng.integers(1, 33)))
        out.append(_wl(f"rows{i}", R, R * G, K, S, B, H, dt, float(rng.choice([0.0, 1.0, 3.0])),
                       block=blk))
    return out


RANDOM_ROWS = _random_rows(24, 12)


@pytest.mark.parametrize("wl", RANDOM_ROWS, ids=[w.name for w in RANDOM_ROWS])
def test_random_row_widths(td, wl):
    """The moves at seeded random row widths, K and weight blocks, element by
    element against the oracle (odd cases take the bounded plan)."""
    i = int(wl.name[4:])
    ids, w = W.make_routing(wl, 200 + i)
    _full_case(td, wl, ids.reshape(-1), w.reshape(-1), 7, bool(i & 1))


def test_identity_expert_mean_returns_hidden(td):
    """y = recv and w = 1/K with K a power of two: combine gives back hidden bit for bit."""
    wl = _wl("identity", 8, 64, 8, 900, 8, 512, W.BF16, 2.0)
    dims = _dims(td, wl)
    ids, _ = W.make_routing(wl, seed=2)
    plan_buf, _ = run_plan(td, dims, ids, DEV)
    hid = W.make_hidden(wl, 2).to(DEV)
    recv = torch.empty((wl.R, wl.SK, wl.H), dtype=hid.dtype, device=DEV)
    out = torch.empty_like(hid)
    w = torch.full((wl.R, wl.S, wl.K), 1.0 / wl.K, dtype=torch.float32, device=DEV)
    td.moonep_dispatch(dims, plan_buf, hid, recv)
    td.moonep_combine(dims, plan_buf, recv, w, out)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), hid.view(torch.int16))


def test_launch_count(td):
    """The per-call launch count of the chunked moves: one launch for a small
    problem, several at the K3 shape, and counting enqueues nothing."""
    for name, several in (("tiny", False), ("k3", True)):
        wl = W.WORKLOADS[name]
        dims = _dims(td, wl)
        for op in (td.OP_DISPATCH, td.OP_COMBINE):
            n = td.moonep_launch_count(dims, op)
            assert 1 <= n <= wl.n_tok
            assert (n > 1) == several, (name, op, n)
    torch.cuda.synchronize()


def test_deterministic_and_stream_ordered(td):
    wl = W.WORKLOADS["zipf"].replace(S=512)
    dims = _dims(td, wl)
    ids, _ = W.make_routing(wl, seed=1)
    s = torch.cuda.Stream(DEV)
    bufs = []
    for _ in range(3):
        pb = td.new_plan_buffer(dims, DEV)
        with torch.cuda.stream(s):
            ids_d = torch.from_numpy(ids).to(DEV, non_blocking=False)
            td.moonep_plan(dims, ids_d, pb, stream=s)
        bufs.append(pb)
    torch.cuda.synchronize()
    a = read_plan(td, dims, bufs[0])
    assert_plan_equal(a, oracle.plan(wl.R, wl.E, wl.K, wl.S, wl.B, ids))
    for pb in bufs[1:]:
        assert_plan_equal(read_plan(td, dims, pb), a)


def test_two_streams_at_once(td):
    """The library keeps no state between calls: two independent steps (plan,
    dispatch, combine) enqueued on two streams and running concurrently, with
    different shapes and routings, each match the oracle."""
    cases = [_wl("stream_a", 8, 64, 8, 1500, 8, 256, W.BF16, 2.0),
             _wl("stream_b", 4, 32, 4, 2500, 4, 128, W.F32, 1.5)]
    streams = [torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)]
    runs = []
    for wl, s, seed in zip(cases, streams, (11, 12)):
        dims = _dims(td, wl)
        ids, w = W.make_routing(wl, seed)
        hidden = W.make_hidden(wl, seed)
        with torch.cuda.stream(s):
            ids_d = torch.from_numpy(ids).to(DEV)
            w_d = torch.from_numpy(w).to(DEV)
            hid_d = hidden.to(DEV)
            pb = td.new_plan_buffer(dims, DEV)
            recv = torch.empty((wl.R, wl.SK, wl.H), dtype=hid_d.dtype, device=DEV)
            out = torch.empty_like(hid_d)
        runs.append((wl, dims, ids, w, hidden, ids_d, w_d, hid_d, pb, recv, out, s))
    torch.cuda.synchronize()
    for _ in range(3):  # interleaved enqueues on both streams
        for wl, dims, ids, w, hidden, ids_d, w_d, hid_d, pb, recv, out, s in runs:
            td.moonep_plan(dims, ids_d, pb, stream=s)
        for wl, dims, ids, w, hidden, ids_d, w_d, hid_d, pb, recv, out, s in runs:
            td.moonep_dispatch(dims, pb, hid_d, recv, stream=s)
            td.moonep_combine(dims, pb, recv, w_d, out, stream=s)
    torch.cuda.synchronize()
    for wl, dims, ids, w, hidden, ids_d, w_d, hid_d, pb, recv, out, s in runs:
        p = oracle.plan(wl.R, wl.E, wl.K, wl.S, wl.B, ids)
        assert_plan_equal(read_plan(td, dims, pb), p)
        hid_h = _host_rows(hidden).reshape(wl.n_tok, wl.H)
        want_recv = oracle.dispatch(p, wl.K, hid_h)
        assert np.array_equal(_host_rows(recv).reshape(-1, wl.H).view(np.uint8),
                              want_recv.view(np.uint8)), wl.name
        want_out = oracle.combine(p["dst"], wl.K, want_recv, w, wl.dtype, wl.dtype)
        assert np.array_equal(_host_rows(out).reshape(-1, wl.H).view(np.uint8),
                              want_out.view(np.uint8)), wl.name


def test_plan_buffer_reuse_across_shapes(td):
    """A plan buffer first used for a larger problem gives the same plan for a
    smaller one (no stale state leaks into the result)."""
    big = _wl("big", 8, 64, 8, 2000, 8, 64, W.BF16, 2.5)
    small = _wl("small", 4, 32, 4, 700, 2, 64, W.BF16, 1.0)
    dims_b, dims_s = _dims(td, big), _dims(td, small)
    pb = td.new_plan_buffer(dims_b, DEV)
    ids_b, _ = W.make_routing(big, seed=4)
    ids_s, _ = W.make_routing(small, seed=4)
    lay = td.moonep_plan_layout(dims_s)
    run_plan(td, dims_b, ids_b, DEV, pb)
    run_plan(td, dims_s, ids_s, DEV, pb[:lay.bytes])
    g = read_plan(td, dims_s, pb[:lay.bytes])
    assert_plan_equal(g, oracle.plan(small.R, small.E, small.K, small.S, small.B, ids_s))


@PLANS
def test_plan_from_arbitrary_buffer_contents(td, bounded):
    """The plan buffer needs no initialisation: any starting contents give the
    same plan, and so do the values each call leaves for the next."""
    wl = _wl("sync", 8, 64, 8, 1500, 8, 64, W.BF16, 2.0)
    dims = _dims(td, wl)
    lay = td.moonep_plan_layout(dims)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(7)
    for fill in ("as allocated", "ones", "random"):
        pb = td.new_plan_buffer(dims, DEV)
        if fill == "ones":
            pb.fill_(255)
        elif fill == "random":
            pb.copy_(torch.randint(0, 256, (lay.bytes,), generator=gen, device=DEV,
                                   dtype=torch.int32).to(torch.uint8))
        for seed in (0, 1, 2):
            ids, _ = W.make_routing(wl, seed)
            run_plan(td, dims, ids, DEV, pb, bounded=bounded)
            assert_plan_equal(read_plan(td, dims, pb),
                              oracle.plan(wl.R, wl.E, wl.K, wl.S, wl.B, ids, bounded=bounded))


@PLANS
def test_plan_graph_replays(td, bounded):
    """The plan captured in a HIP graph and replayed on new ids: every replay
    gives the oracle's plan for the ids it sees."""
    wl = _wl("graph", 8, 64, 8, 1000, 8, 64, W.BF16, 2.0)
    dims = _dims(td, wl)
    pb = td.new_plan_buffer(dims, DEV)
    ids0, _ = W.make_routing(wl, 0)
    ids_d = torch.from_numpy(ids0).to(DEV)
    s = torch.cuda.Stream(DEV)
    plan_fn = td.moonep_plan_bounded if bounded else td.moonep_plan
    with torch.cuda.stream(s):
        plan_fn(dims, ids_d, pb, stream=s)  # sets kernel attributes before capture
    s.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        plan_fn(dims, ids_d, pb, stream=s)
    for seed in (1, 2, 3, 1):
        ids, _ = W.make_routing(wl, seed)
        ids_d.copy_(torch.from_numpy(ids).to(DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert_plan_equal(read_plan(td, dims, pb),
                          oracle.plan(wl.R, wl.E, wl.K, wl.S, wl.B, ids, bounded=bounded))


@PLANS
def test_whole_step_graph_replays(td, bounded):
    """Plan, replicate, dispatch, combine and reduce captured in one HIP graph
    and replayed on new router ids and weights: every replay's outputs equal the
    oracle's for the inputs it sees. Eager work (input copies, a reset of the
    home gradients) runs between the replays."""
    wl = _wl("graph_step", 8, 64, 8, 1000, 8, 64, W.BF16, 2.0)
    dims = _dims(td, wl)
    pb = td.new_plan_buffer(dims, DEV)
    ids0, w0 = W.make_routing(wl, 0)
    ids_d = torch.from_numpy(ids0).to(DEV)
    w_d = torch.from_numpy(w0).to(DEV)
    hidden = W.make_hidden(wl, 5)
    hid_d = hidden.to(DEV)
    recv = torch.empty((wl.R, wl.SK, wl.H), dtype=hid_d.dtype, device=DEV)
    out = torch.empty_like(hid_d)
    ew = W.make_expert_weights(wl, 5)
    ew_d = ew.to(DEV)
    dup_w = torch.zeros((wl.R, wl.B) + tuple(wl.block_shape), dtype=ew.dtype, device=DEV)
    dg, hg = W.make_grads(wl, 5)
    dg_d, hg_d = dg.to(DEV), hg.to(DEV)
    plan_fn = td.moonep_plan_bounded if bounded else td.moonep_plan
    s = torch.cuda.Stream(DEV)

    def step():
        plan_fn(dims, ids_d, pb, stream=s)
        td.moonep_replicate(dims, pb, ew_d, dup_w, wl.block_bytes, stream=s)
        td.moonep_dispatch(dims, pb, hid_d, recv, stream=s)
        td.moonep_combine(dims, pb, recv, w_d, out, stream=s)
        td.moonep_reduce_dup_grads(dims, pb, dg_d, hg_d, wl.block_elems, stream=s)

    with torch.cuda.stream(s):
        step()  # sets kernel attributes before capture
    s.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step()
    hid_h = _host_rows(hidden).reshape(wl.n_tok, wl.H)
    ew_h = bf16_bits(ew)
    for seed in (1, 2, 3, 1):
        say(f"graph replay bounded={bounded} seed={seed}")
        ids, w = W.make_routing(wl, seed)
        ids_d.copy_(torch.from_numpy(ids).to(DEV))
        w_d.copy_(torch.from_numpy(w).to(DEV))
        hg_d.copy_(hg.to(DEV))
        dup_w.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        p = oracle.plan(wl.R, wl.E, wl.K, wl.S, wl.B, ids, bounded=bounded)
        assert_plan_equal(read_plan(td, dims, pb), p)
        want_recv = oracle.dispatch(p, wl.K, hid_h)
        assert np.array_equal(_host_rows(recv).reshape(-1, wl.H).view(np.uint16),
                              want_recv.view(np.uint16)), "dispatch"
        want_out = oracle.combine(p["dst"], wl.K, want_recv, w, wl.dtype, wl.dtype)
        assert np.array_equal(_host_rows(out).reshape(-1, wl.H).view(np.uint16),
                              want_out.view(np.uint16)), "combine"
        want_w = oracle.replicate(p, wl.B, ew_h)
        assert np.array_equal(_host_rows(dup_w).view(np.uint16), want_w.view(np.uint16)), "replicate"
        want_h = oracle.reduce_dup_grads(p, wl.B, dg.numpy(), hg.numpy())
        assert np.array_equal(f32_bits(hg_d), want_h.view(np.uint32)), "reduce"


def test_rows_past_the_buffer_range(td):
    """Rows of 2 GiB (H = 2^30 bf16): combine and the backward of dispatch read
    them with global loads instead of through a buffer resource, whose 32-bit
    range they exceed. Two tokens, one expert each, both paths checked against
    the oracle on every element."""
    R, E, K, S, B, H = 1, 2, 1, 2, 1, 1 << 30
    dims = td.Dims(R, E, K, S, B, W.BF16, H)
    say(f"2 GiB rows: {dims}")
    ids = np.array([1, 0], dtype=np.int32)
    plan_buf, _ = run_plan(td, dims, ids, DEV)
    p = oracle.plan(R, E, K, S, B, ids)
    assert_plan_equal(read_plan(td, dims, plan_buf), p)
    hidden = W.dense((R, S, H), W.BF16, 1.0, 3, "hidden", DEV)
    recv = torch.empty((R, S * K, H), dtype=torch.bfloat16, device=DEV)
    td.moonep_dispatch(dims, plan_buf, hidden, recv)
    w = np.array([0.75, -1.25], dtype=np.float32)
    out = torch.empty_like(hidden)
    td.moonep_combine(dims, plan_buf, recv, torch.from_numpy(w).to(DEV), out)
    back = torch.empty_like(hidden)
    td.moonep_dispatch_backward(dims, plan_buf, recv, back, W.BF16)
    torch.cuda.synchronize()
    say("  kernels done")
    hid_h = bf16_bits(hidden).reshape(S, H)
    del hidden
    want_recv = oracle.dispatch(p, K, hid_h)
    assert np.array_equal(bf16_bits(recv).reshape(S, H), want_recv), "dispatch"
    want_out = oracle.combine(p["dst"], K, want_recv, w, W.BF16, W.BF16)
    assert np.array_equal(bf16_bits(out).reshape(S, H), want_out), "combine"
    del out
    want_back = oracle.dispatch_backward(p["dst"], K, want_recv, W.BF16, W.BF16)
    assert np.array_equal(bf16_bits(back).reshape(S, H), want_back), "dispatch backward"


def _plans_equal_int32(td, dims, plan_buf, p):
    """assert_plan_equal without 64-bit copies: the entry-sized arrays at the
    largest shapes are compared as they are (int32)."""
    v = td.plan_views(dims, plan_buf)
    for k in PLAN_INT_KEYS:
        g = v[k].cpu().numpy().reshape(-1)
        o = np.asarray(p[k]).reshape(-1)
        assert g.shape == o.shape and np.array_equal(g, o.astype(np.int32, copy=False)), k
        del g
    assert int(v["maxT"][0]) == int(p["maxT"][0])
    assert v["maxvio"].cpu().numpy().view(np.uint64)[0] == p["maxvio"].view(np.uint64)[0]


def test_entries_near_int32_limit(td):
    """The largest entry count the library takes: R*S*K = 2 147 483 520, just
    below 2^31 (16 ranks, 64 experts, K = 8, 16 777 215 tokens per rank, 16-byte
    rows). Both plans are compared with the oracle array by array; dispatch on
    every slot against the oracle's inverse map; combine with identity experts and
    weights 1/K, whose exact result is the token's own row, on every token."""
    R, E, K, B, H = 16, 64, 8, 4, 8
    S = ((1 << 31) - 1) // (R * K)
    n_ent, n_tok = R * S * K, R * S
    dims = td.Dims(R, E, K, S, B, W.BF16, H)
    say(f"near-limit case: {dims}, {n_ent} entries")
    ids = W.make_consecutive_ids(R, E, K, S, seed=0)
    say("ids drawn")
    plan_buf, ids_d = run_plan(td, dims, ids, DEV)
    say("water-fill plan on the GPU done")
    p = oracle.plan(R, E, K, S, B, ids)
    say("oracle water-fill done")
    _plans_equal_int32(td, dims, plan_buf, p)
    say(f"water-fill plans equal; duplicates per rank {p['n_dup'].tolist()}")

    hidden = W.dense((R, S, H), W.BF16, 1.0, 0, "hidden", DEV)
    recv = torch.empty((R, S * K, H), dtype=torch.bfloat16, device=DEV)
    td.moonep_dispatch(dims, plan_buf, hidden, recv)
    w_d = torch.full((R, S, K), 1.0 / K, dtype=torch.float32, device=DEV)
    out = torch.empty_like(hidden)
    td.moonep_combine(dims, plan_buf, recv, w_d, out)
    torch.cuda.synchronize()
    say("dispatch and combine done")
    # dispatch: every slot against the oracle's inverse map, 2^24 slots at a time
    # (torch's own kernels refuse a launch over 2^30 elements)
    step = 1 << 24
    hflat, rflat = hidden.view(-1, H), recv.view(-1, H)
    for lo in range(0, n_ent, step):
        hi = min(n_ent, lo + step)
        tok = torch.from_numpy(p["src"][lo:hi].astype(np.int64) // K).to(DEV)
        assert torch.equal(rflat[lo:hi].view(torch.int16), hflat[tok].view(torch.int16)), \
            f"dispatch slots [{lo}, {hi})"
        del tok
    # combine: identity experts and weights 1/K give every token its own row back
    oflat = out.view(-1, H)
    for lo in range(0, n_tok, step):
        assert torch.equal(oflat[lo:lo + step].view(torch.int16),
                           hflat[lo:lo + step].view(torch.int16)), f"combine tokens from {lo}"
    say("every slot and every token equal")
    del recv, out, w_d, hidden

    td.moonep_plan_bounded(dims, ids_d, plan_buf)
    torch.cuda.synchronize()
    say("bounded plan on the GPU done")
    del p
    pb = oracle.plan(R, E, K, S, B, ids, bounded=True)
    say("oracle bounded plan done")
    _plans_equal_int32(td, dims, plan_buf, pb)
    say(f"bounded plans equal; duplicates per rank {pb['n_dup'].tolist()}")


# ------------------------------------------------------------ full-size shapes

@PLANS
@pytest.mark.parametrize("name", ["tiny", "uniform", "zipf", "k3", "decode"])
def test_workload_plans_all_seeds(td, name, bounded):
    wl = W.WORKLOADS[name]
    dims = _dims(td, wl)
    pb = td.new_plan_buffer(dims, DEV)
    for seed in (0, 1, 2):
        say(f"plan {name} seed {seed} bounded={bounded}")
        ids, _ = W.make_routing(wl, seed)
        p = oracle.plan(wl.R, wl.E, wl.K, wl.S, wl.B, ids, bounded=bounded)
        for form in ("two", "four"):
            run_plan(td, dims, ids, DEV, pb, bounded=bounded, form=form)
            assert_plan_equal(read_plan(td, dims, pb), p)
        run_plan(td, dims, ids, DEV, pb, bounded=bounded)
        g = read_plan(td, dims, pb)
        assert_plan_equal(g, p)
        if seed == 0:
            check_plan(wl.R, wl.E, wl.K, wl.S, wl.B, ids, g)
        # every rank holds exactly S*K rows
        assert np.all(g["seg_ptr"][np.arange(wl.R), wl.G + g["n_dup"]] == wl.SK)
        say(f"  maxvio {float(g['maxvio'][0]):.3f}  dups/rank max {int(g['n_dup'].max())} "
            f"(B={wl.B})  total dups {int(g['n_dup'].sum())}  status {int(g['status'][0])}")


FULL_MOVES = [("uniform", False), ("zipf", False), ("k3", False), ("decode", False),
              ("k3", True), ("decode", True)]


def _row_hash(t, rows_per_chunk=8):
    """One int64 per row of a float32 [n, m] tensor: the sum of its bit patterns
    (any write that changes a row changes it with overwhelming probability),
    taken a few rows at a time to bound the temporary."""
    out = torch.empty(t.shape[0], dtype=torch.int64, device=t.device)
    for i in range(0, t.shape[0], rows_per_chunk):
        out[i:i + rows_per_chunk] = t[i:i + rows_per_chunk].view(torch.int32).to(torch.int64).sum(1)
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("name,bounded", FULL_MOVES, ids=[f"{n}-{'bounded' if b else 'waterfill'}"
                                                          for n, b in FULL_MOVES])
def test_workload_data_moves_full_size(td, name, bounded, seed):
    """Every output element of dispatch, combine, replicate and reduce at the
    workload's full size, in the launch configuration the benchmark times, against
    the oracle: dispatch and replicate through the oracle's plan tables, combine
    through the oracle's fma sequence on every token (batches of gathered rows),
    reduce through the oracle on every expert with duplicates, and the experts
    without any checked untouched."""
    wl = W.WORKLOADS[name]
    dims = _dims(td, wl)
    say(f"full-size moves {name} bounded={bounded} seed={seed}: {dims}")
    ids, w = W.make_routing(wl, seed)
    p = oracle.plan(wl.R, wl.E, wl.K, wl.S, wl.B, ids, bounded=bounded)
    pb, _ = run_plan(td, dims, ids, DEV, bounded=bounded)
    assert_plan_equal(read_plan(td, dims, pb), p)
    src_d = torch.from_numpy(p["src"].astype(np.int64)).to(DEV)
    rng = np.random.default_rng(99 + seed)

    # dispatch: every slot against the oracle's inverse map, windows through the oracle
    hid = W.make_hidden(wl, seed, DEV)
    recv = torch.empty((wl.R, wl.SK, wl.H), dtype=hid.dtype, device=DEV)
    say("  dispatch")
    td.moonep_dispatch(dims, pb, hid, recv)
    torch.cuda.synchronize()
    hflat, rflat = hid.view(wl.n_tok, wl.H), recv.view(-1, wl.H)
    assert bool((src_d >= 0).all())
    for r in range(wl.R):
        sl = slice(r * wl.SK, (r + 1) * wl.SK)
        assert torch.equal(rflat[sl].view(torch.int16),
                           hflat[src_d[sl] // wl.K].view(torch.int16)), f"dispatch rank {r}"
    hid_h = bf16_bits(hid).reshape(wl.n_tok, wl.H)
    for lo in list(rng.integers(0, wl.n_ent - 64, 6)) + [0, wl.n_ent - 64]:
        want = oracle.dispatch(p, wl.K, hid_h, int(lo), int(lo) + 64)
        assert np.array_equal(bf16_bits(rflat[int(lo):int(lo) + 64]), want)
    del hid_h, hflat, hid

    # combine: y = seeded expert outputs; every token through the oracle
    say("  combine")
    y = recv
    g = torch.Generator(device=DEV)
    g.manual_seed(1234 + seed)
    for r in range(wl.R):
        y[r].copy_(torch.randn((wl.SK, wl.H), generator=g, device=DEV, dtype=torch.float32))
    w_d = torch.from_numpy(w).to(DEV)
    out = torch.empty((wl.R, wl.S, wl.H), dtype=torch.bfloat16, device=DEV)
    td.moonep_combine(dims, pb, y, w_d, out)
    torch.cuda.synchronize()
    dst_tok = p["dst"].reshape(wl.n_tok, wl.K)
    dst_d = torch.from_numpy(np.maximum(p["dst"], 0).astype(np.int64)).to(DEV)
    wf = w.reshape(-1)
    yflat, oflat = y.view(-1, wl.H), out.view(wl.n_tok, wl.H)
    budget = 1 << 30
    stage_y = HostStage(budget)
    stage_o = HostStage(budget // wl.K + wl.row_bytes)
    for t0, n in token_batches(wl.n_tok, wl.K, wl.row_bytes, budget):
        a0, a1 = t0 * wl.K, (t0 + n) * wl.K
        y_rows = stage_y.fetch(yflat.index_select(0, dst_d[a0:a1]))
        want = oracle.combine(local_dst(dst_tok[t0:t0 + n]), wl.K, y_rows, wf[a0:a1], W.BF16,
                              W.BF16)
        got = stage_o.fetch(oflat[t0:t0 + n])
        if not np.array_equal(got, want):
            bad = np.nonzero((got != want).any(axis=1))[0]
            raise AssertionError(f"combine differs at tokens {(t0 + bad[:8]).tolist()}")
    say(f"  combine: all {wl.n_tok} tokens equal")
    del y, recv, out, stage_y, stage_o

    # replicate: every materialised duplicate against the oracle's table
    say("  replicate")
    ew = W.make_expert_weights(wl, seed, DEV)
    dup_w = torch.zeros((wl.R, wl.B) + tuple(wl.block_shape), dtype=ew.dtype, device=DEV)
    td.moonep_replicate(dims, pb, ew, dup_w, wl.block_bytes)
    torch.cuda.synchronize()
    for r in range(wl.R):
        for b in range(min(int(p["n_dup"][r]), wl.B)):
            e = int(p["dup_expert"][r, b])
            assert torch.equal(dup_w[r, b].view(torch.int16), ew[e].view(torch.int16))
    del ew, dup_w

    # reduce: every expert with duplicates through the oracle; the others untouched
    say("  reduce")
    dg, hg = W.make_grads(wl, seed, DEV)
    n = wl.block_elems
    nl = int(p["n_list"][0])
    exps = sorted(set(p["list_expert"][:nl].tolist()))
    exps_d = torch.tensor(exps, dtype=torch.int64, device=DEV)
    before = hg.index_select(0, exps_d)
    hash0 = _row_hash(hg)
    td.moonep_reduce_dup_grads(dims, pb, dg, hg, n)
    torch.cuda.synchronize()
    most = max((sum(1 for q in range(int(p["dup_ptr"][e]), int(p["dup_ptr"][e + 1]))
                    if p["list_b"][q] < wl.B) for e in exps), default=0)
    stage = HostStage(4 * n * (most + 1))
    for i, e in enumerate(exps):
        q0, q1 = int(p["dup_ptr"][e]), int(p["dup_ptr"][e + 1])
        sel = [q for q in range(q0, q1) if p["list_b"][q] < wl.B]
        rows = [before[i]] + [dg[int(p["list_rank"][q]), int(p["list_b"][q])] for q in sel]
        h = stage.fetch(torch.stack(rows)).copy()
        sub = {"dup_ptr": np.array([0, len(sel)], np.int32),
               "list_rank": np.zeros(len(sel), np.int32),
               "list_b": np.arange(len(sel), dtype=np.int32)}
        want = oracle.reduce_dup_grads(sub, len(sel), h[1:].reshape(1, len(sel), n),
                                       h[0].reshape(1, n))
        got = stage.fetch(hg[e])
        assert np.array_equal(got.view(np.uint32), want.reshape(-1).view(np.uint32)), \
            f"reduce e={e}"
    untouched = torch.ones(wl.E, dtype=torch.bool, device=DEV)
    untouched[exps_d] = False
    assert torch.equal(_row_hash(hg)[untouched], hash0[untouched]), "an expert without duplicates changed"
    say(f"  ok (all {len(exps)} experts with duplicates reduced equal, "
        f"{int(untouched.sum())} untouched)")


@pytest.mark.parametrize("name", ["uniform", "zipf", "k3", "decode"])
def test_workload_closed_forms_full_size(td, name):
    """Properties that hold at any size, checked on every element at the full
    workload shapes (K a power of two, bf16 rows), bitwise on the GPU:
    - identity experts (y = recv) with weights 1/K: combine gives hidden back;
    - the backward of dispatch applied to a dispatch gives K * hidden (exact);
    - unit weights: grad_y of every slot is the grad_out row of its token."""
    wl = W.WORKLOADS[name]
    assert wl.K & (wl.K - 1) == 0 and wl.dtype == W.BF16
    dims = _dims(td, wl)
    say(f"closed forms {name}: {dims}")
    ids, _ = W.make_routing(wl, 5)
    pb, _ = run_plan(td, dims, ids, DEV)
    p = oracle.plan(wl.R, wl.E, wl.K, wl.S, wl.B, ids)
    assert np.array_equal(read_plan(td, dims, pb)["dst"], p["dst"])
    hid = W.make_hidden(wl, 5, DEV)
    recv = torch.empty((wl.R, wl.SK, wl.H), dtype=hid.dtype, device=DEV)
    td.moonep_dispatch(dims, pb, hid, recv)
    w_d = torch.full((wl.R, wl.S, wl.K), 1.0 / wl.K, dtype=torch.float32, device=DEV)
    out = torch.empty_like(hid)
    td.moonep_combine(dims, pb, recv, w_d, out)
    back = torch.empty_like(hid)
    td.moonep_dispatch_backward(dims, pb, recv, back)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), hid.view(torch.int16)), "combine of identity experts"
    assert torch.equal(back.view(torch.int16),
                       (hid.float() * wl.K).to(torch.bfloat16).view(torch.int16)), \
        "backward of dispatch of a dispatch"
    del out, back
    gout = W.dense((wl.R, wl.S, wl.H), W.BF16, 1.0, 6, "hidden", DEV)
    w_d.fill_(1.0)
    td.moonep_combine_backward(dims, pb, gout, w_d, None, recv, None)
    torch.cuda.synchronize()
    src_d = torch.from_numpy(p["src"].astype(np.int64)).to(DEV)
    gflat, rflat = gout.view(wl.n_tok, wl.H), recv.view(-1, wl.H)
    for r in range(wl.R):
        sl = slice(r * wl.SK, (r + 1) * wl.SK)
        assert torch.equal(rflat[sl].view(torch.int16),
                           gflat[src_d[sl] // wl.K].view(torch.int16)), f"grad_y rank {r}"
    say("  ok")
