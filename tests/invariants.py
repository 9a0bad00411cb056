"""Properties every valid balanced plan has, whichever placement it chose.

They restate what the pages require of the method: each rank receives exactly
S x K assignments whatever the skew, via duplicate experts of overloaded home
experts (news.hamidun.com EN, "How MoonEP works"), and rows sit at positions
grouped by expert (same page, "Why this matters to engineers"). The checker reads
a plan given as a dict of numpy arrays (from the oracle or from the GPU) and
raises AssertionError naming the first property that fails.
"""
import numpy as np


def check_plan(R, E, K, S, B, ids, p, valid_input=True):
    ids = np.asarray(ids).reshape(-1).astype(np.int64)
    G, SK, NE = E // R, S * K, R * S * K
    dst = np.asarray(p["dst"]).astype(np.int64)
    src = np.asarray(p["src"]).astype(np.int64)
    T = np.asarray(p["T"]).astype(np.int64)
    n_dup = np.asarray(p["n_dup"]).astype(np.int64)
    dcap = np.asarray(p["dup_expert"]).shape[1]
    dup_expert = np.asarray(p["dup_expert"]).astype(np.int64)
    dup_start = np.asarray(p["dup_start"]).astype(np.int64)
    dup_count = np.asarray(p["dup_count"]).astype(np.int64)
    valid = (ids >= 0) & (ids < E)

    # histogram and skew metric
    assert np.array_equal(T, np.bincount(ids[valid], minlength=E)), "T is not the histogram"
    maxT = int(T.max()) if E else 0
    assert int(np.asarray(p["maxT"]).reshape(-1)[0]) == maxT, "maxT"
    assert float(np.asarray(p["maxvio"]).reshape(-1)[0]) == (maxT * E) / NE - 1.0, "maxvio"

    # bijection between placed entries and filled slots
    assert np.all(dst[~valid] == -1), "invalid entries must not be placed"
    vd = dst[valid]
    assert np.all((vd >= 0) & (vd < NE)), "dst out of range"
    assert np.unique(vd).size == vd.size, "two entries share a slot"
    assert np.array_equal(src[vd], np.nonzero(valid)[0]), "src is not the inverse of dst"
    assert np.sum(src >= 0) == vd.size, "a slot names an entry that is not placed there"

    rows = np.array([np.sum(src[r * SK:(r + 1) * SK] >= 0) for r in range(R)])
    if valid_input:
        assert np.all(rows == SK), "a rank does not hold exactly S*K rows"
        assert rows.max() / SK - 1.0 == 0.0, "rank-level maxvio after balancing is not 0"

    L = np.array([T[r * G:(r + 1) * G].sum() for r in range(R)])
    keep = np.minimum(L, SK)
    # each rank keeps a prefix of its rows for home experts, filled slots are a prefix
    for r in range(R):
        s = src[r * SK:(r + 1) * SK]
        filled = np.nonzero(s >= 0)[0]
        assert np.array_equal(filled, np.arange(filled.size)), "filled slots are not a prefix"
        ex = ids[s[filled]]
        assert np.all(ex[:keep[r]] // G == r), "kept rows are not home experts"
        # contiguous expert grouping: an expert occupies one run per rank
        if ex.size:
            starts = np.concatenate([[True], ex[1:] != ex[:-1]])
            assert np.unique(ex[starts]).size == starts.sum(), "an expert is split inside a rank"
            assert np.all(np.diff(ex[:keep[r]]) >= 0), "home experts not in id order"
        # duplicates of this rank
        nd = int(n_dup[r])
        assert nd <= dcap
        runs_e, runs_s, runs_n = [], [], []
        i = int(keep[r])
        while i < filled.size:
            j = i
            while j < filled.size and ex[j] == ex[i]:
                j += 1
            runs_e.append(ex[i]); runs_s.append(i); runs_n.append(j - i)
            i = j
        assert nd == len(runs_e), "n_dup is not the number of duplicate runs"
        assert np.array_equal(dup_expert[r, :nd], runs_e), "dup_expert"
        assert np.array_equal(dup_start[r, :nd], runs_s), "dup_start"
        assert np.array_equal(dup_count[r, :nd], runs_n), "dup_count"
        assert np.all(dup_expert[r, nd:] == -1) and np.all(dup_start[r, nd:] == -1)
        assert np.all(dup_count[r, nd:] == 0)
        for e in runs_e:
            assert e // G != r, "a duplicate sits on its own home rank"
        if nd:
            assert keep[r] < SK, "a rank without deficit holds a duplicate"

    # each placed entry is on its home rank or on a rank holding a duplicate of its expert
    has_dup = np.zeros((R, E), dtype=bool)
    for r in range(R):
        has_dup[r, dup_expert[r, :n_dup[r]]] = True
    va = np.nonzero(valid)[0]
    d_rank, e_of = dst[va] // SK, ids[va]
    away = d_rank != e_of // G
    assert np.all(has_dup[d_rank[away], e_of[away]]), "entry on a rank without its expert"

    # minimal movement: exactly sum(max(L - SK, 0)) entries leave home
    assert away.sum() == np.sum(np.maximum(L - SK, 0)), "moved entries are not the minimum"
    # every expert's rows: kept + duplicates = T
    tot = np.zeros(E, dtype=np.int64)
    for r in range(R):
        np.add.at(tot, dup_expert[r, :n_dup[r]], dup_count[r, :n_dup[r]])
        s = src[r * SK:r * SK + keep[r]]
        tot += np.bincount(ids[s], minlength=E)
    assert np.array_equal(tot, T), "rows of an expert do not add up to T"
    n_pieces = int(n_dup.sum())
    if n_pieces:
        n_over_exp = int(np.unique(np.concatenate(
            [dup_expert[r, :n_dup[r]] for r in range(R)])).size)
        n_def = int(np.sum(keep < SK))
        assert n_pieces <= n_over_exp + n_def - 1, "more pieces than the merge allows"

    # segments: home experts in id order then duplicates; they tile the filled rows
    seg_ptr = np.asarray(p["seg_ptr"]).astype(np.int64)
    seg_expert = np.asarray(p["seg_expert"]).astype(np.int64)
    for r in range(R):
        ns = G + int(n_dup[r])
        sp = seg_ptr[r, :ns + 1]
        assert sp[0] == 0 and np.all(np.diff(sp) >= 0), "segments not monotone"
        assert sp[-1] == rows[r], "segments do not end at the last filled row"
        assert np.all(seg_ptr[r, ns + 1:] == -1) and np.all(seg_expert[r, ns:] == -1)
        assert np.array_equal(seg_expert[r, :G], np.arange(r * G, (r + 1) * G))
        assert np.array_equal(seg_expert[r, G:ns], dup_expert[r, :n_dup[r]])
        s = src[r * SK:r * SK + rows[r]]
        for i in range(ns):
            assert np.all(ids[s[sp[i]:sp[i + 1]]] == seg_expert[r, i]), "segment holds another expert"

    # global list: every duplicate once, ordered by (expert, rank)
    n_list = int(np.asarray(p["n_list"]).reshape(-1)[0])
    le = np.asarray(p["list_expert"]).astype(np.int64)
    lr = np.asarray(p["list_rank"]).astype(np.int64)
    lb = np.asarray(p["list_b"]).astype(np.int64)
    assert n_list == n_pieces
    want = sorted((int(dup_expert[r, b]), r, b) for r in range(R) for b in range(n_dup[r]))
    got = list(zip(le[:n_list].tolist(), lr[:n_list].tolist(), lb[:n_list].tolist()))
    assert got == want, "global duplicate list"
    assert np.all(le[n_list:] == -1) and np.all(lr[n_list:] == -1) and np.all(lb[n_list:] == -1)
    dup_ptr = np.asarray(p["dup_ptr"]).astype(np.int64)
    assert np.array_equal(dup_ptr, np.searchsorted(le[:n_list], np.arange(E + 1), side="left"))

    # status flags
    st = int(np.asarray(p["status"]).reshape(-1)[0])
    bad = bool(np.any(~valid))
    rep = any(len(set(t[(t >= 0) & (t < E)].tolist())) < np.sum((t >= 0) & (t < E))
              for t in ids.reshape(-1, K))
    assert bool(st & 1) == bad and bool(st & 2) == rep and bool(st & 4) == bool(np.any(n_dup > B))
    return True
