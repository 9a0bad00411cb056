"""A second, independent formulation of the water-fill plan, used only to pin the
oracle: sort-and-slice with numpy instead of running counters and prefix sums.

For each home rank: stable-sort its entries by expert (entries are already in
(token, k) order, so this gives (expert, token, k) order); keep the first S*K;
the rest is that rank's overflow. Concatenating the overflow lists in rank order
gives the global overflow order (home rank, expert, token, k); concatenating the
deficit slots of every rank in rank order gives the order they are filled in.
A duplicate is a maximal group of consecutive overflow entries that share the
expert and the receiving rank.

The method is described on the news.hamidun.com EN page ("How MoonEP works":
exactly S x K per rank by scheduling duplicate experts) and the tokens land at
expert-grouped positions ("Why this matters to engineers").
"""
import numpy as np


def plan_by_sorting(R, E, K, S, ids):
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    G, SK = E // R, S * K
    a_all = np.arange(ids.size)
    valid = (ids >= 0) & (ids < E)
    home = np.where(valid, ids // G, -1)
    dst = np.full(ids.size, -1, dtype=np.int64)
    n_keep = np.zeros(R, dtype=np.int64)
    overflow = []
    for r in range(R):
        mine = a_all[home == r]
        order = np.argsort(ids[mine], kind="stable")
        lst = mine[order]
        kept = lst[:SK]
        dst[kept] = r * SK + np.arange(kept.size)
        n_keep[r] = kept.size
        overflow.append(lst[SK:])
    over = np.concatenate(overflow) if overflow else np.zeros(0, np.int64)
    deficit = np.concatenate([r * SK + np.arange(n_keep[r], SK) for r in range(R)])
    assert over.size <= deficit.size
    dst[over] = deficit[:over.size]

    src = np.full(R * SK, -1, dtype=np.int64)
    src[dst[valid]] = a_all[valid]

    # duplicates: consecutive overflow entries with the same (expert, receiving rank)
    pieces = []  # (rank, expert, first slot, rows)
    i = 0
    while i < over.size:
        e, r = ids[over[i]], dst[over[i]] // SK
        j = i
        while j < over.size and ids[over[j]] == e and dst[over[j]] // SK == r:
            j += 1
        pieces.append((int(r), int(e), int(dst[over[i]] % SK), int(j - i)))
        i = j
    per_rank = [[p for p in pieces if p[0] == r] for r in range(R)]
    n_dup = np.array([len(x) for x in per_rank], dtype=np.int64)
    dups = [(r, b, e, s0, n) for r in range(R) for b, (_, e, s0, n) in enumerate(per_rank[r])]
    lst = sorted(((e, r, b) for (r, b, e, _, _) in dups))
    list_expert = np.array([x[0] for x in lst], dtype=np.int64)
    dup_ptr = np.searchsorted(list_expert, np.arange(E + 1), side="left")
    T = np.bincount(ids[valid], minlength=E)
    return {
        "T": T, "dst": dst, "src": src, "n_dup": n_dup, "dups": dups, "list": lst,
        "dup_ptr": dup_ptr, "n_keep": n_keep,
    }
