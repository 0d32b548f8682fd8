"""Checks the routing step's integer tables against their definition.

The bucketing step groups a batch's (token, slot) pairs by expert (pair q = t*k + j is
slot j of token t).  Given the ids, the tables are unique:

  * the used experts are the distinct ids, ascending; for a single token they may
    instead keep its rank order (its k experts are distinct, one bucket each);
  * each used expert owns one contiguous bucket of the pair table, buckets in the order
    of the used experts, pairs ascending inside a bucket;
  * the job record of used expert u is (expert, first position, count, 0, the first
    `record_pairs` pair ids of its bucket, -1 past the count);
  * the pair-expert table gives each bucketed position its bucket's expert.

From these follow the invariants: the counts sum to T*k, every pair appears exactly
once, and the used-expert count equals the size of the set of ids.  Integer work, so
the comparison is exact.  Pure numpy: the CPU tests plant mistakes in correct tables
to show that each one is caught.
"""
from __future__ import annotations

import numpy as np


def expected_tables(ids: np.ndarray, record_pairs: int, rank_order: bool = False) -> dict:
    """The tables the definition gives for ids [T, k] (rank_order: one token's experts
    in its rank order instead of ascending)."""
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    if rank_order:
        assert T == 1
        used = [int(e) for e in flat]
    else:
        used = sorted(set(int(e) for e in flat))
    records, pairs, pair_expert = [], [], []
    for e in used:
        bucket = [q for q in range(T * k) if flat[q] == e]
        rec = [e, len(pairs), len(bucket), 0] + [-1] * record_pairs
        for a, q in enumerate(bucket[:record_pairs]):
            rec[4 + a] = q
        records.append(rec)
        pairs += bucket
        pair_expert += [e] * len(bucket)
    return {"n_used": len(used), "records": np.array(records, dtype=np.int64).reshape(len(used), 4 + record_pairs),
            "pairs": np.array(pairs, dtype=np.int64), "pair_expert": np.array(pair_expert, dtype=np.int64)}


def check_tables(tab: dict, ids: np.ndarray) -> None:
    """Asserts that the tables `tab` (numpy ints: n_used, records [U, 4 + record_pairs],
    pairs [T*k], pair_expert [T*k]) are those of ids [T, k]."""
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    rp = int(tab["record_pairs"])
    n_used = int(tab["n_used"])
    recs = np.asarray(tab["records"], dtype=np.int64)
    pairs = np.asarray(tab["pairs"], dtype=np.int64)
    pexp = np.asarray(tab["pair_expert"], dtype=np.int64)
    # the invariants, stated on their own
    assert n_used == len(set(ids.reshape(-1).tolist())), f"used experts {n_used} vs {len(set(ids.reshape(-1)))}"
    assert recs.shape[0] == n_used
    assert int(recs[:, 2].sum()) == T * k, "bucket counts must sum to T*k"
    assert np.array_equal(np.sort(pairs), np.arange(T * k)), "every pair exactly once"
    assert len(set(recs[:, 0].tolist())) == n_used, "a used expert listed twice"
    # the unique tables
    rank = T == 1 and recs[:, 0].tolist() == ids[0].tolist()
    want = expected_tables(ids, rp, rank_order=rank)
    assert np.array_equal(recs, want["records"]), "job records"
    assert np.array_equal(pairs, want["pairs"]), "bucketed pairs"
    assert np.array_equal(pexp, want["pair_expert"]), "expert of each bucketed position"
