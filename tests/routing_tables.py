"""Checks the routing step's integer tables against their definition.

The bucketing step groups a batch's (token, slot) pairs by expert (pair q = t*k + j is
slot j of token t).  Given the ids, the tables are fixed up to two orders:

  * the job records: one per used expert, each (expert, first position, count, 0, the
    first `record_pairs` pair ids of its bucket, -1 past the count), in one of two orders:
    experts ascending (the batch launches), or order of first appearance -- record u is
    the expert of the u-th pair, in pair order, that is the first pair to pick its expert
    (batches routed inside one workgroup; for one token that is its rank order);
  * the pair table: each used expert owns one contiguous bucket, pairs ascending inside
    it, buckets laid out with experts ascending or in order of first appearance;
  * the pair-expert table gives each bucketed position its bucket's expert.

From these follow the invariants: the counts sum to T*k, every pair appears exactly
once, and the used-expert count equals the size of the set of ids.  Integer work, so
the comparison is exact.  Pure numpy: the CPU tests plant mistakes in correct tables
to show that each one is caught.
"""
from __future__ import annotations

import numpy as np

ORDERS = ("ascending", "first")


def expert_order(ids: np.ndarray, order: str) -> list[int]:
    """Used experts, ascending or in order of first appearance (pair order)."""
    flat = [int(e) for e in np.asarray(ids).reshape(-1)]
    if order == "ascending":
        return sorted(set(flat))
    seen: list[int] = []
    for e in flat:
        if e not in seen:
            seen.append(e)
    return seen


def expected_tables(ids: np.ndarray, record_pairs: int, record_order: str = "ascending",
                    layout_order: str = "ascending") -> dict:
    """The tables of ids [T, k] for the given record order and bucket layout order."""
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    buckets = {e: [q for q in range(T * k) if flat[q] == e] for e in set(flat.tolist())}
    start, pairs, pair_expert = {}, [], []
    for e in expert_order(ids, layout_order):
        start[e] = len(pairs)
        pairs += buckets[e]
        pair_expert += [e] * len(buckets[e])
    records = []
    for e in expert_order(ids, record_order):
        rec = [e, start[e], len(buckets[e]), 0] + [-1] * record_pairs
        for a, q in enumerate(buckets[e][:record_pairs]):
            rec[4 + a] = q
        records.append(rec)
    return {"n_used": len(records), "records": np.array(records, dtype=np.int64).reshape(len(records), 4 + record_pairs),
            "pairs": np.array(pairs, dtype=np.int64), "pair_expert": np.array(pair_expert, dtype=np.int64)}


def check_tables(tab: dict, ids: np.ndarray) -> tuple[str, str]:
    """Asserts that the tables `tab` (numpy ints: n_used, records [U, 4 + record_pairs],
    pairs [T*k], pair_expert [T*k]) are those of ids [T, k] under one of the allowed
    orders; returns (record order, layout order)."""
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
    # the unique tables of one of the allowed orders
    used = recs[:, 0].tolist()
    rorder = [o for o in ORDERS if used == expert_order(ids, o)]
    assert rorder, f"job records in neither ascending nor first-appearance order: {used}"
    by_start = [int(e) for e in recs[np.argsort(recs[:, 1], kind="stable"), 0]]
    lorder = [o for o in ORDERS if by_start == expert_order(ids, o)]
    assert lorder, "bucket layout in neither ascending nor first-appearance order"
    want = expected_tables(ids, rp, rorder[0], lorder[0])
    assert np.array_equal(recs, want["records"]), "job records"
    assert np.array_equal(pairs, want["pairs"]), "bucketed pairs"
    assert np.array_equal(pexp, want["pair_expert"]), "expert of each bucketed position"
    return rorder[0], lorder[0]
