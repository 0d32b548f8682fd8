"""The bucketing-table checker catches each plausible mistake in the tables (CPU).

Correct tables are built from their definition for random routings; each planted
mistake -- a pair listed twice, a used expert listed twice, pairs out of order inside a
bucket, a wrong count, start, inline pair id or bucket expert, a wrong used-expert
count -- must fail the check.
"""
from __future__ import annotations

import numpy as np
import pytest

from tests.routing_tables import check_tables, expected_tables

RP = 12


def _ids(T, k, E, seed):
    rng = np.random.default_rng(seed)
    return np.stack([rng.choice(E, k, replace=False) for _ in range(T)])


def _tables(ids, record_order="ascending", layout_order="ascending"):
    t = expected_tables(ids, RP, record_order, layout_order)
    t["record_pairs"] = RP
    return t


ORDER_PAIRS = [("ascending", "ascending"), ("first", "ascending"), ("first", "first")]


@pytest.mark.parametrize("orders", ORDER_PAIRS)
@pytest.mark.parametrize("T,k,E", [(1, 8, 256), (2, 8, 256), (8, 8, 256), (17, 8, 64), (40, 2, 4), (6, 16, 24)])
def test_correct_tables_pass(T, k, E, orders):
    ids = _ids(T, k, E, T * 1000 + k)
    assert check_tables(_tables(ids, *orders), ids) in [orders, ("ascending", "ascending"),
                                                         ("first", "first"), ("first", "ascending")]


def test_single_token_in_rank_order_passes():
    # one token: first appearance is its rank order
    ids = np.array([[7, 3, 200, 1, 9, 100, 50, 2]])
    assert check_tables(_tables(ids, "first", "first"), ids) == ("first", "first")
    assert check_tables(_tables(ids), ids) == ("ascending", "ascending")


def test_first_appearance_order_by_hand():
    # pairs 0..5 pick experts 5 3 | 3 9 | 1 5: first appearances 5, 3, 9, 1
    ids = np.array([[5, 3], [3, 9], [1, 5]])
    t = _tables(ids, "first", "ascending")
    assert t["records"][:, 0].tolist() == [5, 3, 9, 1]
    assert t["records"][:, 1].tolist() == [3, 1, 5, 0]  # positions with experts ascending: 1 3 3 5 5 9
    assert t["pairs"].tolist() == [4, 1, 2, 0, 5, 3]
    check_tables(t, ids)


def _mutants(ids, orders=("ascending", "ascending")):
    base = _tables(ids, *orders)

    def m(fn):
        t = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in base.items()}
        fn(t)
        return t

    big = int(np.argmax(base["records"][:, 2]))  # a bucket of at least two pairs
    s = int(base["records"][big, 1])

    def dup_pair(t):
        t["pairs"][s + 1] = t["pairs"][s]

    def swap_in_bucket(t):
        t["pairs"][s], t["pairs"][s + 1] = t["pairs"][s + 1], t["pairs"][s]
        t["records"][big, 4], t["records"][big, 5] = t["records"][big, 5], t["records"][big, 4]

    def dup_expert(t):
        t["records"][1, 0] = t["records"][0, 0]

    def count(t):
        t["records"][big, 2] += 1

    def start(t):
        t["records"][big, 1] += 1

    def inline_pair(t):
        t["records"][0, 4] += 1

    def no_terminator(t):
        r = int(np.argmin(t["records"][:, 2]))
        t["records"][r, 4 + t["records"][r, 2]] = 0

    def pair_expert(t):
        t["pair_expert"][s] += 1

    def n_used(t):
        t["n_used"] += 1

    def order_of_used(t):
        t["records"][[0, 1]] = t["records"][[1, 0]]

    return {f.__name__: m(f) for f in (dup_pair, swap_in_bucket, dup_expert, count, start, inline_pair,
                                         no_terminator, pair_expert, n_used, order_of_used)}


@pytest.mark.parametrize("orders", ORDER_PAIRS)
@pytest.mark.parametrize("name", ["dup_pair", "swap_in_bucket", "dup_expert", "count", "start", "inline_pair",
                                  "no_terminator", "pair_expert", "n_used", "order_of_used"])
def test_planted_mistakes_fail(name, orders):
    ids = _ids(8, 8, 48, 5)  # 64 pairs over at most 48 experts: shared buckets
    with pytest.raises(AssertionError):
        check_tables(_mutants(ids, orders)[name], ids)
