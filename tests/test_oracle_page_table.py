"""Pins of the oracle's page-table builder (page "msa.py", _build_page_table):
hand-derived cases, the generator's own page tables rebuilt from the
allocator's map it implies, packed and padded forms against each other, and
the caller errors it refuses."""
import json
import os

import numpy as np
import pytest

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def _map(c):
    if "req_to_token" in c:
        return np.array(c["req_to_token"], np.int32)
    rows = []
    for ranges in c["req_to_token_ranges"]:
        n = max(b for _, b, _ in ranges)
        row = np.full(n, -1, np.int32)
        for a, b, s in ranges:
            row[a:b] = s + np.arange(b - a)
        rows.append(row)
    return np.array(rows, np.int32)


def test_hand_derived_cases(orc):
    for c in json.load(open(os.path.join(HERE, "golden", "page_table_cases.json")))["cases"]:
        table, packed, indptr = oracle.page_table(_map(c), np.array(c["slot_ids"]),
                                                  np.array(c["kv_lens"]), c["page_size"],
                                                  c["max_pages"])
        np.testing.assert_array_equal(table, c["page_table"], err_msg=c["why"])
        np.testing.assert_array_equal(packed, c["kv_indices"], err_msg=c["why"])
        np.testing.assert_array_equal(indptr, c["kv_indptr"], err_msg=c["why"])


@pytest.mark.parametrize("kw", [
    dict(batch=4, q_len=1), dict(batch=3, q_len=8, page_size=4),
    dict(batch=5, q_len=3, page_size=64), dict(batch=2, q_len=2, table="identity"),
])
def test_rebuilds_the_generators_tables(orc, kw):
    """The generator draws each request's pages; the allocator map they imply
    (slot of position p = page_table[b, p // P] * P + p % P, written here with
    numpy) goes back to the same table, for the step's whole key range."""
    x = synth.make_inputs(synth.small(**kw))
    w = x.w
    P = w.page_size
    B = w.batch
    stride = x.max_pages * P
    rng = np.random.default_rng(3)
    rows = rng.permutation(B + 3)[:B]  # request b lives in allocator row rows[b]
    r2t = np.full((B + 3, stride), -7, np.int32)
    for b in range(B):
        p = np.arange(int(x.cache_seqlens[b]))
        r2t[rows[b], p] = x.page_table[b, p // P] * P + p % P
    table, packed, indptr = oracle.page_table(r2t, rows, x.cache_seqlens, P, x.max_pages)
    np.testing.assert_array_equal(table, x.page_table)
    n = -(-x.cache_seqlens.astype(np.int64) // P)
    np.testing.assert_array_equal(np.diff(indptr), n)
    for b in range(B):
        np.testing.assert_array_equal(packed[indptr[b]:indptr[b + 1]], table[b, :n[b]])


def test_padded_slots_and_caller_errors(orc):
    r2t = np.arange(40, dtype=np.int32).reshape(2, 20)
    table, packed, indptr = oracle.page_table(r2t, np.array([1, 0]), np.array([0, -3]), 4, 5)
    assert np.all(table == -1) and len(packed) == 0 and list(indptr) == [0, 0, 0]
    with pytest.raises(ValueError):  # slot id outside the map
        oracle.page_table(r2t, np.array([2]), np.array([4]), 4, 5)
    with pytest.raises(ValueError):  # a page starting past the map's row
        oracle.page_table(r2t, np.array([0]), np.array([21]), 4, 6)
    with pytest.raises(ValueError):  # more pages than the padded table holds
        oracle.page_table(r2t, np.array([0]), np.array([17]), 4, 4)
