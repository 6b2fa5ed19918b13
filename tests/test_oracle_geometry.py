"""Pins for window geometry and visibility (oracle only, CPU)."""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_entry_counts_match_stated_workloads():
    rows = json.load(open(os.path.join(GOLD, "entry_counts.json")))
    for r in rows["rows"]:
        assert oracle.n_entries(r["L"], r["w"], r["s"]) == r["N"], r
    for r in rows["approximate"]:
        n = oracle.n_entries(r["L"], r["w"], r["s"])
        assert abs(n - r["N_about"]) <= r["rel_tol"] * r["N_about"], (n, r)


def test_start_padded_placement_is_ruled_out():
    # A window placement padded at the start would give L/s entries; the stated
    # counts (1023 at 4096, 8191 at 32768) rule it out.
    assert oracle.n_entries(4096, 8, 4) == 4096 // 4 - 1
    assert oracle.n_entries(32768, 8, 4) == 32768 // 4 - 1


@pytest.mark.parametrize("w,s", [(8, 4), (128, 128), (4, 4), (3, 1), (1, 1)])
def test_visibility_closed_forms(w, s):
    N = 200
    for p in range(0, 400):
        n = oracle.n_visible(p, w, s, N)
        closed = 0 if p < w - 1 else min(N, (p - w + 1) // s + 1)
        assert n == closed, (p, n, closed)
        # every visible entry ends at or before p, the next one does not
        if n:
            assert oracle.entry_span(n - 1, w, s)[1] - 1 <= p
        if n < N:
            assert oracle.entry_span(n, w, s)[1] - 1 > p


def test_visibility_special_forms():
    # CSA (8 at stride 4): floor((p+1)/4) - 1 visible entries once p >= 7;
    # HCA (128 disjoint): floor((p+1)/128).
    for p in range(7, 1000):
        assert oracle.n_visible(p, 8, 4, 10**6) == (p + 1) // 4 - 1
    for p in range(0, 2000):
        assert oracle.n_visible(p, 128, 128, 10**6) == (p + 1) // 128
    # Decode at the last position sees every entry of a 2^20 sequence.
    L = 1 << 20
    assert (L - 1 + 1) // 4 - 1 == oracle.n_entries(L, 8, 4)
    assert (L - 1 + 1) // 128 == oracle.n_entries(L, 128, 128)
    # Identity geometry (one entry per position): query j of a 1024-chunk at the
    # end of 131072 entries sees 130049 + j entries.
    for j in (0, 1, 500, 1023):
        assert oracle.n_visible(131072 - 1024 + j, 1, 1, 131072) == 130049 + j


def test_window_rows():
    assert list(oracle.window_rows(0, 128)) == [0]
    assert list(oracle.window_rows(5, 128)) == list(range(0, 6))
    r = oracle.window_rows(1000, 128)
    assert r[0] == 873 and r[-1] == 1000 and len(r) == 128
