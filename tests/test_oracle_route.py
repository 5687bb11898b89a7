"""Pins for the oracle's expert sort (CPU only): a brute-force loop written
from the definition, plus the invariants of a band layout."""

import numpy as np
import pytest

from oracle import route_sort
from moe_grouped_gemm_route_amd.synth import make_problem, make_config


def _brute(ids, E):
    T, k = ids.shape
    rows = []
    for e in range(E):                      # bands in expert order
        for t in range(T):                  # pairs in flat order inside a band
            for j in range(k):
                if ids[t, j] == e:
                    rows.append(t * k + j)
    return rows


def _check(ids, E):
    r = route_sort(ids, E)
    T, k = ids.shape
    M = T * k
    rows = _brute(ids, E)
    n = len(rows)
    assert r["err_count"] == M - n
    assert r["sorted_pair"][:n].tolist() == rows
    assert np.all(r["sorted_pair"][n:] == -1) and np.all(r["sorted_token"][n:] == -1)
    assert r["sorted_token"][:n].tolist() == [p // k for p in rows]
    for row, p in enumerate(rows):
        assert r["pair_row"][p] == row
    dropped = set(range(M)) - set(rows)
    for p in dropped:
        assert r["pair_row"][p] == -1
    off = r["group_offsets"]
    assert off[0] == 0 and off[-1] == n and np.all(np.diff(off) >= 0)
    for e in range(E):
        assert off[e + 1] - off[e] == int(np.sum(ids == e))
        band = r["sorted_pair"][off[e]:off[e + 1]]
        assert np.all(ids.reshape(-1)[band] == e)
        assert np.all(np.diff(band) > 0)
    return r


def test_route_sort_small_random():
    rng = np.random.default_rng(0)
    for T, k, E in [(1, 1, 1), (5, 2, 3), (17, 4, 9), (40, 6, 16)]:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        _check(ids, E)


def test_route_sort_duplicates_and_all_on_one_expert():
    ids = np.zeros((7, 3), dtype=np.int32)
    r = _check(ids, 4)
    assert r["group_offsets"].tolist() == [0, 21, 21, 21, 21]


def test_route_sort_invalid_ids_are_dropped():
    ids = np.array([[0, 5], [-1, 2], [2, 1]], dtype=np.int32)
    r = _check(ids, 3)
    assert r["err_count"] == 2
    assert r["pair_row"][1] == -1 and r["pair_row"][2] == -1


def test_route_sort_matches_library_stable_argsort_on_config1():
    cfg = make_config(1)
    ids = cfg["topk_ids"]
    r = _check(ids, cfg["E"])
    assert np.array_equal(r["sorted_pair"], np.argsort(ids.reshape(-1), kind="stable"))
    assert r["group_offsets"][8] - r["group_offsets"][7] == 0   # expert 7 forced empty


@pytest.mark.parametrize("routing", ["uniform", "zipf"])
def test_route_sort_large_shapes_invariants(routing):
    p = make_problem(T=4096, k=6, E=256, K=32, N=1, seed=4, routing=routing)
    ids = p["topk_ids"]
    r = route_sort(ids, 256)
    assert np.array_equal(r["sorted_pair"], np.argsort(ids.reshape(-1), kind="stable"))
    inv = np.empty_like(r["pair_row"])
    inv[r["sorted_pair"]] = np.arange(ids.size)
    assert np.array_equal(inv, r["pair_row"])
    assert np.array_equal(np.diff(r["group_offsets"]), np.bincount(ids.reshape(-1), minlength=256))
