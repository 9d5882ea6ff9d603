"""Pins for the oracle's sharding maps: brute force, round trips, the pages'
worked example, and the explicit formulas of the long-context and tiny
workloads.  A planted mistake in any map must fail one of these."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import maps
import dsa_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GRID = [(S, I) for S in (1, 2, 3, 4, 8) for I in (1, 5, 64)]


def _brute(N, S, I):
    """Enumerate the ownership rule token by token: each shard's tokens in
    global order, so a token's local position is its index in that list."""
    lists = [[] for _ in range(S)]
    for t in range(N):
        lists[(t // I) % S].append(t)
    return lists


@pytest.mark.parametrize("S,I", GRID)
def test_maps_vs_brute_force(S, I):
    N = 3 * S * I + 17
    lists = _brute(N, S, I)
    for r, toks in enumerate(lists):
        for l, t in enumerate(toks):
            assert int(oracle.owner(t, S, I)) == r
            assert int(oracle.local(t, S, I)) == l
            assert int(oracle.global_id(r, l, S, I)) == t
    for n in range(N + 1):
        for r in range(S):
            brute = sum(1 for t in lists[r] if t < n)
            assert int(oracle.local_count(n, r, S, I)) == brute


@pytest.mark.parametrize("S,I", GRID)
def test_round_trip_and_monotone(S, I):
    t = np.arange(5 * S * I + 3)
    r = oracle.owner(t, S, I)
    l = oracle.local(t, S, I)
    assert np.array_equal(oracle.global_id(r, l, S, I), t)
    for rr in range(S):
        g = oracle.global_id(rr, np.arange(40), S, I)
        assert np.all(np.diff(g) > 0)
    # local counts of all shards add up to n
    for n in range(0, 4 * S * I):
        assert sum(int(oracle.local_count(n, rr, S, I)) for rr in range(S)) == n


def test_pages_worked_example():
    ex = json.load(open(os.path.join(GOLDEN, "dcp_localize_example.json")))
    S, r, I, L, T = ex["world"], ex["rank"], ex["interleave"], ex["request_len"], ex["tokens"]
    per_token_global = [L - T + 1 + j for j in range(T)]
    right = [int(oracle.local_count(n, r, S, I)) for n in per_token_global]
    assert right == ex["expected_local_lens"]
    req_local = int(oracle.local_count(L, r, S, I))
    wrong = [req_local - (T - 1 - j) for j in range(T)]
    assert wrong == ex["wrong_order_local_lens"]


def test_pages_example_is_unique_in_range():
    hits = [L for L in range(3, 40)
            if [int(oracle.local_count(n, 1, 2, 1)) for n in (L - 2, L - 1, L)] == [4, 4, 5]
            and [int(oracle.local_count(L, 1, 2, 1)) - 2 + j for j in range(3)] == [3, 4, 5]]
    assert hits == [10]


def test_long_context_formula():
    # 8 shards, interleave 64: shard (t // 64) % 8, local (t // 512) * 64 + t % 64
    t = np.arange(0, 131072, 37)
    assert np.array_equal(oracle.owner(t, 8, 64), (t // 64) % 8)
    assert np.array_equal(oracle.local(t, 8, 64), (t // 512) * 64 + t % 64)


def test_tiny_formula():
    # 2 shards, interleave 1: shard t % 2, local t // 2
    t = np.arange(4096)
    assert np.array_equal(oracle.owner(t, 2, 1), t % 2)
    assert np.array_equal(oracle.local(t, 2, 1), t // 2)


@pytest.mark.parametrize("S,I", [(4, 1), (8, 64), (3, 5), (2, 3)])
def test_generator_layout_matches_maps(S, I):
    """The input generator places logits by a reshape; the oracle's maps must
    describe the same placement."""
    ctx = 7 * S * I + 11
    g = np.arange(ctx, dtype=np.int64)[None, :]
    sh = dsa_inputs.shard_layout(g, S, I, -1)[:, 0, :]
    for r in range(S):
        n = int(oracle.local_count(ctx, r, S, I))
        assert np.array_equal(sh[r, :n], oracle.global_id(r, np.arange(n), S, I))
        assert np.all(sh[r, n:] == -1)


# ---- planted mistakes: each must be caught by the brute-force pin ----------
def _mut_local_count_noclamp(n, r, S, I):
    n = np.asarray(n)
    return (n // (I * S)) * I + np.maximum(n % (I * S) - r * I, 0)


def _mut_owner_no_interleave(t, S, I):
    return np.asarray(t) % S


def _mut_local_swapped(t, S, I):
    t = np.asarray(t)
    return (t // (I * S)) * I + (t // I) % I


@pytest.mark.parametrize("name,fn", [("local_count", _mut_local_count_noclamp),
                                     ("owner", _mut_owner_no_interleave),
                                     ("local", _mut_local_swapped)])
def test_planted_mistakes_are_caught(monkeypatch, name, fn):
    monkeypatch.setattr(oracle, name, fn)
    failed = False
    for S, I in [(2, 5), (3, 5), (8, 64)]:
        try:
            test_maps_vs_brute_force(S, I)
        except AssertionError:
            failed = True
    assert failed, f"a wrong {name} passed the brute-force pin"
