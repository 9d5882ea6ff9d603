"""Pins for the oracle's top-K, merge and index conversion: brute-force full
sort on tiny inputs, the library special case (distinct scores), the
sharded-then-merged == unsharded invariant, and conversion round trips."""
import numpy as np
import pytest
import torch

import oracle
from oracle import select as osel


def _brute_topk(scores, k):
    """Full sort by (score desc, index asc) in plain Python; -0.0 == +0.0."""
    order = sorted(range(len(scores)), key=lambda t: (-float(scores[t]), t))
    return sorted(order[:k])


def _tie_heavy(rng, R, C):
    x = np.round(rng.standard_normal((R, C)) * 4.0) / 4.0     # many equal values
    return x.astype(np.float32)


@pytest.mark.parametrize("seed", range(6))
def test_single_shard_vs_brute_force(seed):
    rng = np.random.default_rng(seed)
    R, C, k = 3, 97, 20
    x = _tie_heavy(rng, R, C)
    starts = np.array([0, 5, 40], dtype=np.int32)
    ends = np.array([97, 60, 52], dtype=np.int32)
    idx, cand = oracle.topk_select(x[None], starts, ends, C, k, 1, 1)
    for i in range(R):
        seg = x[i, starts[i]:ends[i]]
        exp = [starts[i] + t for t in _brute_topk(seg, k)]
        m = len(exp)
        assert idx[0, i, :m].tolist() == exp
        assert np.all(idx[0, i, m:] == -1)
        assert np.array_equal(cand[i, :m, 0].view(np.uint32), x[i, exp].view(np.uint32))
        assert cand[i, :m, 1].tolist() == [float(e) for e in exp]
        assert np.all(cand[i, m:, 1] == -1.0) and np.all(np.isneginf(cand[i, m:, 0]))


def test_signed_zero_ties_break_by_position():
    x = np.array([[0.0, -0.0, 1.0, -0.0, 0.0, -1.0]], dtype=np.float32)
    idx, _ = oracle.topk_select(x[None], np.array([0]), np.array([6]), 6, 3, 1, 1)
    # 1.0 first, then the zeros in position order: positions 0 and 1
    assert idx[0, 0].tolist() == [0, 1, 2]


def test_distinct_scores_match_library_topk():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((4, 3000)).astype(np.float32)
    idx, _ = oracle.topk_select(x[None], np.zeros(4, np.int32), np.full(4, 3000, np.int32), 3000, 512, 1, 1)
    ref = torch.topk(torch.from_numpy(x), 512, dim=1).indices.numpy()
    for i in range(4):
        assert set(idx[0, i].tolist()) == set(ref[i].tolist())


@pytest.mark.parametrize("S,I", [(1, 1), (2, 1), (3, 5), (4, 1), (8, 64), (2, 3)])
@pytest.mark.parametrize("seed", [0, 1])
def test_sharded_then_merged_equals_unsharded(S, I, seed):
    rng = np.random.default_rng(100 * S + I + seed)
    R, C, k = 4, 1500, 128
    g = _tie_heavy(rng, R, C)
    starts = np.array([0, 3, 200, 0], dtype=np.int32)
    ends = np.array([C, 1200, 260, 50], dtype=np.int32)   # last rows: fewer than k
    # place by the oracle's own maps
    ld = int(oracle.local_count(C, 0, S, I))
    sh = np.full((S, R, ld), 99.0, dtype=np.float32)
    for r in range(S):
        n = int(oracle.local_count(C, r, S, I))
        sh[r, :, :n] = g[:, oracle.global_id(r, np.arange(n), S, I)]
    _, cand = oracle.topk_select(sh, starts, ends, C, k, S, I)
    ids = oracle.merge_candidates(cand, k)
    for i in range(R):
        exp = oracle.unsharded_topk(g[i], starts[i], ends[i], k)
        assert ids[i, :len(exp)].tolist() == exp.tolist()
        assert np.all(ids[i, len(exp):] == -1)
        # and the unsharded helper itself agrees with brute force
        bf = [starts[i] + t for t in _brute_topk(g[i, starts[i]:ends[i]], k)]
        assert exp.tolist() == bf


def test_merge_vs_brute_force_with_cross_shard_ties():
    # every score equal: the k smallest ids win, wherever they sit
    rng = np.random.default_rng(3)
    N, k = 40, 7
    ids = rng.permutation(1000)[:N].astype(np.float32)
    cand = np.stack([np.full(N, 2.5, np.float32), ids], axis=-1)[None]
    cand[0, 5] = (9.0, -1.0)          # padding never wins, whatever its score
    out = oracle.merge_candidates(cand, k)
    valid = sorted(int(v) for j, v in enumerate(ids) if j != 5)
    assert out[0].tolist() == valid[:k]
    # generic brute force with mixed scores
    sc = np.round(rng.standard_normal(N) * 2) / 2
    cand2 = np.stack([sc.astype(np.float32), ids], axis=-1)[None]
    out2 = oracle.merge_candidates(cand2, k)
    order = sorted(range(N), key=lambda j: (-float(sc[j]), int(ids[j])))
    assert out2[0].tolist() == sorted(int(ids[j]) for j in order[:k])


def test_merge_fewer_valid_than_k():
    cand = np.array([[[1.0, 4.0], [-np.inf, -1.0], [3.0, 2.0], [-np.inf, -1.0]]], np.float32)
    assert oracle.merge_candidates(cand, 3)[0].tolist() == [2, 4, -1]


@pytest.mark.parametrize("S,I", [(1, 1), (4, 1), (8, 64), (3, 5)])
def test_convert_round_trip(S, I):
    rng = np.random.default_rng(S * 10 + I)
    R, C, k, B = 3, 2000, 300, 64
    ld = int(oracle.local_count(C, 0, S, I))
    W = -(-ld // B)
    nb = S * R * W
    bt = rng.permutation(nb).astype(np.int32).reshape(S, R, W)
    ids = np.full((R, k), -1, np.int32)
    for i in range(R):
        n = [k, 100, 0][i]
        ids[i, :n] = np.sort(rng.choice(C, n, replace=False))
    slots, counts = oracle.convert_index(ids, None, bt, B, S, I)
    nvalid = (ids >= 0).sum(axis=1)
    assert np.array_equal(counts.sum(axis=0), nvalid)
    inv = {}                               # physical block -> (shard, req, col)
    for r in range(S):
        for q in range(R):
            for c in range(W):
                inv[int(bt[r, q, c])] = (r, q, c)
    for i in range(R):
        got = []
        for r in range(S):
            c = counts[r, i]
            assert np.all(slots[r, i, c:] == -1)
            locs = []
            for s in slots[r, i, :c]:
                rr, q, col = inv[int(s) // B]
                assert rr == r and q == i
                locs.append(col * B + int(s) % B)
            assert locs == sorted(locs)              # ascending local position
            got += [int(oracle.global_id(r, l, S, I)) for l in locs]
        assert sorted(got) == sorted(int(v) for v in ids[i] if v >= 0)
    if S == 1:                                     # plain paged lookup
        for i in range(R):
            for j in range(counts[0, i]):
                g = ids[i, j]
                assert slots[0, i, j] == bt[0, i, g // B] * B + g % B


def test_convert_guards_rows_and_columns_outside_the_table():
    # a request outside the table keeps nothing; a block column past the
    # table width is dropped, the rest keep their order
    S, I, B = 1, 1, 4
    bt = np.array([[[7, 3]]], np.int32)            # one request, two blocks
    ids = np.array([[1, 6, 9, -1], [0, 1, 2, 3]], np.int32)
    slots, counts = oracle.convert_index(ids, np.array([0, 3], np.int32), bt, B, S, I)
    assert slots[0, 0].tolist() == [7 * 4 + 1, 3 * 4 + 2, -1, -1]   # id 9: column 2 >= 2
    assert counts[0].tolist() == [2, 0]
    assert slots[0, 1].tolist() == [-1, -1, -1, -1]
    slots, counts = oracle.convert_index(ids[:1], np.array([-1], np.int32), bt, B, S, I)
    assert counts[0].tolist() == [0]


# ---- planted mistakes ------------------------------------------------------
def test_planted_tie_break_mistake_is_caught(monkeypatch):
    def wrong_order(scores, ids):                 # ties by descending id
        s = np.asarray(scores, dtype=np.float64) + 0.0
        return np.lexsort((-np.asarray(ids), -s))
    monkeypatch.setattr(osel, "_rank_order", wrong_order)
    with pytest.raises(AssertionError):
        for seed in range(6):
            test_single_shard_vs_brute_force(seed)


def test_planted_signed_zero_mistake_is_caught(monkeypatch):
    def raw_bits_order(scores, ids):              # compares -0.0 below +0.0
        s = np.asarray(scores, dtype=np.float64)
        key = np.where(np.signbit(s) & (s == 0), -1e-300, s)
        return np.lexsort((np.asarray(ids), -key))
    monkeypatch.setattr(osel, "_rank_order", raw_bits_order)
    with pytest.raises(AssertionError):
        test_signed_zero_ties_break_by_position()


def test_planted_shard_offset_mistake_is_caught(monkeypatch):
    real = osel.global_id
    monkeypatch.setattr(osel, "global_id", lambda r, l, S, I: real(0, l, S, I))
    with pytest.raises(AssertionError):
        test_sharded_then_merged_equals_unsharded(4, 1, 0)
