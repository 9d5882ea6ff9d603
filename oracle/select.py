"""Top-K selection, candidate merge and index conversion (oracle, test-only).

Total order used throughout.  Candidate a precedes candidate b when its score
is numerically larger, or when the scores are equal and a's global token id
is smaller (the ascending-global-id tie-break of the DSA path).  -0.0 and
+0.0 are equal scores.  A NaN score ranks after every number (never produced
by the workloads).  Inside one shard, local order equals global-id order
because ``global_id(r, .)`` is increasing, so "ascending position" and
"ascending global id" are the same tie-break there.

Output order (the pages leave it open): selected entries first, in ascending
local position / global id, then -1 padding.
"""
from __future__ import annotations

import numpy as np

from .maps import owner, local, global_id, local_count


def _rank_order(scores: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Indices sorting candidates by the total order (best first)."""
    s = np.asarray(scores, dtype=np.float64) + 0.0        # -0.0 -> +0.0
    return np.lexsort((np.asarray(ids), -s))             # NaN sorts last


def unsharded_topk(row_logits: np.ndarray, lo: int, hi: int, k: int) -> np.ndarray:
    """Top-k global ids of one unsharded row restricted to [lo, hi), in
    ascending id order (no padding)."""
    pos = np.arange(lo, hi)
    order = _rank_order(row_logits[lo:hi], pos)
    return np.sort(pos[order[:min(k, hi - lo)]])


def topk_select(logits, row_starts, row_ends, ctx, k, S, I, first=0, count=None):
    """Per-shard stable top-K with fused (score, global_id) packing.

    PR #46076 report, 关键源码片段 (key source excerpts), ``_merge_dcp_topk_global``:
    each rank holds the top-K positions of its local KV shard; the pack step
    turns every one into a ``(score, global_id)`` pair of a float32
    ``[batch, topk, 2]`` buffer; the all-gather along dim 1 puts rank r's k
    pairs at columns ``[r*k, (r+1)*k)``; -1 marks padding.  Row bounds are
    global (``row_starts``/``row_ends``) and are localised per shard with
    ``local_count`` (the ownership rule of ``_dcp_localize_decode_seq_lens``).

    ``logits``: ``[count][R][ld]`` — slice j holds shard ``first + j``.
    Returns ``local_idx [count][R][k]`` int32 and ``cand [R][S*k][2]`` float32
    (columns of shards outside the processed range stay as padding).
    Padding entries are ``local_idx = -1`` and ``cand = (-inf, -1.0)``.
    """
    count = S - first if count is None else count
    R = logits.shape[1]
    local_idx = np.full((count, R, k), -1, dtype=np.int32)
    cand = np.empty((R, S * k, 2), dtype=np.float32)
    cand[..., 0] = -np.inf
    cand[..., 1] = -1.0
    for j in range(count):
        r = first + j
        for i in range(R):
            lo = int(local_count(row_starts[i], r, S, I))
            hi = int(min(local_count(row_ends[i], r, S, I), local_count(ctx, r, S, I)))
            if hi <= lo:
                continue
            pos = np.arange(lo, hi)
            order = _rank_order(logits[j, i, lo:hi], pos)
            sel = np.sort(pos[order[:min(k, hi - lo)]])
            m = len(sel)
            local_idx[j, i, :m] = sel
            cand[i, r * k:r * k + m, 0] = logits[j, i, sel]          # a copy
            cand[i, r * k:r * k + m, 1] = global_id(r, sel, S, I).astype(np.float32)
    return local_idx, cand


def merge_candidates(cand, k):
    """Stable global top-K over gathered candidates.

    PR #46076 report, 实现拆解 (implementation) item 1 and the selector call in
    ``_merge_dcp_topk_global``: from all ranks' ``(score, global_id)`` pairs
    choose the global top-K token ids; padding (id < 0) never wins.  Output
    ``ids [R][k]`` int32: ascending global id, then -1.
    """
    R, N, _ = cand.shape
    ids_out = np.full((R, k), -1, dtype=np.int32)
    for i in range(R):
        sc = cand[i, :, 0].astype(np.float64)
        gid = cand[i, :, 1].astype(np.float64)
        valid = gid >= 0
        sc, gid = sc[valid], gid[valid].astype(np.int64)
        order = _rank_order(sc, gid)
        sel = np.sort(gid[order[:min(k, len(gid))]])
        ids_out[i, :len(sel)] = sel
    return ids_out


def convert_index(ids, row_req, block_table, block_size, S, I, first=0, count=None):
    """Global token ids -> per-shard physical cache slots, compacted.

    PR #46076 report, 实现拆解 item 4 (``_convert_req_index_to_global_index_kernel``
    with ``DCP_SIZE/DCP_RANK/DCP_INTERLEAVE`` and ``COMPACT_TO_FRONT``): a
    rank keeps only the ids it owns, de-interleaves each to its local
    position, looks the position up in its block table, and packs the valid
    slots at the front with -1 after them.  Compaction keeps input order (the
    page allocates with an atomic counter, whose order varies run to run; the
    input order is one of its outcomes).

    ``block_table``: ``[count][Rq][W]`` (slice j = shard ``first + j``);
    ``row_req``: request of each row (None = identity).
    Returns ``slots [count][R][k]`` int32, ``counts [count][R]`` int32.

    Outside the pages' domain (a reading, not a statement of the pages: the
    page's kernel is handed a table that covers every id it sees): a row
    whose request is outside ``[0, Rq)`` keeps nothing, and an id whose block
    column is ``>= W`` is dropped.  Inside the domain neither rule changes a
    result.
    """
    count = S - first if count is None else count
    R, k = ids.shape
    slots = np.full((count, R, k), -1, dtype=np.int32)
    counts = np.zeros((count, R), dtype=np.int32)
    n_req, width = block_table.shape[1], block_table.shape[2]
    for j in range(count):
        r = first + j
        for i in range(R):
            req = i if row_req is None else int(row_req[i])
            out = []
            if not 0 <= req < n_req:       # no such request: nothing to look up
                continue
            for g in ids[i]:
                g = int(g)
                if g < 0 or int(owner(g, S, I)) != r:
                    continue
                l = int(local(g, S, I))
                if l // block_size >= width:  # beyond the table: not a cached token
                    continue
                blk = int(block_table[j, req, l // block_size])
                out.append(blk * block_size + l % block_size)
            slots[j, i, :len(out)] = out
            counts[j, i] = len(out)
    return slots, counts
