"""Multi-token decode inputs: per-token lengths are expanded globally, then
localised per shard (PR #46076 report, 评论区精华: the DCP decode length
localisation order fix — expanding per token after localising the request
length gives [3, 4, 5] instead of the right [4, 4, 5] for world 2, rank 1).
"""
import numpy as np

import dsa_inputs
import oracle


def test_mtp_rows_share_their_request_table_and_expand_lengths():
    c = dsa_inputs.make("mtp_s", with_cache=False)
    q_len = c.spec.q_len
    assert q_len == 3 and c.rows == 9
    assert c.row_req.tolist() == [0, 0, 0, 1, 1, 1, 2, 2, 2]
    assert c.block_table.shape[1] == c.rows // q_len          # one table per request
    ends = c.row_ends.reshape(-1, q_len)
    assert np.all(np.diff(ends, axis=1) == 1)                  # consecutive query tokens
    assert ends[0, -1] == c.ctx                                # the first request is full


def test_mtp_localisation_reproduces_the_pages_example():
    # three query tokens of one request whose global length is 10, world 2,
    # rank 1: the expanded global lengths [8, 9, 10] localise to [4, 4, 5]
    sp = dsa_inputs.Spec("mtp_example", rows=3, ctx=10, shards=2, interleave=1, k=512,
                         heads=16, seed=0, q_len=3)
    c = dsa_inputs.make(sp, with_cache=False)
    assert c.row_ends.tolist() == [8, 9, 10]
    local = [int(oracle.local_count(int(e), 1, 2, 1)) for e in c.row_ends]
    assert local == [4, 4, 5]
    # localising the request length first and then expanding is the mistake
    # the page fixes
    wrong = [int(oracle.local_count(10, 1, 2, 1)) - (2 - j) for j in range(3)]
    assert wrong == [3, 4, 5] and wrong != local
