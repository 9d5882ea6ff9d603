"""Index maps of the interleaved context sharding (oracle, test-only).

PR #46076 report, section 关键源码片段 (key source excerpts), the metadata
helper ``_dcp_localize_decode_seq_lens``: a rank owns the tokens whose
``(pos // interleave) % world`` equals its rank, and global sequence lengths
become per-rank local lengths.  The long-context workload states the same rule
for 8 shards, interleave 64: token t sits on shard ``(t // 64) % 8`` at local
position ``(t // 512) * 64 + t % 64``.

With S shards and interleave I, a "round" of I*S consecutive tokens gives I
tokens to every shard; a shard keeps its tokens in global order.
"""
from __future__ import annotations

import numpy as np


def owner(t, S, I):
    """Shard that holds global token ``t``."""
    return (np.asarray(t) // I) % S


def local(t, S, I):
    """Position of global token ``t`` inside its owner's local sequence:
    full rounds before it contribute I each, plus its offset in its run."""
    t = np.asarray(t)
    return (t // (I * S)) * I + t % I


def global_id(r, l, S, I):
    """Inverse of (owner, local): the global token at local position ``l`` of
    shard ``r`` — run ``l // I`` of the shard lies in round ``l // I``."""
    l = np.asarray(l)
    return ((l // I) * S + r) * I + l % I


def local_count(n, r, S, I):
    """How many of the global tokens ``0 .. n-1`` shard ``r`` holds: I per
    full round, plus the part of the last, partial round that falls in the
    shard's run ``[r*I, (r+1)*I)``."""
    n = np.asarray(n, dtype=np.int64)
    rem = n % (I * S)
    return (n // (I * S)) * I + np.minimum(np.maximum(rem - r * I, 0), I)
