"""Sparse MLA partial attention and LSE combine (oracle, test-only).

Sources:
* PR #52046 report, 关键源码片段: the layer calls ``forward_mqa`` to get
  ``(attn_out, lse)`` from the latent cache, returns zeros when there are no
  tokens, and merges the per-shard partials with ``dcp_manager.combine``.
* PR #52046 report, same section, the fused kernel's cache write: a latent
  cache entry is the normalised ``kv_c`` (512) followed by the roped ``k_pe``
  (64); attention reads all 576 as the key and the first 512 as the value
  (multi-query latent attention: every head shares the entry).
* PR #46076 report, 实现拆解 item 5 and 评论区精华 (review) "LSE 基数归一化":
  the backend's LSE is base 2 and is multiplied by ln 2 before the DCP
  reducer, which expects base e.  The oracle computes base e directly.

Numbers: keys and values are decoded exactly (bf16, or e4m3 code x fp32
scale), everything else is float64.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64, e4m3_to_f64

D_LATENT = 576
D_V = 512


def decode_rows(cache, cache_dtype, scale, slots):
    """Latent rows at ``slots`` as float64 ``[n][576]``."""
    flat = cache.reshape(-1, D_LATENT)
    rows = flat[np.asarray(slots, dtype=np.int64)]
    if cache_dtype == "fp8":
        return e4m3_to_f64(rows) * np.float64(scale)
    return bf16_to_f64(rows)


def _attend(qh: np.ndarray, K: np.ndarray, sm_scale: float):
    """softmax(sm_scale * q K^T) V with V = K[:, :512]; returns (out, lse).

    lse = M + ln(sum_j exp(s_j - M)), M = max_j s_j."""
    s = (qh @ K.T) * np.float64(sm_scale)                 # [H][c]
    M = s.max(axis=1, keepdims=True)
    e = np.exp(s - M)
    z = e.sum(axis=1, keepdims=True)
    lse = (M + np.log(z))[:, 0]
    out = (e / z) @ K[:, :D_V]
    return out, lse


def sparse_mla_partial(q, cache, cache_dtype, scale, slots, counts, sm_scale):
    """Per-shard partial attention over each row's compacted slot list.

    ``q``: ``[R][H][576]`` bf16 bits; ``slots``: ``[P][R][k]``; ``counts``:
    ``[P][R]``.  Returns ``out [P][R][H][512]`` and ``lse [P][R][H]`` (float64).
    A shard with no selected tokens yields out = 0 and lse = -inf (it still
    emits a partial, as every rank must join the combine — PR #40996 report,
    评论区精华 item 1, rank-invariant collective gating).
    """
    P, R, _ = slots.shape
    H = q.shape[1]
    out = np.zeros((P, R, H, D_V), dtype=np.float64)
    lse = np.full((P, R, H), -np.inf, dtype=np.float64)
    for p in range(P):
        for i in range(R):
            c = int(counts[p, i])
            if c == 0:
                continue
            K = decode_rows(cache, cache_dtype, scale, slots[p, i, :c])
            out[p, i], lse[p, i] = _attend(bf16_to_f64(q[i]), K, sm_scale)
    return out, lse


def attention_over_ids(q_row, cache, cache_dtype, scale, slot_list, sm_scale):
    """Unsharded attention of one row over an explicit slot list."""
    K = decode_rows(cache, cache_dtype, scale, slot_list)
    return _attend(bf16_to_f64(q_row), K, sm_scale)


def lse_combine(part_out, part_lse):
    """LSE-weighted merge of per-shard partials (the DCP reducer).

    lse = ln sum_r exp(lse_r) over the finite partials (-inf if none);
    out = sum_r exp(lse_r - lse) * out_r (0 if none)."""
    part_lse = np.asarray(part_lse, dtype=np.float64)
    M = np.max(part_lse, axis=0)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    w = np.exp(part_lse - Ms[None])                       # exp(-inf) = 0
    z = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(finite, Ms + np.log(np.where(finite, z, 1.0)), -np.inf)
    wn = np.where(finite[None], w / np.where(finite, z, 1.0)[None], 0.0)
    out = np.einsum("prh,prhd->rhd", wn, np.asarray(part_out, dtype=np.float64))
    return out, lse
