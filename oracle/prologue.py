"""Fused RMSNorm + RoPE prologue and latent-cache insert (oracle, test-only).

PR #52046 report, 实现拆解 item 1 and 关键源码片段 (``_fused_norm_rope_kernel``,
branch ``pid == 1``):

* ``kv_c`` (512 wide) goes through RMSNorm with weight ``w`` and epsilon;
* ``k_pe`` (64 wide) is rotated in interleaved pairs: for pair i the inputs
  are elements 2i and 2i+1, ``r1 = x1*cos - x2*sin``, ``r2 = x2*cos + x1*sin``,
  stored back at 2i and 2i+1;
* when output buffers are given the results are materialised (bf16);
* when a slot mapping is given the entry at that slot becomes
  ``[kv_c (512) | k_pe (64)]``; for an fp8 cache each value is divided by the
  per-tensor scale and cast to e4m3.

Readings taken where the page is silent:
* RMSNorm is ``y = x / sqrt(mean(x^2) + eps) * w`` with a plain multiplicative
  weight, evaluated exactly and rounded once to bf16;
* the RoPE table row for position p is ``[cos(p*f_0..f_31) | sin(...)]``
  (the usual cos/sin cache layout), supplied as an fp32 input;
* "materialised then inserted": the insert quantises the materialised bf16
  values, so an fp8 entry is ``e4m3(bf16(v) / scale)``;
* slots < 0 are skipped (padding of a slot mapping).
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64, f64_to_bf16, f64_to_e4m3

D_V = 512
D_ROPE = 64
D_INDEX = 128


def rmsnorm_rope(kv_c, k_pe, w, eps, cos_sin, positions):
    """Returns ``(kv_c_out, k_pe_out)`` as bf16 bits, ``[T][512]`` and ``[T][64]``."""
    x = bf16_to_f64(kv_c)                                      # [T][512]
    wv = bf16_to_f64(w)
    inv_rms = 1.0 / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + np.float64(eps))
    y = x * inv_rms * wv[None, :]
    kv_out = f64_to_bf16(y)

    pe = bf16_to_f64(k_pe)                                     # [T][64]
    cs = np.asarray(cos_sin, dtype=np.float64)[np.asarray(positions, dtype=np.int64)]
    c, s = cs[:, :D_ROPE // 2], cs[:, D_ROPE // 2:]
    x1, x2 = pe[:, 0::2], pe[:, 1::2]
    r = np.empty_like(pe)
    r[:, 0::2] = x1 * c - x2 * s
    r[:, 1::2] = x2 * c + x1 * s
    return kv_out, f64_to_bf16(r)


def cache_insert(cache, slot_mapping, kv_c_out, k_pe_out, cache_dtype, scale):
    """Write the materialised rows into a copy of the cache at their slots."""
    out = cache.copy()
    flat = out.reshape(-1, D_V + D_ROPE)
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        entry = np.concatenate([kv_c_out[t], k_pe_out[t]])
        if cache_dtype == "fp8":
            flat[slot] = f64_to_e4m3(bf16_to_f64(entry) / np.float64(scale))
        else:
            flat[slot] = entry
    return out


# ---------------------------------------------------------------------------
# Indexer-key branch (pid == 0 of the same fused kernel).
#
# PR #52046 report, 实现拆解 item 1: the indexer-K branch materialises the
# indexer key into ``index_k_out`` when that output is given, and quantises it
# to FP8 and writes it into the indexer cache only when both the indexer cache
# and the slot mapping are given.  The pages do not print this branch's
# arithmetic; readings taken (the plainest ones the page's other branch
# supports):
# * the key is 128 wide: 64 unrotated dimensions followed by a 64-dimension
#   rotary part (the order of the latent entry, kv_c before k_pe);
# * "norm" is the kernel's only norm, RMSNorm, over all 128 dimensions with
#   the branch's own multiplicative weight and epsilon; RoPE rotates the
#   normalised rotary part in interleaved pairs with the same cos/sin table
#   and position as the latent branch; evaluated exactly, rounded once to
#   bf16;
# * FP8 quantisation is the page's quant of the latent branch, e4m3(value /
#   scale) with a per-tensor scale, applied to the materialised bf16 values.

def index_norm_rope(index_k, w, eps, cos_sin, positions):
    """Returns the materialised indexer keys as bf16 bits, ``[T][128]``."""
    x = bf16_to_f64(index_k)                                   # [T][128]
    wv = bf16_to_f64(w)
    y = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + np.float64(eps)) * wv[None, :]
    cs = np.asarray(cos_sin, dtype=np.float64)[np.asarray(positions, dtype=np.int64)]
    c, s = cs[:, :D_ROPE // 2], cs[:, D_ROPE // 2:]
    nope = D_INDEX - D_ROPE
    x1, x2 = y[:, nope::2], y[:, nope + 1::2]
    out = y.copy()
    out[:, nope::2] = x1 * c - x2 * s
    out[:, nope + 1::2] = x2 * c + x1 * s
    return f64_to_bf16(out)


def index_cache_insert(cache, slot_mapping, index_k_out, scale):
    """Write the materialised indexer keys into a copy of the fp8 indexer
    cache ``[...][128]`` at their slots (slots < 0 are skipped)."""
    out = cache.copy()
    flat = out.reshape(-1, D_INDEX)
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        flat[slot] = f64_to_e4m3(bf16_to_f64(index_k_out[t]) / np.float64(scale))
    return out
