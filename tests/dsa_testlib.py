"""Shared test helpers: moving generated inputs to the GPU, running the
oracle on the same inputs, and the comparison tolerances.

Tolerances (the DSA path's stated bar, plus a relative term that gives the
absolute bound power on nearly-uniform attention):
* indices, candidates, merged ids, slots, counts, inserted fp8 bytes: exact;
* attention outputs: max |gpu - oracle| <= 1e-2 and, per (part, row, head),
  ||gpu - oracle||_2 <= 1e-2 * ||oracle||_2;
* LSE: |gpu - oracle| <= 1e-3 (both -inf for empty partials);
* materialised bf16 rows: within 1 bf16 ulp of the correctly rounded value.
"""
from __future__ import annotations

import numpy as np

OUT_ABS = 1e-2
OUT_REL_L2 = 1e-2
LSE_ABS = 1e-3


def bf16_bits_to_f64(t_bits: np.ndarray) -> np.ndarray:
    return (np.asarray(t_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def attn_mismatch(gpu_out, ref_out, gpu_lse, ref_lse):
    """Returns a list of human-readable violations (empty when in tolerance).
    ``*_out``: [..., heads, 512]; ``*_lse``: [..., heads]."""
    bad = []
    g = np.asarray(gpu_out, dtype=np.float64)
    r = np.asarray(ref_out, dtype=np.float64)
    if not np.all(np.isfinite(g)):
        bad.append("non-finite output")
        return bad
    err = np.abs(g - r)
    if err.max() > OUT_ABS:
        bad.append(f"max abs err {err.max():.3e} > {OUT_ABS}")
    num = np.sqrt(((g - r) ** 2).sum(-1))
    den = np.sqrt((r ** 2).sum(-1))
    rel = np.where(den > 0, num / np.where(den > 0, den, 1), num)
    if rel.max() > OUT_REL_L2:
        bad.append(f"max rel l2 err {rel.max():.3e} > {OUT_REL_L2}")
    gl = np.asarray(gpu_lse, dtype=np.float64)
    rl = np.asarray(ref_lse, dtype=np.float64)
    inf_g, inf_r = np.isneginf(gl), np.isneginf(rl)
    if not np.array_equal(inf_g, inf_r):
        bad.append(f"-inf lse pattern differs ({inf_g.sum()} vs {inf_r.sum()})")
    fin = ~inf_r & ~inf_g
    if fin.any():
        le = np.abs(gl[fin] - rl[fin]).max()
        if le > LSE_ABS:
            bad.append(f"max lse err {le:.3e} > {LSE_ABS}")
    return bad


def bf16_ulp_diff(a_bits, b_bits) -> np.ndarray:
    """Distance in bf16 ulps between two bf16 bit arrays (same sign assumed
    near zero handled through the ordered integer map)."""
    def ordered(x):
        x = np.asarray(x, dtype=np.uint16).astype(np.int32)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + x)
    return np.abs(ordered(a_bits) - ordered(b_bits))
