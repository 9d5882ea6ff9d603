"""bf16 and fp8 e4m3 storage formats, written from their definitions
(oracle, test-only).

* bf16: the upper 16 bits of an IEEE-754 binary32 (1 sign, 8 exponent,
  7 fraction bits).  Rounding is to nearest, ties to even, done here directly
  from float64 so there is no intermediate rounding.
* e4m3 ("fn" variant of the OCP 8-bit floating point specification): 1 sign,
  4 exponent bits with bias 7, 3 fraction bits; exponent field 0 encodes
  subnormals ``m/8 * 2^-6``; there are no infinities; the all-ones code
  (S.1111.111) is NaN; the largest finite magnitude is 1.75 * 2^8 = 448.
  Encoding rounds to nearest, ties to the even code, and saturates finite
  values beyond 448 (the plainest reading of a cache-writing cast; never
  reached by the workloads here).
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------- bf16 ----
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 to bf16 bits, nearest-even, without double rounding.

    Works on the float64 bit pattern: keep the sign, the 11-bit exponent and
    the top 7 fraction bits, rounding the 45 dropped bits; then re-bias the
    exponent from 1023 to 127.  Handles zeros, normals of bf16 range and
    saturates nothing (inputs here are far inside the range)."""
    x = np.asarray(x, dtype=np.float64)
    u = x.view(np.uint64)
    sign = (u >> np.uint64(63)).astype(np.uint32)
    mag = u & np.uint64(0x7FFFFFFFFFFFFFFF)
    keep = mag >> np.uint64(45)
    drop = mag & np.uint64((1 << 45) - 1)
    half = np.uint64(1 << 44)
    up = (drop > half) | ((drop == half) & ((keep & np.uint64(1)) == np.uint64(1)))
    keep = keep + up.astype(np.uint64)           # carries into the exponent
    exp64 = (keep >> np.uint64(7)).astype(np.int64)
    frac = (keep & np.uint64(0x7F)).astype(np.uint32)
    exp16 = exp64 - 1023 + 127
    is_zero = mag == 0
    if np.any(~is_zero & ((exp16 <= 0) | (exp16 >= 255))):
        raise ValueError("value outside the normal bf16 range")
    out = (sign << np.uint32(15)) | (np.clip(exp16, 0, 255).astype(np.uint32) << np.uint32(7)) | frac
    out = np.where(is_zero, sign << np.uint32(15), out)
    return out.astype(np.uint16)


# ---------------------------------------------------------------- e4m3 ----
def _e4m3_table() -> np.ndarray:
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * (m / 8.0) * 2.0 ** -6
        else:
            vals[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3 = _e4m3_table()
E4M3_MAX = 448.0
# non-negative finite codes 0x00 .. 0x7E in increasing value order
_POS_CODES = np.arange(0x7F)
_POS_VALS = E4M3[_POS_CODES]


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    return E4M3[np.asarray(codes, dtype=np.uint8)]


def f64_to_e4m3(x: np.ndarray) -> np.ndarray:
    """Nearest e4m3 code, ties to even code, sign kept (also for zero)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS_VALS, a, side="left")      # first value >= a
    hi = np.clip(hi, 0, len(_POS_VALS) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALS) - 1)
    dlo = a - _POS_VALS[lo]
    dhi = _POS_VALS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((_POS_CODES[hi] & 1) == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)
    code = np.where(np.isnan(x), np.uint8(0x7F), code)
    return code.astype(np.uint8)
