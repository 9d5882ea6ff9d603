"""Pins for the oracle's indexer-key branch (materialise + fp8 indexer-cache
insert): torch's RMSNorm and a complex-number rotation as independent
formulations, the identity rotation at position 0, the unrotated half not
depending on the position, pair norms, the constant-row closed form, the
insert layout and skipped slots.  Planted mistakes must fail these pins."""
import numpy as np
import pytest
import torch

import dsa_inputs
import oracle
from oracle import prologue as opro
from oracle.formats import bf16_to_f64, f64_to_bf16

T = 6


def _inputs(seed=5):
    rng = np.random.default_rng(seed)
    k = dsa_inputs._draw_bf16_normal(rng, (T, 128), 1.0)
    w = f64_to_bf16(rng.uniform(0.5, 1.5, 128))
    cs = dsa_inputs._cos_sin_table(70000)
    pos = np.array([0, 1, 17, 1000, 65535, 4095], np.int32)
    return k, w, cs, pos


def _reference(k, w, eps, cs, pos):
    """torch RMSNorm (float64), then the rotary half as complex numbers."""
    x = torch.from_numpy(bf16_to_f64(k))
    y = torch.nn.functional.rms_norm(x, (128,), weight=torch.from_numpy(bf16_to_f64(w)),
                                     eps=eps).numpy()
    c = cs[pos, :32].astype(np.float64)
    s = cs[pos, 32:].astype(np.float64)
    z = (y[:, 64::2] + 1j * y[:, 65::2]) * (c + 1j * s)
    out = y.copy()
    out[:, 64::2] = z.real
    out[:, 65::2] = z.imag
    return out


def _ulps(a, b):
    def ordered(v):
        v = np.asarray(v, dtype=np.uint16).astype(np.int32)
        return np.where(v & 0x8000, 0x8000 - (v & 0x7FFF), 0x8000 + v)
    return np.abs(ordered(a) - ordered(b))


def test_matches_torch_rmsnorm_and_complex_rotation():
    k, w, cs, pos = _inputs()
    got = oracle.index_norm_rope(k, w, 1e-6, cs, pos)
    ref = f64_to_bf16(_reference(k, w, 1e-6, cs, pos))
    assert _ulps(got, ref).max() <= 1


def test_position_zero_is_the_plain_norm_and_unrotated_half_ignores_position():
    k, w, cs, pos = _inputs(6)
    at0 = oracle.index_norm_rope(k, w, 1e-6, cs, np.zeros(T, np.int32))
    x = bf16_to_f64(k)
    norm = x / np.sqrt((x * x).mean(1, keepdims=True) + 1e-6) * bf16_to_f64(w)[None, :]
    assert np.array_equal(at0, f64_to_bf16(norm))
    got = oracle.index_norm_rope(k, w, 1e-6, cs, pos)
    assert np.array_equal(got[:, :64], at0[:, :64])
    # rotation keeps each pair's norm: the rotated pairs, rounded once to bf16
    # (relative error <= 2^-9 per component), against the exact norms
    b = bf16_to_f64(got[:, 64:])
    exact = norm[:, 64::2] ** 2 + norm[:, 65::2] ** 2
    assert np.allclose(b[:, 0::2] ** 2 + b[:, 1::2] ** 2, exact, rtol=2 ** -7, atol=1e-6)
    assert not np.array_equal(got[1:, 64:], at0[1:, 64:])   # positions 1.. do rotate


def test_constant_rows_closed_form():
    c = np.array([0.25, -2.0, 3e-3])
    k = np.repeat(f64_to_bf16(c)[:, None], 128, axis=1)
    rng = np.random.default_rng(8)
    w = f64_to_bf16(rng.uniform(0.5, 1.5, 128))
    out = oracle.index_norm_rope(k, w, 1e-6, dsa_inputs._cos_sin_table(2), np.zeros(3, np.int32))
    cb = bf16_to_f64(f64_to_bf16(c))
    exp = bf16_to_f64(w)[None, :] * (cb / np.sqrt(cb * cb + 1e-6))[:, None]
    assert np.array_equal(out, f64_to_bf16(exp))


def test_index_cache_insert_layout_and_skip():
    k, w, cs, pos = _inputs(9)
    mat = oracle.index_norm_rope(k, w, 1e-6, cs, pos)
    cache = np.zeros((2, 64, 128), np.uint8)
    slots = np.array([3, -1, 64 + 63, 0, -5, 70], np.int64)
    scale = 2.0 ** -4
    out = oracle.index_cache_insert(cache, slots, mat, scale).reshape(-1, 128)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        exp = torch.from_numpy((bf16_to_f64(mat[t]) / scale).astype(np.float32)) \
            .to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(out[s], exp)
    touched = {int(s) for s in slots if s >= 0}
    assert all(np.all(out[s] == 0) for s in range(out.shape[0]) if s not in touched)


# ---- planted mistakes ------------------------------------------------------
def _planted(kind):
    def wrong(index_k, w, eps, cos_sin, positions):
        x = bf16_to_f64(index_k)
        wv = bf16_to_f64(w)
        width = 64 if kind == "norm over 64" else 128
        y = x / np.sqrt(np.mean(x[:, :width] ** 2, axis=1, keepdims=True) + eps) * wv[None, :]
        cs = np.asarray(cos_sin, np.float64)[np.asarray(positions, np.int64)]
        c, s = cs[:, :32], cs[:, 32:]
        if kind == "sin sign":
            s = -s
        lo = 0 if kind == "rope on the first half" else 64
        out = y.copy()
        x1, x2 = y[:, lo::2][:, :32], y[:, lo + 1::2][:, :32]
        out[:, lo:lo + 64:2] = x1 * c - x2 * s
        out[:, lo + 1:lo + 64:2] = x2 * c + x1 * s
        return f64_to_bf16(out)
    return wrong


@pytest.mark.parametrize("kind", ["norm over 64", "sin sign", "rope on the first half"])
def test_planted_indexer_mistakes_are_caught(monkeypatch, kind):
    monkeypatch.setattr(oracle, "index_norm_rope", _planted(kind))
    failed = 0
    for pin in (test_matches_torch_rmsnorm_and_complex_rotation,
                test_position_zero_is_the_plain_norm_and_unrotated_half_ignores_position):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed, f"planted mistake '{kind}' passed every pin"
