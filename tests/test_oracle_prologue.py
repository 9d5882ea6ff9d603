"""Pins for the oracle's formats and the RMSNorm + RoPE prologue: the OCP
e4m3 definition (spot values and all 256 codes against torch's float8 type),
correctly-rounded bf16 against torch's cast, RoPE identities and the RMSNorm
closed form on constant rows."""
import numpy as np
import pytest
import torch

import oracle
from oracle import formats as fmt
from oracle.formats import bf16_to_f64, f64_to_bf16, e4m3_to_f64, f64_to_e4m3
import dsa_inputs


# ---------------------------------------------------------------- e4m3 ----
def test_e4m3_spec_values():
    # values fixed by the OCP FP8 definition of E4M3 (bias 7, no inf)
    assert e4m3_to_f64(0x00) == 0.0
    assert e4m3_to_f64(0x01) == 2.0 ** -9          # smallest subnormal
    assert e4m3_to_f64(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert e4m3_to_f64(0x08) == 2.0 ** -6          # smallest normal
    assert e4m3_to_f64(0x38) == 1.0
    assert e4m3_to_f64(0x7E) == 448.0              # largest finite
    assert np.isnan(e4m3_to_f64(0x7F)) and np.isnan(e4m3_to_f64(0xFF))
    assert e4m3_to_f64(0xB8) == -1.0
    assert e4m3_to_f64(0x80) == 0.0 and np.signbit(e4m3_to_f64(0x80))


def test_e4m3_table_vs_torch_all_codes():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3_to_f64(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])


def test_e4m3_encode_vs_torch_including_midpoints():
    vals = fmt._POS_VALS
    mids = (vals[:-1] + vals[1:]) / 2
    xs = np.concatenate([vals, mids, mids * (1 + 1e-6), mids * (1 - 1e-6),
                         np.linspace(-440, 440, 20001)])
    xs = np.concatenate([xs, -xs]).astype(np.float32)      # exactly fp32
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = f64_to_e4m3(xs.astype(np.float64))
    assert np.array_equal(ref, ours)


def test_e4m3_round_trip_and_saturation():
    c = np.array([k for k in range(256) if (k & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(f64_to_e4m3(e4m3_to_f64(c)), c)
    assert f64_to_e4m3(np.array([1000.0]))[0] == 0x7E
    assert f64_to_e4m3(np.array([-1000.0]))[0] == 0xFE


# ---------------------------------------------------------------- bf16 ----
def test_bf16_round_vs_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-5, 5, 100000),
                        [1.0, -2.5, 3.0e-3]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f64_to_bf16(x.astype(np.float64)), ref)


def test_bf16_exact_midpoints_and_double_rounding():
    # 1 + 2^-8 is halfway between bf16 1.0 and 1+2^-7 -> even (1.0)
    assert bf16_to_f64(f64_to_bf16(np.array([1 + 2.0 ** -8])))[0] == 1.0
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6 -> even (1+2^-6)
    assert bf16_to_f64(f64_to_bf16(np.array([1 + 3 * 2.0 ** -8])))[0] == 1 + 2.0 ** -6
    # just above a midpoint in float64 (below fp32 resolution) must round up;
    # a detour through fp32 would land on the midpoint and round to even
    x = 1 + 2.0 ** -8 + 2.0 ** -40
    assert bf16_to_f64(f64_to_bf16(np.array([x])))[0] == 1 + 2.0 ** -7
    # a mantissa carry into the exponent
    assert bf16_to_f64(f64_to_bf16(np.array([2.0 - 2.0 ** -9])))[0] == 2.0
    assert f64_to_bf16(np.array([-0.0]))[0] == 0x8000


# ----------------------------------------------------------- prologue ----
def _bf16(x):
    return f64_to_bf16(np.asarray(x, dtype=np.float64))


def test_rope_position_zero_is_identity_and_preserves_pair_norms():
    rng = np.random.default_rng(1)
    T = 5
    kv = dsa_inputs._draw_bf16_normal(rng, (T, 512), 1.0)
    pe = dsa_inputs._draw_bf16_normal(rng, (T, 64), 1.0)
    w = _bf16(np.ones(512))
    cs = dsa_inputs._cos_sin_table(4096)
    _, pe0 = oracle.rmsnorm_rope(kv, pe, w, 1e-6, cs, np.zeros(T, np.int32))
    assert np.array_equal(pe0, pe)
    pos = np.array([1, 17, 1000, 4095, 2048], np.int32)
    _, per = oracle.rmsnorm_rope(kv, pe, w, 1e-6, cs, pos)
    a, b = bf16_to_f64(pe), bf16_to_f64(per)
    n0 = a[:, 0::2] ** 2 + a[:, 1::2] ** 2
    n1 = b[:, 0::2] ** 2 + b[:, 1::2] ** 2
    assert np.allclose(n0, n1, rtol=2 ** -7)
    # the first pair rotates by angle pos * 1 (frequency 1 for i = 0)
    ang = pos.astype(np.float64)
    r1 = a[:, 0] * np.cos(ang) - a[:, 1] * np.sin(ang)
    assert np.allclose(b[:, 0], r1, rtol=2 ** -7, atol=1e-6)


def test_rmsnorm_constant_rows_closed_form():
    c = np.array([0.5, -3.0, 1e-3], dtype=np.float64)
    kv = np.repeat(_bf16(c)[:, None], 512, axis=1)
    rng = np.random.default_rng(2)
    w = _bf16(rng.uniform(0.5, 1.5, 512))
    pe = _bf16(np.zeros((3, 64)))
    eps = 1e-6
    out, _ = oracle.rmsnorm_rope(kv, pe, w, eps, dsa_inputs._cos_sin_table(2), np.zeros(3, np.int32))
    cb = bf16_to_f64(_bf16(c))
    exp = bf16_to_f64(w)[None, :] * (cb / np.sqrt(cb * cb + eps))[:, None]
    assert np.array_equal(out, f64_to_bf16(exp))


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8"])
def test_insert_layout_and_skip(cache_dtype):
    rng = np.random.default_rng(3)
    T = 4
    kv_out = dsa_inputs._draw_bf16_normal(rng, (T, 512), 1.0)
    pe_out = dsa_inputs._draw_bf16_normal(rng, (T, 64), 1.0)
    dt = np.uint8 if cache_dtype == "fp8" else np.uint16
    cache = np.zeros((2, 64, 576), dtype=dt)
    slots = np.array([5, -1, 64 + 63, 0], np.int64)
    scale = 2.0 ** -4
    out = oracle.cache_insert(cache, slots, kv_out, pe_out, cache_dtype, scale)
    flat = out.reshape(-1, 576)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        entry = np.concatenate([kv_out[t], pe_out[t]])
        if cache_dtype == "fp8":
            # x / scale then e4m3; for a power-of-two scale the division is exact
            exp = torch.from_numpy((bf16_to_f64(entry) / scale).astype(np.float32)) \
                .to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(flat[s], exp)
        else:
            assert np.array_equal(flat[s], entry)
    touched = {int(s) for s in slots if s >= 0}
    for s in range(flat.shape[0]):
        if s not in touched:
            assert np.all(flat[s] == 0)


# ------------------------------------------------------- RoPE table ----
# The table is an input that both sides receive, so parity alone cannot see a
# wrong frequency in it.  It is pinned from the definition instead: with base
# 10000 over 64 rotary dimensions pair i turns by 10000^(-2i/64) = 10^(-i/8)
# radians per position, so pairs 8, 16 and 24 turn by exactly 0.1, 0.01 and
# 0.001, and positions 10, 100 and 1000 put each of them at an angle of one
# radian; pair 0 turns by one radian per position for any base.
def _check_rope_table(cs):
    c1, s1 = np.float32(np.cos(1.0)), np.float32(np.sin(1.0))
    assert cs.shape[1] == 64 and cs.dtype == np.float32
    for pos, pair in ((1, 0), (10, 8), (100, 16), (1000, 24)):
        assert cs[pos, pair] == c1, f"cos of pair {pair} at position {pos}"
        assert cs[pos, 32 + pair] == s1, f"sin of pair {pair} at position {pos}"
    # position 0 is the identity rotation for every pair
    assert np.all(cs[0, :32] == 1.0) and np.all(cs[0, 32:] == 0.0)


def test_rope_table_frequencies_from_the_definition():
    _check_rope_table(dsa_inputs._cos_sin_table(1001))


def test_rope_table_of_the_fp8_workload():
    c = dsa_inputs.make(dsa_inputs.spec("fp8_s"), with_cache=False)
    _check_rope_table(c.cos_sin)
    assert c.cos_sin.shape[0] == c.ctx          # one row per context position


def _planted_table(n_pos, inv_freq):
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


@pytest.mark.parametrize("what,inv_freq", [
    ("base 1000", 1000.0 ** (-2.0 * np.arange(32) / 64)),
    ("exponent -i/64", 10000.0 ** (-1.0 * np.arange(32) / 64)),
    ("pairs shifted by one", 10000.0 ** (-2.0 * (np.arange(32) + 1) / 64)),
])
def test_planted_rope_table_mistakes_are_caught(what, inv_freq):
    with pytest.raises(AssertionError):
        _check_rope_table(_planted_table(1001, inv_freq))
