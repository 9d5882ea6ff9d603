"""Pins for the oracle's sparse MLA partial attention and LSE combine:
an independent library formulation (torch scaled_dot_product_attention and
logsumexp in float64), closed-form special cases, the base-2 / base-e LSE
identity, and combine(shard partials) == attention over the union."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt
from oracle.formats import bf16_to_f64
import dsa_inputs


def _rand_case(seed, H=8, n=50, std=1.0, nslots=300):
    rng = np.random.default_rng(seed)
    cache = dsa_inputs._draw_bf16_normal(rng, (nslots // 64 + 1, 64, 576), std)
    q = dsa_inputs._draw_bf16_normal(rng, (1, H, 576), 1.0)
    slots = rng.choice(cache.shape[0] * 64, n, replace=False).astype(np.int32)
    return q, cache, slots


@pytest.mark.parametrize("seed,std", [(0, 1.0), (1, 1 / 24), (2, 0.3)])
def test_matches_torch_sdpa_fp64(seed, std):
    q, cache, slots = _rand_case(seed, std=std)
    sm = float(np.float32(1 / 24))
    out, lse = oracle.attention_over_ids(q[0], cache, "bf16", 1.0, slots, sm)
    Q = torch.from_numpy(bf16_to_f64(q[0]))[None]                 # [1][H][576]
    K = torch.from_numpy(bf16_to_f64(cache.reshape(-1, 576)[slots]))[None, None]
    V = K[..., :512]
    H = Q.shape[1]
    ref = torch.nn.functional.scaled_dot_product_attention(
        Q.reshape(1, H, 1, 576), K.expand(1, H, -1, -1), V.expand(1, H, -1, -1), scale=sm)
    ref = ref.reshape(-1, 512).numpy()
    ref_lse = torch.logsumexp(sm * (Q[0] @ K[0, 0].T), dim=-1).numpy()
    assert np.max(np.abs(out - ref)) < 1e-12
    assert np.max(np.abs(lse - ref_lse)) < 1e-12


def test_single_token_closed_form():
    q, cache, slots = _rand_case(3, n=1)
    sm = 0.05
    out, lse = oracle.attention_over_ids(q[0], cache, "bf16", 1.0, slots, sm)
    K = bf16_to_f64(cache.reshape(-1, 576)[slots])
    assert np.allclose(out, np.broadcast_to(K[0, :512], out.shape), atol=0, rtol=0)
    assert np.allclose(lse, sm * (bf16_to_f64(q[0]) @ K[0]), rtol=1e-15, atol=1e-15)


def test_identical_keys_closed_form():
    q, cache, slots = _rand_case(4, n=1)
    c = 37
    flat = cache.reshape(-1, 576).copy()
    flat[:c] = flat[slots[0]]
    cache2 = flat.reshape(cache.shape)
    sm = 0.1
    out, lse = oracle.attention_over_ids(q[0], cache2, "bf16", 1.0, np.arange(c), sm)
    K0 = bf16_to_f64(flat[0])
    s0 = sm * (bf16_to_f64(q[0]) @ K0)
    assert np.allclose(lse, s0 + math.log(c), rtol=0, atol=1e-12)
    assert np.allclose(out, np.broadcast_to(K0[:512], out.shape), rtol=0, atol=1e-12)


def test_base2_lse_identity():
    rng = np.random.default_rng(5)
    s = rng.standard_normal(1000) * 3
    base_e = np.log(np.sum(np.exp(s)))
    base_2 = np.log2(np.sum(np.exp2(s * math.log2(math.e))))
    assert abs(base_2 * math.log(2) - base_e) < 1e-12


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8"])
def test_combine_of_shards_equals_union(cache_dtype):
    rng = np.random.default_rng(6)
    H, P = 6, 4
    nb = 10
    if cache_dtype == "fp8":
        cache = dsa_inputs._draw_fp8_normal(rng, (nb, 64, 576), 16.0)
        scale = 2.0 ** -4
    else:
        cache = dsa_inputs._draw_bf16_normal(rng, (nb, 64, 576), 1.0)
        scale = 1.0
    q = dsa_inputs._draw_bf16_normal(rng, (1, H, 576), 1.0)
    allslots = rng.choice(nb * 64, 200, replace=False).astype(np.int32)
    k = 80
    slots = np.full((P, 1, k), -1, np.int32)
    counts = np.zeros((P, 1), np.int32)
    parts = [allslots[:70], allslots[70:150], np.array([], np.int32), allslots[150:]]
    for p, s in enumerate(parts):
        slots[p, 0, :len(s)] = s
        counts[p, 0] = len(s)
    sm = 1 / 24
    pout, plse = oracle.sparse_mla_partial(q, cache, cache_dtype, scale, slots, counts, sm)
    assert np.all(pout[2] == 0) and np.all(np.isneginf(plse[2]))
    out, lse = oracle.lse_combine(pout, plse)
    ref, ref_lse = oracle.attention_over_ids(q[0], cache, cache_dtype, scale, allslots, sm)
    assert np.max(np.abs(out[0] - ref)) < 1e-12
    assert np.max(np.abs(lse[0] - ref_lse)) < 1e-12
    # single partial is the identity; the order of partials does not matter
    o1, l1 = oracle.lse_combine(pout[:1], plse[:1])
    assert np.array_equal(o1, pout[0]) and np.array_equal(l1, plse[0])
    perm = [3, 1, 0, 2]
    o2, l2 = oracle.lse_combine(pout[perm], plse[perm])
    assert np.max(np.abs(o2 - out)) < 1e-13 and np.max(np.abs(l2 - lse)) < 1e-13


def test_combine_all_empty():
    pout = np.zeros((3, 1, 2, 512))
    plse = np.full((3, 1, 2), -np.inf)
    out, lse = oracle.lse_combine(pout, plse)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


# ---- planted mistakes ------------------------------------------------------
def test_planted_value_width_mistake_is_caught(monkeypatch):
    real = oatt._attend

    def wrong(qh, K, sm):                         # value taken from the rope part
        Kw = K.copy()
        Kw[:, :64] = K[:, 512:576]
        o, l = real(qh, K, sm)
        o2, _ = real(qh, Kw, sm)
        return o2, l
    monkeypatch.setattr(oatt, "_attend", wrong)
    with pytest.raises(AssertionError):
        test_matches_torch_sdpa_fp64(0, 1.0)


def test_planted_lse_base_mistake_is_caught(monkeypatch):
    real = oatt._attend
    monkeypatch.setattr(oatt, "_attend", lambda qh, K, sm: (real(qh, K, sm)[0], real(qh, K, sm)[1] / math.log(2)))
    with pytest.raises(AssertionError):
        test_matches_torch_sdpa_fp64(1, 1 / 24)
