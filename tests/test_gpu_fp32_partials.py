"""GPU parity of the attention's fp32 partial-output mode (a checking mode:
the partial outputs written without the bf16 rounding) and of the combine
reading fp32 partials.

* the fp32 partials, rounded to bf16 to nearest even, are bit for bit the
  bf16 partials of the same call, and the LSEs are identical (both modes
  share every step up to the final store);
* the fp32 partials and their combine match the oracle to the attention
  tolerance;
* cases: bf16 and fp8 caches, 4 and 8 shards, split-K, a head count that
  leaves a partial head group.
"""
import sys

import numpy as np
import pytest
import torch

import dsa_inputs
import oracle
from dsa_testlib import attn_mismatch, bf16_bits_to_f64

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import sparse_attention_indexer_topk_amd as dsa  # noqa: E402
from sparse_attention_indexer_topk_amd.pipeline import DecodePath  # noqa: E402


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even (finite inputs)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def merge_splits(po, pl, S, splits):
    """Each part's split-K partials merged by the oracle's combine."""
    outs, lses = [], []
    for p in range(S):
        o, l = oracle.lse_combine(po[p * splits:(p + 1) * splits], pl[p * splits:(p + 1) * splits])
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


@pytest.mark.parametrize("name,splits", [("decode_s", 1), ("decode_s", 3), ("fp8_s", 2),
                                         ("long_s", 2), ("heads_s", 1)])
def test_fp32_partials(name, splits):
    print(f"[fp32 partials] case {name} splits {splits}", file=sys.stderr, flush=True)
    c = dsa_inputs.make(name)
    path = DecodePath(**dsa_inputs.device_arrays(c))
    path.run_topk()
    path.run_merge_convert()
    torch.cuda.synchronize()
    _, ocand = oracle.topk_select(c.logits, c.row_starts, c.row_ends, c.ctx, c.k, c.S, c.I)
    oids = oracle.merge_candidates(ocand, c.k)
    oslots, ocounts = oracle.convert_index(oids, c.row_req, c.block_table, 64, c.S, c.I)
    assert np.array_equal(path.slots.cpu().numpy(), oslots)
    assert np.array_equal(path.counts.cpu().numpy(), ocounts)

    kw = dict(sm_scale=path.sm_scale, splits=splits, cache_scale=path.cache_scale)
    o16, l16 = dsa.sparse_mla_decode(path.q, path.cache, path.slots, path.counts, **kw)
    o32, l32 = dsa.sparse_mla_decode(path.q, path.cache, path.slots, path.counts,
                                     out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    assert o32.dtype == torch.float32
    assert torch.equal(l16, l32), "the two modes' LSEs differ"
    g32 = o32.cpu().numpy()
    assert np.all(np.isfinite(g32))
    assert np.array_equal(f32_to_bf16_rne(g32), bits16(o16)), \
        "fp32 partials rounded to bf16 differ from the bf16 partials"

    opo, opl = oracle.sparse_mla_partial(c.q, c.cache, c.cache_dtype, c.cache_scale, oslots,
                                         ocounts, c.sm_scale)
    gpo, gpl = merge_splits(g32.astype(np.float64), l32.cpu().numpy().astype(np.float64),
                            c.S, splits)
    bad = attn_mismatch(gpo, opo, gpl, opl)
    assert not bad, f"fp32 partials: {bad}"

    oo, ol = oracle.lse_combine(opo, opl)
    out32, lse32 = dsa.lse_combine(o32, l32)
    out16, lse16 = dsa.lse_combine(o16, l16)
    torch.cuda.synchronize()
    bad = attn_mismatch(bf16_bits_to_f64(bits16(out32)), oo, lse32.cpu().numpy(), ol)
    assert not bad, f"combined fp32 partials: {bad}"
    # the two combines differ only by the partials' bf16 rounding (half an
    # ulp of a partial) and the outputs' own (half an ulp each)
    diff = np.abs(bf16_bits_to_f64(bits16(out32)) - bf16_bits_to_f64(bits16(out16)))
    assert diff.max() <= 2.0 ** -8 * (np.abs(g32).max() + np.abs(oo).max())
    assert torch.equal(lse32, lse16)
