"""GPU parity of lse_combine over its shape space: feature widths whose
8-feature slices split evenly over a thread's two slices and widths that do
not (8, 16, 24, 512), partial counts on each register path (1-8, 9-16, more),
bf16 and fp32 partials, empty partials (lse = -inf) and a (row, head) with
no partial at all (output 0, lse -inf).  The bar is the combine's own: the
oracle's fp64 result within the output's bf16 rounding plus the fp32
accumulation of the partials, and the LSE within 1e-5.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from dsa_testlib import bf16_bits_to_f64

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import sparse_attention_indexer_topk_amd as dsa  # noqa: E402


def f64_to_bf16_bits(x):
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("dim", [8, 16, 24, 512])
@pytest.mark.parametrize("P", [1, 3, 9, 17, 40])
@pytest.mark.parametrize("f32", [False, True])
def test_combine_shapes(dim, P, f32):
    print(f"[combine] dim {dim} P {P} fp32 {f32}", file=sys.stderr, flush=True)
    R, H = 3, 5
    r = np.random.default_rng(dim * 1000 + P * 10 + int(f32))
    po = r.standard_normal((P, R, H, dim))
    pl = r.standard_normal((P, R, H)) * 3.0
    pl[r.random((P, R, H)) < 0.2] = -np.inf       # empty partials
    pl[:, 1, 2] = -np.inf                          # a (row, head) with none at all
    po[np.isneginf(pl)] = 0.0                      # empty partials write 0
    if f32:
        po_in = po.astype(np.float32)
        dpo = torch.from_numpy(po_in).cuda()
    else:
        bits = f64_to_bf16_bits(po)
        po_in = bf16_bits_to_f64(bits)
        dpo = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    pl32 = pl.astype(np.float32)
    out, lse = dsa.lse_combine(dpo, torch.from_numpy(pl32).cuda())
    torch.cuda.synchronize()
    oo, ol = oracle.lse_combine(np.asarray(po_in, np.float64), pl32.astype(np.float64))
    g = bf16_bits_to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16))
    gl = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(gl), np.isneginf(ol))
    assert np.all(g[1, 2] == 0.0)
    fin = ~np.isneginf(ol)
    assert np.abs(gl[fin] - ol[fin]).max() <= 1e-5
    # the output's bf16 rounding, plus the fp32 accumulation of the weighted
    # partials (which may cancel, so it is bounded by their size, not the sum's)
    err = np.abs(g - oo)
    bound = 2.0 ** -8 * np.abs(oo) + 1e-5 * np.abs(po_in).max()
    assert np.all(err <= bound), f"max err {err.max():.3e}"
