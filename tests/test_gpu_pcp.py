"""GPU parity of the sequence-sharded (PCP) prologue: materialise per rank,
gather, insert.

cache_insert writes already materialised K rows into a bf16 or fp8 cache; it
is checked byte for byte against the oracle's insert, with slots that are
skipped (negative, past the pool) and a strided row buffer.  The PCP prologue
(each rank materialises its slice of the new rows into the gathered buffer,
then every row is inserted) must leave the same cache and the same
materialised rows as the fused prologue, bit for bit.  The whole PCP decode
path is covered against the oracle by the `pcp_s` parity case.
"""
import sys

import numpy as np
import pytest
import torch

import dsa_inputs
import oracle

pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import sparse_attention_indexer_topk_amd as dsa  # noqa: E402
from sparse_attention_indexer_topk_amd.pipeline import DecodePath  # noqa: E402

DEV = "cuda"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def bits_u16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8"])
def test_cache_insert_matches_oracle(cache_dtype):
    r = np.random.default_rng(41)
    T, n_slots, ld = 37, 500, 520
    # materialised rows as bf16 bits, including values past the e4m3 range
    vals = r.standard_normal((T, 576)) * np.where(r.random((T, 576)) < 0.05, 300.0, 1.0)
    rows = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    kv = np.zeros((T, ld), np.uint16)
    kv[:, :512] = rows[:, :512]
    pe = rows[:, 512:].copy()
    slots = r.choice(n_slots, size=T, replace=False).astype(np.int64)
    slots[3] = -1                      # padding: skipped
    slots[7] = n_slots + 4             # past the pool: skipped
    scale = np.float32(2.0 ** -3)
    if cache_dtype == "fp8":
        cache0 = r.integers(0, 256, size=(n_slots, 576), dtype=np.uint8)
        dcache = torch.from_numpy(cache0.copy()).to(DEV)
        dscale = torch.tensor([scale], dtype=torch.float32, device=DEV)
    else:
        cache0 = r.integers(0, 1 << 16, size=(n_slots, 576), dtype=np.uint16)
        dcache = bits_u16(cache0.copy())
        dscale = None
    log(f"cache_insert {cache_dtype}: {T} rows")
    dsa.cache_insert(bits_u16(kv)[:, :512], bits_u16(pe), dcache,
                     torch.from_numpy(slots).to(DEV), cache_scale=dscale)
    torch.cuda.synchronize()
    ok = (slots >= 0) & (slots < n_slots)
    exp = oracle.cache_insert(cache0, np.where(ok, slots, -1), rows[:, :512], rows[:, 512:],
                              cache_dtype, scale)
    got = dcache.cpu().numpy() if cache_dtype == "fp8" else dcache.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, exp)


@pytest.mark.parametrize("ranks", [2, 3, 5])
def test_pcp_prologue_equals_fused_insert(ranks):
    c = dsa_inputs.make("pcp_s")
    log(f"pcp prologue, {ranks} ranks")
    fused = DecodePath(**{**dsa_inputs.device_arrays(c), "pcp_ranks": 0})
    split = DecodePath(**{**dsa_inputs.device_arrays(c), "pcp_ranks": ranks})
    fused.run_prologue()
    split.run_prologue()
    torch.cuda.synchronize()
    assert torch.equal(fused.cache, split.cache)
    assert torch.equal(fused.kv_c_out.view(torch.int16), split.kv_c_out.view(torch.int16))
    assert torch.equal(fused.k_pe_out.view(torch.int16), split.k_pe_out.view(torch.int16))
