"""GPU: the output check has power.  One wrong latent row among a row's
selected tokens (the slot of one selection replaced by another slot of the
pool) must fail the tolerance check against the oracle's attention on the
correct selection, while the unchanged path passes it."""
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

from sparse_attention_indexer_topk_amd.pipeline import DecodePath  # noqa: E402


def _final(path):
    path.run_attention()
    path.run_combine()
    torch.cuda.synchronize()
    out = bf16_bits_to_f64(path.out.view(torch.int16).cpu().numpy().view(np.uint16))
    return out, path.lse.cpu().numpy()


def test_one_wrong_slot_fails_the_output_check():
    print("[mutation] case decode_s", file=sys.stderr, flush=True)
    c = dsa_inputs.make("decode_s")
    path = DecodePath(**dsa_inputs.device_arrays(c), splits=1)
    path.run_topk()
    path.run_merge_convert()
    torch.cuda.synchronize()
    slots = path.slots.cpu().numpy()
    counts = path.counts.cpu().numpy()

    po, pl = oracle.sparse_mla_partial(c.q, c.cache, c.cache_dtype, c.cache_scale, slots, counts,
                                       c.sm_scale)
    ref_out, ref_lse = oracle.lse_combine(po, pl)

    out, lse = _final(path)
    assert not attn_mismatch(out, ref_out, lse, ref_lse), "the unchanged path must pass"

    # shard 0, row 0: its first selection now reads a slot outside the row's
    # selection (a different block of the pool)
    assert counts[0, 0] > 0
    num_slots = c.cache.reshape(-1, 576).shape[0]
    chosen = set(slots[:, 0][slots[:, 0] >= 0].tolist())
    wrong = (int(slots[0, 0, 0]) + 64 * 97) % num_slots
    while wrong in chosen:
        wrong = (wrong + 64) % num_slots
    mutated = slots.copy()
    mutated[0, 0, 0] = wrong
    path.slots.copy_(torch.from_numpy(mutated).to(path.slots.device))
    out_m, lse_m = _final(path)
    bad = attn_mismatch(out_m, ref_out, lse_m, ref_lse)
    print(f"[mutation] violations with one wrong slot: {bad}", file=sys.stderr, flush=True)
    assert bad, "one wrong latent row went unnoticed"
