"""The fused norm + RoPE call's contract on the GPU (PR #52046 report,
实现拆解 item 1): outputs are materialised only when given; each cache is
written only when it and the slot mapping are given; with every output and the
slot mapping absent nothing at all is written (the profiling path)."""
import sys

import numpy as np
import pytest
import torch

import dsa_inputs
import oracle
from dsa_testlib import bf16_ulp_diff

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import sparse_attention_indexer_topk_amd as dsa  # noqa: E402


def _args():
    c = dsa_inputs.make("idx_s")
    d = dsa_inputs.device_arrays(c)
    p = d["prologue"]
    return c, d, p


def _snap(*ts):
    torch.cuda.synchronize()
    return [t.clone() for t in ts]


def test_nothing_written_without_outputs_and_slot_mapping():
    print("[contract] profiling path", file=sys.stderr, flush=True)
    c, d, p = _args()
    before = _snap(d["cache"], p["index_cache"])
    kv, pe, ik = dsa.fused_rmsnorm_rope(p["kv_c"], p["k_pe"], p["rms_w"], p["eps"], p["cos_sin"],
                                        p["positions"], cache=d["cache"],
                                        cache_scale=d["cache_scale"], index_k=p["index_k"],
                                        index_w=p["index_w"], index_cache=p["index_cache"],
                                        index_cache_scale=p["index_cache_scale"])
    assert kv is None and pe is None and ik is None
    after = _snap(d["cache"], p["index_cache"])
    assert all(torch.equal(a, b) for a, b in zip(before, after))


def test_indexer_cache_needs_the_slot_mapping_and_the_latent_insert_is_independent():
    print("[contract] cache rules", file=sys.stderr, flush=True)
    c, d, p = _args()
    T = len(c.slot_mapping)
    ik_out = torch.empty((T, 128), dtype=torch.bfloat16, device="cuda")
    before = _snap(d["cache"], p["index_cache"])
    # the indexer key materialised, the indexer cache given without a slot
    # mapping: the key is written, neither cache is
    dsa.fused_rmsnorm_rope(None, None, None, p["eps"], p["cos_sin"], p["positions"],
                           index_k=p["index_k"], index_w=p["index_w"], index_k_out=ik_out,
                           index_cache=p["index_cache"], index_cache_scale=p["index_cache_scale"])
    after = _snap(d["cache"], p["index_cache"])
    assert all(torch.equal(a, b) for a, b in zip(before, after))
    ok = oracle.index_norm_rope(c.index_k, c.index_w, c.index_eps, c.cos_sin, c.positions)
    gk = ik_out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert bf16_ulp_diff(gk, ok).max() <= 1
    # slot mapping and the latent cache only: the indexer cache stays as it was
    dsa.fused_rmsnorm_rope(p["kv_c"], p["k_pe"], p["rms_w"], p["eps"], p["cos_sin"],
                           p["positions"], cache=d["cache"], cache_scale=d["cache_scale"],
                           slot_mapping=p["slot_mapping"], index_k=p["index_k"],
                           index_w=p["index_w"])
    torch.cuda.synchronize()
    assert torch.equal(p["index_cache"], before[1])
    assert not torch.equal(d["cache"], before[0])       # the latent rows went in
