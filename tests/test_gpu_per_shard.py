"""What one GPU can show of the multi-GPU layout: every shard as its own
launch (``shard_first = r``, ``shard_count = 1``), as a rank of a
decode-context-parallel group runs it (PR #46076 report, 关键源码片段
``_merge_dcp_topk_global(..., dcp_rank, dcp_world_size, ...)``).

Per shard r: the top-K over shard r's logits slice writes its k columns of
the shared candidate buffer (the all-gather, in place); the merge + convert
launch for shard r alone turns the merged ids into shard r's slot list; the
attention over shard r's slots gives its partial.  The union of the per-shard
launches must equal the oracle at every stage, and the combine of the
per-shard partials the oracle's combined output."""
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
from test_gpu_parity import bits16, check_prologue, host_cache_after_insert  # noqa: E402


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def run_per_shard(c, d, splits=1):
    """Every stage shard by shard; returns the GPU results as host arrays."""
    S, R, k = c.S, c.rows, c.k
    dev = d["logits"].device
    cand = torch.full((R, S * k, 2), float("nan"), dtype=torch.float32, device=dev)
    local_idx, ids, slots, counts, pouts, plses = [], [], [], [], [], []
    for r in range(S):
        li, _ = dsa.topk_select(d["logits"][r:r + 1], k, ctx=c.ctx, num_shards=S,
                                interleave=c.I, row_starts=d["row_starts"],
                                row_ends=d["row_ends"], shard_first=r, cand=cand)
        local_idx.append(li)
    for r in range(S):
        i_r, s_r, n_r = dsa.merge_convert(cand, k, d["block_table"][r:r + 1], id_bound=c.ctx,
                                          block_size=64, num_shards=S, interleave=c.I,
                                          row_req=d["row_req"], shard_first=r)
        o_r, l_r = dsa.sparse_mla_decode(d["q"], d["cache"], s_r, n_r, sm_scale=d["sm_scale"],
                                         splits=splits, cache_scale=d["cache_scale"])
        ids.append(i_r)
        slots.append(s_r)
        counts.append(n_r)
        pouts.append(o_r)
        plses.append(l_r)
    out, lse = dsa.lse_combine(torch.cat(pouts), torch.cat(plses))
    torch.cuda.synchronize()
    return dict(local_idx=torch.cat(local_idx).cpu().numpy(), cand=cand.cpu().numpy(),
                ids=[i.cpu().numpy() for i in ids], slots=torch.cat(slots).cpu().numpy(),
                counts=torch.cat(counts).cpu().numpy(),
                pout=bf16_bits_to_f64(bits16(torch.cat(pouts))),
                plse=torch.cat(plses).cpu().numpy().astype(np.float64),
                out=bf16_bits_to_f64(bits16(out)), lse=lse.cpu().numpy())


def compare(c, g, cache_ref, splits):
    oidx, ocand = oracle.topk_select(c.logits, c.row_starts, c.row_ends, c.ctx, c.k, c.S, c.I)
    assert np.array_equal(g["local_idx"], oidx)
    assert np.array_equal(g["cand"].view(np.uint32), ocand.view(np.uint32))
    oids = oracle.merge_candidates(ocand, c.k)
    for r in range(c.S):    # every rank reaches the same merged ids
        assert np.array_equal(g["ids"][r], oids)
    oslots, ocounts = oracle.convert_index(oids, c.row_req, c.block_table, 64, c.S, c.I)
    assert np.array_equal(g["slots"], oslots)
    assert np.array_equal(g["counts"], ocounts)
    opo, opl = oracle.sparse_mla_partial(c.q, cache_ref, c.cache_dtype, c.cache_scale, oslots,
                                         ocounts, c.sm_scale)
    gpo, gpl = g["pout"], g["plse"]
    if splits > 1:
        outs, lses = [], []
        for p in range(c.S):
            o, l = oracle.lse_combine(gpo[p * splits:(p + 1) * splits],
                                      gpl[p * splits:(p + 1) * splits])
            outs.append(o)
            lses.append(l)
        gpo, gpl = np.stack(outs), np.stack(lses)
    bad = attn_mismatch(gpo, opo, gpl, opl)
    assert not bad, f"per-shard partials: {bad}"
    oo, ol = oracle.lse_combine(opo, opl)
    bad = attn_mismatch(g["out"], oo, g["lse"], ol)
    assert not bad, f"combined: {bad}"


@pytest.mark.parametrize("name,splits", [("decode_s", 1), ("long_s", 2), ("odd_s", 1),
                                         ("fp8_s", 1), ("s16_s", 1), ("pcp_dcp_s", 1),
                                         ("heads_s", 2)])
def test_each_shard_as_its_own_launch(name, splits):
    log(f"[per-shard] case {name}, splits {splits}")
    c = dsa_inputs.make(name)
    d = dsa_inputs.device_arrays(c)
    cache_ref = c.cache
    if c.spec.prologue:     # the new rows go in first, as in the step
        path = DecodePath(**d)
        cache_ref = host_cache_after_insert(c, check_prologue(c, path))
    compare(c, run_per_shard(c, d, splits), cache_ref, splits)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_decode_workload_per_shard_launches():
    """The decode workload at one shard's real shape per launch, every row."""
    log("[per-shard] decode workload: generating")
    c = dsa_inputs.make("decode")
    d = dsa_inputs.device_arrays(c)
    log("[per-shard] decode workload: running")
    g = run_per_shard(c, d)
    log("[per-shard] decode workload: oracle")
    compare(c, g, c.cache, 1)
    log("[per-shard] decode workload: ok")
