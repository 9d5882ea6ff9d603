"""GPU parity: the HIP path through the C ABI against the CPU oracle.

* every small parity case, element by element at every stage (prologue,
  top-K + candidates, merge, convert, partial attention, combine);
* the five full-size workloads in the launch configuration the benchmark
  times: every row of the decode, long and fp8 workloads at every stage, and
  256 (integer stages) and 18 (attention) rows spread over the prefill chunk;
* determinism: two runs are bit-identical;
* 20 seeded random shapes through every stage.
"""
import sys

import numpy as np
import pytest
import torch

import dsa_inputs
import oracle
from dsa_testlib import attn_mismatch, bf16_ulp_diff, bf16_bits_to_f64

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import sparse_attention_indexer_topk_amd as dsa  # noqa: E402
from sparse_attention_indexer_topk_amd.pipeline import DecodePath  # noqa: E402


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def cache_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.uint8:
        return t.cpu().numpy()
    return bits16(t)


def check_prologue(c, path):
    """Materialised rows within 1 bf16 ulp; inserted bytes exact w.r.t. the
    GPU's own materialised rows.  Returns the oracle's own inserted rows."""
    path.run_prologue()
    torch.cuda.synchronize()
    kvo, peo = bits16(path.kv_c_out), bits16(path.k_pe_out)
    okv, ope = oracle.rmsnorm_rope(c.kv_c, c.k_pe, c.rms_w, c.rms_eps, c.cos_sin, c.positions)
    assert bf16_ulp_diff(kvo, okv).max() <= 1
    assert bf16_ulp_diff(peo, ope).max() <= 1
    T = len(c.slot_mapping)
    sm = torch.from_numpy(c.slot_mapping).to(path.cache.device)
    g_rows = cache_bits(path.cache.view(-1, 576)[sm])
    blank = np.zeros((T, 576), dtype=g_rows.dtype)
    exp_rows = oracle.cache_insert(blank, np.arange(T), kvo, peo, c.cache_dtype, c.cache_scale)
    assert np.array_equal(g_rows, exp_rows), "inserted cache bytes differ"
    if c.spec.indexer:
        check_indexer_branch(c, path)
    return oracle.cache_insert(blank, np.arange(T), okv, ope, c.cache_dtype, c.cache_scale)


def check_indexer_branch(c, path):
    """The prologue's indexer-key branch (run by path.run_prologue): keys
    within 1 bf16 ulp of the oracle; with an indexer cache, the inserted bytes
    are the oracle's quantisation of the GPU's own keys and no other slot
    moved."""
    gk = bits16(path.index_k_out)
    ok = oracle.index_norm_rope(c.index_k, c.index_w, c.index_eps, c.cos_sin, c.positions)
    assert bf16_ulp_diff(gk, ok).max() <= 1, "indexer keys differ"
    icache = path.prologue.index_cache
    if icache is None:          # sequence-sharded: keys materialised only
        return
    g = icache.cpu().numpy().reshape(-1, 128)
    exp = oracle.index_cache_insert(c.index_cache, c.slot_mapping, gk, c.index_scale)
    assert np.array_equal(g, exp.reshape(-1, 128)), "indexer cache bytes differ"


def host_cache_after_insert(c, rows_oracle):
    flat = c.cache.reshape(-1, 576).copy()
    flat[c.slot_mapping] = rows_oracle
    return flat.reshape(c.cache.shape)


@pytest.mark.parametrize("name", list(dsa_inputs.PARITY_CASES))
def test_path_matches_oracle_every_stage(name):
    log(f"[parity] case {name}")
    check_every_stage(dsa_inputs.make(name))


def random_spec(i):
    """A seeded random shape: 1-16 shards with assorted interleaves, k of 512,
    1024 or 2048, shard rows from a few hundred positions to chunked sweeps,
    16-144 heads, bf16 or fp8 caches, window and mixed row bounds, a shared
    request or multi-token rows, sometimes the fused prologue."""
    r = np.random.default_rng(7000 + i)
    S = int(r.choice([1, 2, 3, 4, 5, 8, 16]))
    I = int(r.choice([1, 2, 3, 7, 64]))
    k = int(r.choice([512, 1024, 2048]))
    q_len = int(r.choice([1, 1, 2]))
    rows = q_len * int(r.integers(1, 4))
    # per-shard length first: short rows, one resident chunk, chunked sweeps
    local = int(r.choice([int(r.integers(600, 3000)), int(r.integers(3000, 12000)),
                          int(r.integers(12000, 40000))]))
    ctx = max(1200, min(local * S, 64000))
    cache = str(r.choice(["bf16", "fp8"]))
    return dsa_inputs.Spec(
        f"rand{i}", rows=rows, ctx=ctx, shards=S, interleave=I, k=k,
        heads=int(r.choice([16, 32, 48, 64, 128, 144])), seed=9000 + i,
        logits=str(r.choice(["normal", "rounded64", "bumps"])), cache=cache,
        latent_std=float(r.choice([1.0, 1.0 / 24.0])),
        one_request=bool(q_len == 1 and r.random() < 0.25),
        row_ends=None if q_len > 1 else r.choice([None, "mixed"]),
        row_starts=r.choice([None, "window"]),
        prologue=bool(r.random() < 0.3), q_len=q_len)


@pytest.mark.parametrize("i", range(20))
def test_random_shapes_every_stage(i):
    sp = random_spec(i)
    log(f"[parity] random case {i}: {sp}")
    check_every_stage(dsa_inputs.make(sp))


def check_every_stage(c):
    """Every stage of one case, element by element against the oracle."""
    path = DecodePath(**dsa_inputs.device_arrays(c))
    cache_ref = c.cache
    if c.spec.prologue:
        rows_oracle = check_prologue(c, path)
        cache_ref = host_cache_after_insert(c, rows_oracle)
        # nothing else in the cache moved
        g = cache_bits(path.cache).reshape(-1, 576)
        untouched = np.ones(g.shape[0], bool)
        untouched[c.slot_mapping] = False
        assert np.array_equal(g[untouched], c.cache.reshape(-1, 576)[untouched])

    path.run_topk(with_local_idx=True)
    torch.cuda.synchronize()
    oidx, ocand = oracle.topk_select(c.logits, c.row_starts, c.row_ends, c.ctx, c.k, c.S, c.I)
    assert np.array_equal(path.local_idx.cpu().numpy(), oidx)
    assert np.array_equal(path.cand.cpu().numpy().view(np.uint32), ocand.view(np.uint32))

    path.run_merge()
    torch.cuda.synchronize()
    oids = oracle.merge_candidates(ocand, c.k)
    gids = path.ids.cpu().numpy()
    assert np.array_equal(gids, oids)
    for i in range(c.rows):   # sharded-then-merged == unsharded
        e = oracle.unsharded_topk(c.global_logits[i], c.row_starts[i], c.row_ends[i], c.k)
        assert gids[i, :len(e)].tolist() == e.tolist()

    path.run_convert()
    torch.cuda.synchronize()
    oslots, ocounts = oracle.convert_index(oids, c.row_req, c.block_table, 64, c.S, c.I)
    assert np.array_equal(path.slots.cpu().numpy(), oslots)
    assert np.array_equal(path.counts.cpu().numpy(), ocounts)

    # the fused launch the bench times: the same three outputs
    fids, fslots, fcounts = dsa.merge_convert(
        path.cand, c.k, path.block_table, id_bound=c.ctx, block_size=64, num_shards=c.S,
        interleave=c.I, row_req=path.row_req)
    torch.cuda.synchronize()
    assert np.array_equal(fids.cpu().numpy(), oids)
    assert np.array_equal(fslots.cpu().numpy(), oslots)
    assert np.array_equal(fcounts.cpu().numpy(), ocounts)

    opo, opl = oracle.sparse_mla_partial(c.q, cache_ref, c.cache_dtype, c.cache_scale, oslots,
                                         ocounts, c.sm_scale)
    oo, ol = oracle.lse_combine(opo, opl)
    auto_splits = path.splits
    for splits in sorted({1, auto_splits, 3}):
        check_attention(c, path, splits, opo, opl, oo, ol, ocounts)


def split_partials_to_parts(gpo, gpl, S, splits):
    """Merge each part's split-K partials (GPU bf16 outputs) with the oracle's
    own combine, giving one partial per part."""
    outs, lses = [], []
    for p in range(S):
        o, l = oracle.lse_combine(gpo[p * splits:(p + 1) * splits], gpl[p * splits:(p + 1) * splits])
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def check_attention(c, path, splits, opo, opl, oo, ol, ocounts):
    path.splits = splits
    S, R, H = c.S, c.rows, c.heads
    path.pout = torch.empty((S * splits, R, H, 512), dtype=torch.bfloat16, device="cuda")
    path.plse = torch.empty((S * splits, R, H), dtype=torch.float32, device="cuda")
    path.run_attention()
    torch.cuda.synchronize()
    gpo = bf16_bits_to_f64(bits16(path.pout))
    gpl = path.plse.cpu().numpy().astype(np.float64)
    if splits == 1:
        empty = ocounts == 0
        if empty.any():   # empty shards still emit (0, -inf)
            assert np.all(gpo[empty] == 0) and np.all(np.isneginf(gpl[empty]))
    gpo_p, gpl_p = split_partials_to_parts(gpo, gpl, S, splits)
    bad = attn_mismatch(gpo_p, opo, gpl_p, opl)
    assert not bad, f"partials (splits={splits}): {bad}"
    path.run_combine()
    torch.cuda.synchronize()
    bad = attn_mismatch(bf16_bits_to_f64(bits16(path.out)), oo, path.lse.cpu().numpy(), ol)
    assert not bad, f"combined (splits={splits}): {bad}"


def integer_rows(name, R):
    """Rows whose selection, merge and conversion are compared bit for bit:
    every row, except on prefill (8192 rows), where 256 rows spread over the
    chunk plus the short-row boundary are."""
    if name != "prefill":
        return np.arange(R, dtype=np.int64)
    picks = {0, 1, 2, 3, 63, 511, 2046, 2047, 2048, 2049, 4095, 8190, 8191}
    picks |= set(np.linspace(0, R - 1, 256).round().astype(int).tolist())
    picks |= set(attention_rows(name, R).tolist())
    return np.array(sorted(picks), dtype=np.int64)


def attention_rows(name, R):
    """Rows whose partial and combined attention is compared: every row,
    except on prefill, where the oracle's fp64 attention over 8192 rows would
    take too long and 18 rows spread over the chunk are compared."""
    if name != "prefill":
        return np.arange(R, dtype=np.int64)
    picks = [0, 1, 2, 3, 63, 511, 2046, 2047, 2048, 2049, 4095, 6000, 8190, 8191]
    rng = np.random.default_rng(123)
    picks += rng.choice(R, 4, replace=False).tolist()
    return np.array(sorted(set(picks)), dtype=np.int64)


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(dsa_inputs.CONFIGS))
def test_full_size_workload(name):
    log(f"[full] workload {name}: generating")
    c = dsa_inputs.make(name)
    path = DecodePath(**dsa_inputs.device_arrays(c))
    rows_oracle = None
    if c.spec.prologue:
        rows_oracle = check_prologue(c, path)
    log(f"[full] workload {name}: running the step")
    path.run_topk()
    path.run_merge_convert()          # the launch sequence the bench times
    path.run_attention()
    path.run_combine()
    torch.cuda.synchronize()
    if rows_oracle is not None:
        flat = c.cache.reshape(-1, 576)
        flat[c.slot_mapping] = rows_oracle        # in place: the host copy is ours

    rs = integer_rows(name, c.rows)
    log(f"[full] workload {name}: selection, merge, conversion on {len(rs)} rows")
    _, ocand = oracle.topk_select(c.logits[:, rs], c.row_starts[rs], c.row_ends[rs], c.ctx, c.k,
                                  c.S, c.I)
    gcand = path.cand[torch.from_numpy(rs).cuda()].cpu().numpy()
    assert np.array_equal(gcand.view(np.uint32), ocand.view(np.uint32))
    oids = oracle.merge_candidates(ocand, c.k)
    assert np.array_equal(path.ids.cpu().numpy()[rs], oids)
    oslots, ocounts = oracle.convert_index(oids, c.row_req[rs], c.block_table, 64, c.S, c.I)
    assert np.array_equal(path.slots.cpu().numpy()[:, rs], oslots)
    assert np.array_equal(path.counts.cpu().numpy()[:, rs], ocounts)

    ar = attention_rows(name, c.rows)
    pos = np.searchsorted(rs, ar)
    assert np.array_equal(rs[pos], ar)
    log(f"[full] workload {name}: attention and combine on {len(ar)} rows")
    opo, opl = oracle.sparse_mla_partial(c.q[ar], c.cache, c.cache_dtype, c.cache_scale,
                                         oslots[:, pos], ocounts[:, pos], c.sm_scale)
    gpo = bf16_bits_to_f64(bits16(path.pout[:, torch.from_numpy(ar).cuda()]))
    gpl = path.plse.cpu().numpy()[:, ar].astype(np.float64)
    gpo, gpl = split_partials_to_parts(gpo, gpl, c.S, path.splits)
    bad = attn_mismatch(gpo, opo, gpl, opl)
    assert not bad, f"partials: {bad}"
    oo, ol = oracle.lse_combine(opo, opl)
    go = bf16_bits_to_f64(bits16(path.out[torch.from_numpy(ar).cuda()]))
    bad = attn_mismatch(go, oo, path.lse.cpu().numpy()[ar], ol)
    assert not bad, f"combined: {bad}"
    log(f"[full] workload {name}: ok")


@pytest.mark.parametrize("name", ["decode_s", "odd_s", "fp8_s"])
def test_two_runs_are_bit_identical(name):
    c = dsa_inputs.make(name)
    outs = []
    for _ in range(2):
        path = DecodePath(**dsa_inputs.device_arrays(c))
        path.step(with_local_idx=True)
        torch.cuda.synchronize()
        outs.append([t.cpu().clone() for t in (path.local_idx, path.cand, path.ids, path.slots,
                                              path.counts, path.pout.view(torch.int16),
                                              path.plse, path.out.view(torch.int16), path.lse)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint8) if a.dtype.is_floating_point else a,
                           b.view(torch.uint8) if b.dtype.is_floating_point else b)


def test_native_library_is_loaded():
    import os
    with open("/proc/self/maps") as f:
        maps = f.read()
    assert os.path.realpath(dsa.LIB_PATH) in maps or dsa.LIB_PATH in maps


@pytest.mark.parametrize("cache_dtype,splits", [("bf16", 1), ("bf16", 2), ("fp8", 1)])
def test_attention_score_jump_restarts_exactly(cache_dtype, splits):
    """The kernel fixes its softmax reference max from the first tile; a later
    tile whose scores exceed it by more than 2^64 (base 2) makes the workgroup
    restart its token list.  Scores here jump by ~77 (base 2) after the first
    three tiles, with distinct values among the high rows, so the result is
    only right if the restart path is."""
    from oracle.formats import f64_to_bf16, f64_to_e4m3
    rng = np.random.default_rng(7)
    R, H, P, k = 2, 128, 1, 512
    nslots = 8 * 64
    vals = np.zeros((nslots, 576))
    vals[:, :512] = rng.standard_normal((nslots, 512))          # values
    order = rng.permutation(nslots)
    cnt = 300
    late = order[100:cnt]                                         # tiles 3.. of the list
    vals[late, 512:] = 2.5 + 0.05 * rng.standard_normal((len(late), 64))
    scale = 2.0 ** -4
    if cache_dtype == "fp8":
        cache = f64_to_e4m3(vals / scale).reshape(8, 64, 576)
        cache_t = torch.from_numpy(cache).cuda()
        cs = torch.tensor([scale], dtype=torch.float32, device="cuda")
    else:
        cache = f64_to_bf16(vals).reshape(8, 64, 576)
        cache_t = torch.from_numpy(cache.view(np.int16)).cuda().view(torch.bfloat16)
        cs = None
    qv = np.zeros((R, H, 576))
    qv[:, :, 512:] = 8.0 * (1 + np.arange(H) / 512.0)[None, :, None]
    qb = f64_to_bf16(qv)
    slots = np.full((P, R, k), -1, np.int32)
    counts = np.zeros((P, R), np.int32)
    for i in range(R):
        slots[0, i, :cnt] = order[:cnt] if i == 0 else order[cnt - 1::-1][:cnt]
        counts[0, i] = cnt
    sm = float(np.float32(1 / 24))
    out, lse = dsa.sparse_mla_decode(
        torch.from_numpy(qb.view(np.int16)).cuda().view(torch.bfloat16), cache_t,
        torch.from_numpy(slots).cuda(), torch.from_numpy(counts).cuda(), sm_scale=sm,
        splits=splits, cache_scale=cs)
    torch.cuda.synchronize()
    gpo = bf16_bits_to_f64(bits16(out))
    gpl = lse.cpu().numpy().astype(np.float64)
    gpo, gpl = split_partials_to_parts(gpo, gpl, P, splits)
    opo, opl = oracle.sparse_mla_partial(qb, cache, cache_dtype, scale if cache_dtype == "fp8" else 1.0,
                                         slots, counts, sm)
    bad = attn_mismatch(gpo, opo, gpl, opl)
    assert not bad, bad
