"""GPU parity of the selection stages on inputs built to reach every branch.

Top-K: rows whose threshold bin is crowded (constant rows, a few distinct
values, thousands of +inf, a crowd of copies of the k-th value) take the
radix fallback; NaN / +-inf / -0 scores; rows with n = 0, 1, k, k + 1; a
row whose 16-byte-aligned start would overflow one chunk (element loads);
rows longer than 16K local positions (chunked sweeps); interleaved shards;
one output at a time; a candidate buffer that is only 8-byte aligned.

Merge: ties at the threshold score few enough to rank directly and too many
(id radix); invalid ids, NaN scores; fewer valid candidates than k; odd and
misaligned candidate buffers (8-byte loads); more than 16K candidates;
an id range needing several bitmap sweeps.

Convert: rows whose request is outside the table.

Merge + convert in one launch: shard sub-ranges, odd shard counts, k = 512,
ties, padding, missing requests, a narrow table, with and without the ids
output.

Every selection result is compared element by element (bit for bit) with the
oracle.

Attention: bf16 and fp8 pools larger than 4 GiB (the 64-bit gather
addresses), against the oracle to the attention tolerance.
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

DEV = torch.device("cuda:0")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def shard_rows(g, S, I):
    """[R][ctx] global logits -> [S][R][ld] shard-major local logits (gaps 0)."""
    R, C = g.shape
    ld = int(oracle.local_count(C, 0, S, I))
    ld = (ld + 3) // 4 * 4
    out = np.zeros((S, R, ld), dtype=np.float32)
    t = np.arange(C)
    own = oracle.owner(t, S, I)
    loc = oracle.local(t, S, I)
    for r in range(S):
        m = own == r
        out[r][:, loc[m]] = g[:, m]
    return out


def check_topk(g, starts, ends, k, S, I, *, cand_offset=0, outputs="both"):
    R, C = g.shape
    sh = shard_rows(g, S, I)
    oidx, ocand = oracle.topk_select(sh, starts, ends, C, k, S, I)
    lg = torch.from_numpy(sh).to(DEV)
    st = torch.from_numpy(np.asarray(starts, np.int32)).to(DEV)
    en = torch.from_numpy(np.asarray(ends, np.int32)).to(DEV)
    cand = None
    if outputs in ("both", "cand"):
        n = R * S * k * 2
        buf = torch.full((n + 4,), 7.0, dtype=torch.float32, device=DEV)
        cand = buf[cand_offset:cand_offset + n].view(R, S * k, 2)
    idx, cand = dsa.topk_select(lg, k, ctx=C, num_shards=S, interleave=I, row_starts=st,
                                row_ends=en, cand=cand, want_local_idx=outputs in ("both", "idx"),
                                want_cand=outputs in ("both", "cand"))
    torch.cuda.synchronize()
    if idx is not None:
        assert np.array_equal(idx.cpu().numpy(), oidx), "local_idx differs"
    if cand is not None:
        assert np.array_equal(cand.cpu().numpy().view(np.uint32), ocand.view(np.uint32)), \
            "candidates differ"


RNG = np.random.default_rng(20240611)


def normal(R, C, seed):
    return np.random.default_rng(seed).standard_normal((R, C)).astype(np.float32)


@pytest.mark.parametrize("k", [512, 2048])
def test_topk_crowded_threshold_bins(k):
    S, I, C = 2, 1, 16384
    g = normal(5, C, 1)
    g[0] = 0.5                                           # constant row
    g[1] = np.random.default_rng(2).integers(0, 4, C)   # four distinct values
    g[2, :] = np.float32(-3.0)                           # thousands of +inf on top
    g[2, ::3] = np.inf
    kth = np.float32(1.25)                               # a crowd at the k-th value
    g[3] = np.float32(-2.0) + 0.01 * g[3]
    g[3, :k // 2] = 9.0
    g[3, 5000:5000 + 3 * k] = kth
    g[4] = np.round(g[4] * 4.0) / 4.0                    # coarse grid, heavy ties
    log(f"topk crowded k={k}")
    check_topk(g, np.zeros(5, np.int32), np.full(5, C, np.int32), k, S, I)


def test_topk_special_values():
    S, I, C, k = 4, 1, 32768, 2048
    g = normal(4, C, 3)
    r = np.random.default_rng(4)
    for i in range(4):
        m = r.random(C)
        g[i, m < 0.05] = np.nan
        g[i, (m >= 0.05) & (m < 0.06)] = -np.inf
        g[i, (m >= 0.06) & (m < 0.065)] = np.inf
        g[i, (m >= 0.065) & (m < 0.08)] = 0.0
        g[i, (m >= 0.08) & (m < 0.095)] = -0.0
    g[1, 100:200] = np.float32(np.finfo(np.float32).max)
    g[1, 300:400] = np.float32(-np.finfo(np.float32).max)
    g[2, :] = np.nan                                     # only NaN
    g[2, ::7] = 1.0
    g[3, :] = -np.inf                                    # no finite score but one
    g[3, 10] = 2.0
    log("topk specials")
    check_topk(g, np.zeros(4, np.int32), np.full(4, C, np.int32), k, S, I)


def test_topk_small_and_boundary_rows():
    S, I, C, k = 2, 1, 8192, 1024
    g = normal(7, C, 5)
    # shard-local n = 0, 1, k - 1 (2k-1 global), k, k + 1, everything
    starts = np.array([0, 0, 0, 0, 0, 10, 3], np.int32)
    ends = np.array([0, 2, 2 * k - 1, 2 * k, 2 * k + 2, C, C - 5], np.int32)
    log("topk boundary rows")
    check_topk(g, starts, ends, k, S, I)


def test_topk_empty_shards():
    # a context shorter than one interleave period: shards 2 and 3 own no
    # position, shard 1 a partial block
    S, I, C, k = 4, 64, 100, 512
    g = normal(3, C, 6)
    starts = np.array([0, 0, 70], np.int32)
    ends = np.array([C, 50, C], np.int32)
    log("topk empty shards")
    check_topk(g, starts, ends, k, S, I)


def test_topk_element_loads_and_chunked_rows():
    # one shard of 20000 positions: the 16K-per-thread kernel streams it in
    # chunks; a row starting at 3 with 16384 valid positions fits one chunk
    # only when loaded element-wise
    S, I, C, k = 1, 1, 20000, 2048
    g = normal(4, C, 6)
    g[3] = 1.0
    starts = np.array([3, 0, 1, 0], np.int32)
    ends = np.array([3 + 16384, C, C - 7, C], np.int32)
    log("topk element loads / chunked")
    check_topk(g, starts, ends, k, S, I)


def test_topk_long_chunked_interleaved():
    S, I, C, k = 2, 7, 90001, 2048
    g = normal(2, C, 7)
    g[1] = np.round(g[1] * 8.0) / 8.0
    starts = np.array([11, 0], np.int32)
    ends = np.array([C, C - 13], np.int32)
    log("topk long interleaved")
    check_topk(g, starts, ends, k, S, I)


@pytest.mark.parametrize("outputs,offset", [("idx", 0), ("cand", 0), ("both", 2)])
def test_topk_single_output_and_misaligned_cand(outputs, offset):
    S, I, C, k = 3, 5, 7777, 512
    g = normal(3, C, 8)
    log(f"topk outputs={outputs} offset={offset}")
    check_topk(g, np.array([0, 5, 77], np.int32), np.array([C, 6000, C - 1], np.int32), k, S, I,
               cand_offset=offset, outputs=outputs)


# ------------------------------------------------------------------ merge --
def check_merge(cand, k, id_bound, *, offset=0):
    R, N, _ = cand.shape
    exp = oracle.merge_candidates(cand, k)
    n = R * N * 2
    buf = torch.zeros((n + 4,), dtype=torch.float32, device=DEV)
    dev = buf[offset:offset + n]
    dev.copy_(torch.from_numpy(cand.reshape(-1)))
    got = dsa.merge_candidates(dev.view(R, N, 2), k, id_bound=id_bound)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), exp)


def make_cand(R, N, id_bound, seed, score=None):
    r = np.random.default_rng(seed)
    c = np.empty((R, N, 2), np.float32)
    for i in range(R):
        c[i, :, 1] = r.choice(id_bound, size=N, replace=False)
        c[i, :, 0] = r.standard_normal(N) if score is None else score(r, N)
    return c


def test_merge_ties_ranked_and_radix():
    k, N, B = 2048, 8192, 40000
    c = make_cand(3, N, B, 10)
    c[0, :, 0] = np.where(np.arange(N) < 2000, 5.0, 1.0)   # 48 of 6192 tied at 1.0: id radix
    c[1, :, 0] = np.round(c[1, :, 0] * 64.0) / 64.0         # ties ranked in the list
    c[2, :, 0] = 3.0                                        # all equal: smallest ids
    log("merge ties")
    check_merge(c, k, B)


def test_merge_invalid_and_few_valid():
    k, N, B = 1024, 4 * 1024, 9001
    c = make_cand(4, N, B, 11)
    r = np.random.default_rng(12)
    c[0, r.random(N) < 0.3, 1] = -1.0                       # padding entries
    c[0, :50, 0] = np.nan
    c[0, 50:60, 0] = -np.inf
    c[1, :, 1] = -1.0                                       # no valid candidate
    c[2, 100:, 1] = -1.0                                    # fewer valid than k
    c[3, :7, 1] = np.nan
    c[3, 7:20, 0] = np.inf
    log("merge invalid / few")
    check_merge(c, k, B)


@pytest.mark.parametrize("N,offset", [(3 * 512 - 1, 0), (2 * 512, 2)])
def test_merge_element_loads(N, offset):
    k, B = 512, 5000
    c = make_cand(3, N, B, 13)
    c[1, :, 0] = np.round(c[1, :, 0] * 2.0)
    log(f"merge N={N} offset={offset}")
    check_merge(c, k, B, offset=offset)


def test_merge_many_candidates_and_wide_ids():
    # 16 shards x 2048 = 32768 candidates (chunked); ids up to 3e6 (several
    # bitmap sweeps)
    k, N, B = 2048, 16 * 2048, 3_000_000
    c = make_cand(2, N, B, 14)
    c[1, :, 0] = np.round(c[1, :, 0] * 16.0) / 16.0
    log("merge many / wide")
    check_merge(c, k, B)


# ---------------------------------------------------------------- convert --
def test_convert_rows_outside_table():
    S, I, k, bs = 3, 2, 512, 64
    C = 6000
    W = (int(oracle.local_count(C, 0, S, I)) + bs - 1) // bs
    r = np.random.default_rng(15)
    Rq = 3
    bt = r.permutation(S * Rq * W).astype(np.int32).reshape(S, Rq, W)
    ids = np.full((4, k), -1, np.int32)
    for i in range(4):
        n = [k, 300, k, 10][i]
        ids[i, :n] = np.sort(r.choice(C, size=n, replace=False))
    row_req = np.array([0, 2, 5, -1], np.int32)               # last two rows: no request
    es, ec = oracle.convert_index(ids, row_req, bt, bs, S, I)
    gs, gc = dsa.convert_index(torch.from_numpy(ids).to(DEV), torch.from_numpy(bt).to(DEV),
                               block_size=bs, num_shards=S, interleave=I,
                               row_req=torch.from_numpy(row_req).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(gs.cpu().numpy(), es)
    assert np.array_equal(gc.cpu().numpy(), ec)


# ---------------------------------------------------- merge + convert, fused --
@pytest.mark.parametrize("k,S,I,first,count,narrow,R",
                         [(2048, 16, 3, 0, 16, False, 5), (512, 5, 64, 1, 3, True, 5),
                          (1024, 4, 1, 3, 1, False, 5), (512, 4, 2, 0, 4, True, 300),
                          (512, 6, 1, 0, 6, False, 60)])
def test_merge_convert_matches_oracle(k, S, I, first, count, narrow, R):
    """merge_convert equals merge_candidates then convert_index: an odd number
    of shards in the run (a lone field in the last paired scan), a shard
    sub-range, k = 512 (threads past the merged ids idle), ties and padding
    among the candidates, a row with no valid candidate, a row whose request
    is outside the table, a table narrower than the ids (dropped ids), and
    the ids output left out.  The launch splits a row's shards into groups,
    one workgroup each, within one workgroup per CU: 300 rows convert every
    shard in one workgroup (paired scans), 60 rows x 6 shards make three
    groups of two, five rows one group per shard."""
    B, bs, Rq = 60000, 64, 4
    N = min(S * k, 16 * k)
    cand = make_cand(R, N, B, 30 + k + S)
    cand[1, :, 0] = np.round(cand[1, :, 0] * 8.0) / 8.0      # ties at the threshold
    cand[2, N // 3:, 1] = -1.0                               # padding entries
    cand[3, :, 1] = -1.0                                     # no valid candidate
    W = (int(oracle.local_count(B, 0, S, I)) + bs - 1) // bs
    if narrow:
        W -= 3                                               # ids past the table drop
    r = np.random.default_rng(31)
    bt = r.permutation(count * Rq * W).astype(np.int32).reshape(count, Rq, W)
    row_req = np.arange(R, dtype=np.int32) % Rq
    row_req[-1] = 7                                          # the last row: no request
    eids = oracle.merge_candidates(cand, k)
    es, ec = oracle.convert_index(eids, row_req, bt, bs, S, I, first=first, count=count)
    dcand = torch.from_numpy(cand).to(DEV)
    dbt = torch.from_numpy(bt).to(DEV)
    drq = torch.from_numpy(row_req).to(DEV)
    log(f"merge_convert k={k} S={S} I={I} run [{first}, {first + count})")
    for want_ids in (True, False):
        gids, gs, gc = dsa.merge_convert(dcand, k, dbt, id_bound=B, block_size=bs, num_shards=S,
                                         interleave=I, row_req=drq, shard_first=first,
                                         want_ids=want_ids)
        torch.cuda.synchronize()
        if want_ids:
            assert np.array_equal(gids.cpu().numpy(), eids)
        else:
            assert gids is None
        assert np.array_equal(gs.cpu().numpy(), es)
        assert np.array_equal(gc.cpu().numpy(), ec)


# ------------------------------------------------------------ attention --
def test_attention_pool_beyond_4gib_bf16():
    """A bf16 pool larger than 4 GiB gathers with 64-bit addresses; rows near
    its end and near its start must both be read right."""
    from dsa_testlib import attn_mismatch, bf16_bits_to_f64  # noqa: F401
    n_slots = (1 << 32) // 1152 + 40_000            # just past 4 GiB of bf16 rows
    R, H, k = 2, 32, 512
    r = np.random.default_rng(21)
    counts = np.array([[k, 300]], np.int32)
    slots = np.full((1, R, k), -1, np.int32)
    for i in range(R):
        c = counts[0, i]
        hi = r.choice(np.arange(n_slots - 60_000, n_slots), size=c // 2, replace=False)
        lo = r.choice(60_000, size=c - c // 2, replace=False)
        slots[0, i, :c] = np.concatenate([hi, lo])
    used = np.unique(slots[slots >= 0])
    rows_bits = (r.standard_normal((len(used), 576)).astype(np.float32)
                 .view(np.uint32) >> 16).astype(np.uint16)          # bf16 by truncation
    q = (r.standard_normal((R, H, 576)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    log(f"attention pool {n_slots} slots ({n_slots * 1152 / 2**30:.2f} GiB)")
    cache = torch.empty((n_slots, 576), dtype=torch.int16, device=DEV)
    cache[torch.from_numpy(used.astype(np.int64)).to(DEV)] = \
        torch.from_numpy(rows_bits.view(np.int16)).to(DEV)
    sm_scale = float(np.float32(1.0 / 24.0))
    out, lse = dsa.sparse_mla_decode(torch.from_numpy(q.view(np.int16)).to(DEV).view(torch.bfloat16),
                                     cache.view(torch.bfloat16),
                                     torch.from_numpy(slots).to(DEV),
                                     torch.from_numpy(counts).to(DEV), sm_scale=sm_scale)
    torch.cuda.synchronize()
    # the oracle sees only the used rows, with the slots renumbered
    remap = {int(s): j for j, s in enumerate(used)}
    oslots = np.vectorize(lambda s: remap.get(int(s), -1))(slots).astype(np.int32)
    po, pl = oracle.sparse_mla_partial(q, rows_bits, "bf16", None, oslots, counts, sm_scale)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    del cache
    torch.cuda.empty_cache()
    bad = attn_mismatch(bf16_bits_to_f64(got), po, lse.cpu().numpy(), pl)
    assert not bad, bad


@pytest.mark.parametrize("splits", [1, 2])
def test_attention_pool_beyond_4gib_fp8(splits):
    """An fp8 pool larger than 4 GiB (576-byte rows) gathers with 64-bit
    addresses too; rows near its end and near its start, split-K or not."""
    from dsa_testlib import attn_mismatch, bf16_bits_to_f64
    n_slots = (1 << 32) // 576 + 40_000             # just past 4 GiB of fp8 rows
    R, H, k = 2, 32, 512
    r = np.random.default_rng(22 + splits)
    counts = np.array([[k, 300]], np.int32)
    slots = np.full((1, R, k), -1, np.int32)
    for i in range(R):
        c = counts[0, i]
        hi = r.choice(np.arange(n_slots - 60_000, n_slots), size=c // 2, replace=False)
        lo = r.choice(60_000, size=c - c // 2, replace=False)
        slots[0, i, :c] = np.concatenate([hi, lo])
    used = np.unique(slots[slots >= 0])
    scale = np.float32(2.0 ** -4)
    # rows as the workloads draw them: N(0, 1) / scale rounded to e4m3
    codes = dsa_inputs._draw_fp8_normal(r, (len(used), 576), 1.0 / float(scale))
    q = (r.standard_normal((R, H, 576)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    log(f"attention fp8 pool {n_slots} slots ({n_slots * 576 / 2**30:.2f} GiB), splits {splits}")
    cache = torch.empty((n_slots, 576), dtype=torch.uint8, device=DEV)
    cache[torch.from_numpy(used.astype(np.int64)).to(DEV)] = torch.from_numpy(codes).to(DEV)
    sm_scale = float(np.float32(1.0 / 24.0))
    out, lse = dsa.sparse_mla_decode(torch.from_numpy(q.view(np.int16)).to(DEV).view(torch.bfloat16),
                                     cache, torch.from_numpy(slots).to(DEV),
                                     torch.from_numpy(counts).to(DEV), sm_scale=sm_scale,
                                     splits=splits,
                                     cache_scale=torch.tensor([scale], device=DEV))
    torch.cuda.synchronize()
    remap = {int(s): j for j, s in enumerate(used)}
    oslots = np.vectorize(lambda s: remap.get(int(s), -1))(slots).astype(np.int32)
    po, pl = oracle.sparse_mla_partial(q, codes, "fp8", scale, oslots, counts, sm_scale)
    got = bf16_bits_to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16))
    gl = lse.cpu().numpy().astype(np.float64)
    del cache
    torch.cuda.empty_cache()
    if splits > 1:   # merge the split-K partials with the oracle's combine
        got, gl = oracle.lse_combine(got, gl)
        got, gl = got[None], gl[None]
    bad = attn_mismatch(got, po, gl, pl)
    assert not bad, bad

