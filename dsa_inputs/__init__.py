"""Seeded synthetic inputs for the DSA sparse-attention path.

This module only *draws data*: it holds none of the method's arithmetic (no
top-K, no merge, no index conversion, no attention, no normalisation).  Both
the CPU oracle (``oracle/``) and the HIP path (through the tests and the
benchmark) receive exactly the arrays built here, as raw bits:

* fp32 indexer logits as ``float32``;
* bf16 tensors as ``uint16`` bit patterns;
* fp8 e4m3 cache entries as ``uint8`` codes.

Workloads follow the five workloads of the DSA description this library is
built from (tiny / decode / long context / prefill chunk / fp8 cache with the
fused prologue) plus smaller cases that the oracle finishes in seconds.

Layout of the context-sharded inputs.  The sharded KV cache of decode context
parallelism puts global token ``t`` on shard ``(t // I) % S`` (``S`` shards,
interleave ``I``); on its shard the tokens keep their global order.  Each
shard's logits therefore form one slice ``logits[s]`` of a shard-major buffer
``[S][rows][ld]``.  The slice is produced here by a reshape of the global
``[rows][ctx]`` array: ``ctx`` is padded to a multiple of ``I*S`` with the
sentinel value, viewed as ``[rows][ctx/(I*S)][S][I]`` and transposed to
``[S][rows][ctx/(I*S)][I]``.  That is pure data placement; the oracle
re-derives the same placement from its own closed-form index maps and a test
checks that both agree.

Value distributions not fixed by the workload description (see the design
notes) are drawn by inverse-CDF sampling: a uniform 16-bit draw indexes a
65,536-entry table of normal quantiles, rounded once to the storage format.
That gives i.i.d. N(0, std^2) samples quantised at 2^-16 in probability, fast
enough to fill multi-GB caches.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

SENTINEL = np.float32(64.0)   # logit written where no token exists
BLOCK = 64                    # tokens per KV-cache block
D_LATENT = 576                # 512 kv_c + 64 rope
D_V = 512
D_ROPE = 64

__all__ = ["Case", "CONFIGS", "PARITY_CASES", "make", "spec", "SENTINEL",
           "BLOCK", "D_LATENT", "D_V", "D_ROPE", "shard_layout"]


# --------------------------------------------------------------------------
# Workload specifications
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    rows: int
    ctx: int
    shards: int
    interleave: int
    k: int
    heads: int
    seed: int
    logits: str = "normal"          # normal | rounded64 | bumps | causal
    cache: str = "bf16"             # bf16 | fp8
    latent_std: float = 1.0 / 24.0
    one_request: bool = False       # prefill: every row reads request 0
    row_ends: Optional[str] = None  # None (=ctx) | "causal" | "mixed"
    row_starts: Optional[str] = None  # None (=0) | "window"
    prologue: bool = False          # fp8 workload: new K rows + insert
    fp8_scale: float = 2.0 ** -4
    q_pos_step: int = 1             # causal: row i ends at 1 + i*step
    q_len: int = 1                  # query tokens per request (multi-token decode)
    pcp: int = 0                    # >0: prologue in sequence-sharded (PCP) form over pcp ranks
    indexer: bool = False           # prologue also runs the indexer-key branch


CONFIGS = {
    # The five workloads.
    "tiny": Spec("tiny", rows=2, ctx=4096, shards=2, interleave=1, k=512,
                 heads=16, seed=0, logits="rounded64", latent_std=1.0),
    "decode": Spec("decode", rows=64, ctx=32768, shards=4, interleave=1,
                   k=2048, heads=128, seed=1),
    "long": Spec("long", rows=16, ctx=131072, shards=8, interleave=64,
                 k=2048, heads=128, seed=2, logits="bumps"),
    "prefill": Spec("prefill", rows=8192, ctx=32768, shards=4, interleave=1,
                    k=2048, heads=128, seed=3, logits="causal",
                    one_request=True, row_ends="causal"),
    "fp8": Spec("fp8", rows=128, ctx=65536, shards=4, interleave=1, k=2048,
                heads=128, seed=4, cache="fp8", prologue=True),
}

# Smaller cases with the same structure: several tiles, ragged tails, shards
# of unequal length, rows shorter than k, odd interleaves, nonzero starts.
PARITY_CASES = {
    "tiny": CONFIGS["tiny"],
    "decode_s": Spec("decode_s", rows=5, ctx=9001, shards=4, interleave=1,
                     k=1024, heads=32, seed=11, row_ends="mixed"),
    "long_s": Spec("long_s", rows=3, ctx=40000, shards=8, interleave=64,
                   k=2048, heads=16, seed=12, logits="bumps"),
    "prefill_s": Spec("prefill_s", rows=96, ctx=3000, shards=4, interleave=1,
                      k=512, heads=16, seed=13, logits="causal",
                      one_request=True, row_ends="causal", q_pos_step=31),
    "fp8_s": Spec("fp8_s", rows=6, ctx=10000, shards=4, interleave=1, k=512,
                  heads=32, seed=14, cache="fp8", prologue=True),
    "odd_s": Spec("odd_s", rows=4, ctx=7777, shards=3, interleave=5, k=512,
                  heads=48, seed=15, logits="rounded64", latent_std=1.0,
                  row_starts="window", row_ends="mixed"),
    "wide_s": Spec("wide_s", rows=2, ctx=70001, shards=2, interleave=1,
                   k=2048, heads=16, seed=16),
    "fp8_bf16pro_s": Spec("fp8_bf16pro_s", rows=3, ctx=3333, shards=2,
                          interleave=3, k=1024, heads=16, seed=17,
                          prologue=True, latent_std=1.0),
    # multi-token decode: 3 requests x 3 query tokens sharing each request's
    # block table; 2 shards, as in the pages' [4, 4, 5] localisation example
    "mtp_s": Spec("mtp_s", rows=9, ctx=9001, shards=2, interleave=1, k=512,
                  heads=16, seed=18, q_len=3),
    # more heads than one workgroup holds: a full group of 128 and a group of 16
    "heads_s": Spec("heads_s", rows=3, ctx=6000, shards=2, interleave=1, k=512,
                    heads=144, seed=20, row_ends="mixed"),
    # sequence-sharded (PCP) prefill chunk over a replicated fp8 cache: no
    # context sharding; the new K rows are materialised by 3 ranks, gathered
    # and inserted (materialise -> gather -> insert)
    "pcp_s": Spec("pcp_s", rows=24, ctx=3000, shards=1, interleave=1, k=512,
                  heads=16, seed=19, logits="causal", one_request=True,
                  row_ends="causal", q_pos_step=113, cache="fp8", prologue=True, pcp=3),
    # sequence-sharded prologue over 3 ranks combined with a context sharded
    # over 2 shards (PCP x DCP): materialise -> gather -> insert, then the
    # per-shard top-K, merge, attention and the combine of the shard partials
    "pcp_dcp_s": Spec("pcp_dcp_s", rows=6, ctx=4100, shards=2, interleave=1, k=512,
                      heads=32, seed=22, cache="fp8", prologue=True, pcp=3,
                      row_ends="mixed"),
    # the most shards the library takes: 16 shards of interleave 2
    "s16_s": Spec("s16_s", rows=3, ctx=12007, shards=16, interleave=2, k=512,
                  heads=16, seed=21, row_ends="mixed"),
    # the prologue's indexer-key branch in the same launch: materialised and
    # inserted into an fp8 indexer cache (decode), materialised only
    # (sequence-sharded prologue over 2 ranks)
    "idx_s": Spec("idx_s", rows=5, ctx=5000, shards=2, interleave=1, k=512,
                  heads=16, seed=23, cache="fp8", prologue=True, indexer=True,
                  row_ends="mixed"),
    "idx_pcp_s": Spec("idx_pcp_s", rows=4, ctx=3000, shards=1, interleave=1, k=512,
                      heads=16, seed=24, cache="fp8", prologue=True, indexer=True, pcp=2),
}


def spec(name: str) -> Spec:
    if name in CONFIGS:
        return CONFIGS[name]
    return PARITY_CASES[name]


# --------------------------------------------------------------------------
# Format helpers (storage only)
# --------------------------------------------------------------------------
def _f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 bit patterns (via fp32, ties to even).

    Only used to build the sampling tables below; values are far from the
    fp32 limits."""
    f = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((f >> np.uint32(16)) & np.uint32(1))
    return ((f + bias) >> np.uint32(16)).astype(np.uint16)


def _normal_quantiles() -> np.ndarray:
    from scipy.special import ndtri
    p = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
    return ndtri(p)


_TABLES: dict = {}


def _bf16_normal_table(std: float) -> np.ndarray:
    key = ("bf16", float(std))
    if key not in _TABLES:
        _TABLES[key] = _f64_to_bf16_bits(_normal_quantiles() * std)
    return _TABLES[key]


def _fp8_normal_table(inv_scale: float) -> np.ndarray:
    """e4m3 codes of N(0,1)/scale quantiles, rounded by torch's own cast."""
    key = ("fp8", float(inv_scale))
    if key not in _TABLES:
        import torch
        v = torch.from_numpy((_normal_quantiles() * inv_scale).astype(np.float32))
        _TABLES[key] = v.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return _TABLES[key]


def _draw_bf16_normal(rng, shape, std, chunk=1 << 26):
    table = _bf16_normal_table(std)
    out = np.empty(int(np.prod(shape)), dtype=np.uint16)
    for s in range(0, out.size, chunk):
        e = min(out.size, s + chunk)
        out[s:e] = table[rng.integers(0, 65536, e - s, dtype=np.uint16)]
    return out.reshape(shape)


def _draw_fp8_normal(rng, shape, inv_scale, chunk=1 << 26):
    table = _fp8_normal_table(inv_scale)
    out = np.empty(int(np.prod(shape)), dtype=np.uint8)
    for s in range(0, out.size, chunk):
        e = min(out.size, s + chunk)
        out[s:e] = table[rng.integers(0, 65536, e - s, dtype=np.uint16)]
    return out.reshape(shape)


# --------------------------------------------------------------------------
# Sharded placement (data layout only)
# --------------------------------------------------------------------------
def shard_layout(x: np.ndarray, shards: int, interleave: int, fill) -> np.ndarray:
    """Place a global ``[..., ctx]`` array into shard-major ``[S][..., ld]``.

    ``ctx`` is padded with ``fill`` to a multiple of ``I*S``; the result's
    last dimension is ``ld = ceil(ctx / (I*S)) * I``."""
    S, I = shards, interleave
    lead = x.shape[:-1]
    ctx = x.shape[-1]
    period = S * I
    nper = -(-ctx // period)
    pad = np.full(lead + (nper * period,), fill, dtype=x.dtype)
    pad[..., :ctx] = x
    v = pad.reshape(lead + (nper, S, I))
    nd = len(lead)
    perm = (nd + 1,) + tuple(range(nd)) + (nd, nd + 2)
    return np.ascontiguousarray(v.transpose(perm)).reshape((S,) + lead + (nper * I,))


# --------------------------------------------------------------------------
# Case construction
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Case:
    spec: Spec
    global_logits: np.ndarray      # [R][ctx] float32 (sentinel beyond row_end)
    logits: np.ndarray             # [S][R][ld] float32, shard-major
    row_starts: np.ndarray         # [R] int32 (global coordinates)
    row_ends: np.ndarray           # [R] int32 (global coordinates)
    row_req: np.ndarray            # [R] int32 request of each row
    q: np.ndarray                  # [R][H][576] uint16 (bf16)
    cache: np.ndarray              # [nblocks][64][576] uint16 (bf16) or uint8 (e4m3)
    cache_scale: np.float32        # fp8 per-tensor scale (1.0 for bf16)
    block_table: np.ndarray        # [S][Rq][W] int32 physical block ids
    sm_scale: np.float32
    # prologue (new K rows), present when spec.prologue
    kv_c: Optional[np.ndarray] = None        # [T][512] uint16
    k_pe: Optional[np.ndarray] = None        # [T][64] uint16
    rms_w: Optional[np.ndarray] = None       # [512] uint16
    rms_eps: float = 1e-6
    cos_sin: Optional[np.ndarray] = None     # [n_pos][64] float32: cos | sin
    positions: Optional[np.ndarray] = None   # [T] int32
    slot_mapping: Optional[np.ndarray] = None  # [T] int64
    # indexer-key branch of the prologue, present when spec.indexer
    index_k: Optional[np.ndarray] = None       # [T][128] uint16 (bf16)
    index_w: Optional[np.ndarray] = None       # [128] uint16 (bf16)
    index_eps: float = 1e-6
    index_cache: Optional[np.ndarray] = None   # [nblocks][64][128] uint8 (e4m3)
    index_scale: np.float32 = np.float32(2.0 ** -4)

    # convenience views
    @property
    def S(self):
        return self.spec.shards

    @property
    def I(self):
        return self.spec.interleave

    @property
    def k(self):
        return self.spec.k

    @property
    def rows(self):
        return self.spec.rows

    @property
    def ctx(self):
        return self.spec.ctx

    @property
    def heads(self):
        return self.spec.heads

    @property
    def cache_dtype(self):
        return self.spec.cache


def _row_bounds(sp: Spec, rng):
    R, C = sp.rows, sp.ctx
    ends = np.full(R, C, dtype=np.int64)
    if sp.row_ends == "causal":
        ends = np.minimum(1 + np.arange(R, dtype=np.int64) * sp.q_pos_step, C)
    elif sp.row_ends == "mixed":
        # full rows, a row shorter than k, a row of one token, mid lengths
        choices = [C, max(1, sp.k // 2 + 3), 1, C // 3 + 7, C - 5]
        ends = np.array([choices[i % len(choices)] for i in range(R)], dtype=np.int64)
    if sp.q_len > 1:
        # multi-token decode: request r has global length L_r; its j-th of
        # q_len query tokens sees L_r - (q_len - 1 - j) tokens (the per-token
        # lengths are expanded globally, then localised per shard)
        n_req = R // sp.q_len
        base = np.maximum(C - 37 * np.arange(n_req, dtype=np.int64), sp.q_len)
        i = np.arange(R, dtype=np.int64)
        ends = base[i // sp.q_len] - (sp.q_len - 1 - i % sp.q_len)
    starts = np.zeros(R, dtype=np.int64)
    if sp.row_starts == "window":
        starts = np.array([(i * 97) % max(1, C // 4) for i in range(R)], dtype=np.int64)
        starts = np.minimum(starts, ends)
    return starts.astype(np.int32), ends.astype(np.int32)


def _draw_logits(sp: Spec, rng, starts, ends):
    R, C = sp.rows, sp.ctx
    if sp.logits == "rounded64":
        g = np.round(rng.standard_normal((R, C)) * 64.0) / 64.0
        g = g.astype(np.float32)
    elif sp.logits == "normal":
        g = rng.standard_normal((R, C), dtype=np.float32)
    elif sp.logits == "bumps":
        g = rng.standard_normal((R, C)).astype(np.float64)
        centres = rng.uniform(0.0, C, size=(R, 16))
        t = np.arange(C, dtype=np.float64)
        for i in range(R):
            for c in centres[i]:
                lo, hi = int(max(0, c - 8 * 256)), int(min(C, c + 8 * 256 + 1))
                g[i, lo:hi] += 4.0 * np.exp(-((t[lo:hi] - c) ** 2) / (2.0 * 256.0 ** 2))
        g = g.astype(np.float32)
    elif sp.logits == "causal":
        g = rng.standard_normal((R, C), dtype=np.float32)
    else:
        raise ValueError(sp.logits)
    # positions outside [row_start, row_end) hold a sentinel a kernel that
    # ignored the row bounds would pick first
    col = np.arange(C)
    for i in range(R):
        if starts[i] > 0:
            g[i, :starts[i]] = SENTINEL
        if ends[i] < C:
            g[i, ends[i]:] = SENTINEL
    del col
    return g


def _cos_sin_table(n_pos: int, base: float = 10000.0) -> np.ndarray:
    """RoPE table in the usual cache layout: ``[pos][cos(32) | sin(32)]``,
    frequency i = base^(-2i/64), computed in float64 and stored as float32."""
    inv = base ** (-(np.arange(D_ROPE // 2, dtype=np.float64) * 2.0) / D_ROPE)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def make(name_or_spec, *, with_cache: bool = True) -> Case:
    """Build the seeded inputs of a named workload (or an explicit Spec)."""
    sp = spec(name_or_spec) if isinstance(name_or_spec, str) else name_or_spec
    rng = np.random.Generator(np.random.PCG64(sp.seed))
    R, C, S, I, H = sp.rows, sp.ctx, sp.shards, sp.interleave, sp.heads
    starts, ends = _row_bounds(sp, rng)
    # draw order: logits, q, cache, block table, prologue inputs
    g = _draw_logits(sp, rng, starts, ends)
    sharded = shard_layout(g, S, I, SENTINEL)
    ld = sharded.shape[-1]
    q = _draw_bf16_normal(rng, (R, H, D_LATENT), 1.0)

    Rq = 1 if sp.one_request else R // sp.q_len
    W = -(-ld // BLOCK)                       # table width per (shard, request)
    nblocks = S * Rq * W
    if with_cache:
        if sp.cache == "fp8":
            cache = _draw_fp8_normal(rng, (nblocks, BLOCK, D_LATENT), 1.0 / sp.fp8_scale)
            scale = np.float32(sp.fp8_scale)
        else:
            cache = _draw_bf16_normal(rng, (nblocks, BLOCK, D_LATENT), sp.latent_std)
            scale = np.float32(1.0)
    else:
        cache = np.zeros((0, BLOCK, D_LATENT), dtype=np.uint8 if sp.cache == "fp8" else np.uint16)
        scale = np.float32(sp.fp8_scale if sp.cache == "fp8" else 1.0)
    block_table = rng.permutation(nblocks).astype(np.int32).reshape(S, Rq, W)
    row_req = (np.zeros(R, dtype=np.int32) if sp.one_request
               else (np.arange(R, dtype=np.int32) // sp.q_len).astype(np.int32))

    case = Case(spec=sp, global_logits=g, logits=sharded, row_starts=starts,
                row_ends=ends, row_req=row_req, q=q, cache=cache,
                cache_scale=scale, block_table=block_table,
                sm_scale=np.float32(1.0 / math.sqrt(D_LATENT)))

    if sp.prologue:
        # One new token per row, at the last position of the row's context;
        # the cache manager has reserved its slot: the entry of the row's
        # owner shard that holds that position.
        T = R
        case.kv_c = _draw_bf16_normal(rng, (T, D_V), 1.0)
        case.k_pe = _draw_bf16_normal(rng, (T, D_ROPE), 1.0)
        w = rng.uniform(0.5, 1.5, size=D_V)
        case.rms_w = _f64_to_bf16_bits(w)
        case.rms_eps = 1e-6
        case.cos_sin = _cos_sin_table(C)
        pos = (ends.astype(np.int64) - 1).clip(min=0)
        case.positions = pos.astype(np.int32)
        where = shard_layout(np.arange(C, dtype=np.int64)[None, :], S, I, -1)[:, 0, :]
        slots = np.empty(T, dtype=np.int64)
        for t in range(T):
            sh, loc = np.argwhere(where == pos[t])[0]
            blk = block_table[sh, row_req[t], loc // BLOCK]
            slots[t] = int(blk) * BLOCK + int(loc % BLOCK)
        case.slot_mapping = slots
        if sp.indexer:
            # drawn after every other input, so the other cases keep their data
            case.index_k = _draw_bf16_normal(rng, (T, 128), 1.0)
            case.index_w = _f64_to_bf16_bits(rng.uniform(0.5, 1.5, size=128))
            case.index_cache = _draw_fp8_normal(rng, (nblocks, BLOCK, 128), 1.0 / sp.fp8_scale)
            case.index_scale = np.float32(sp.fp8_scale)
    return case


# --------------------------------------------------------------------------
# Upload (storage only): the same bits as the host arrays, as device tensors
# --------------------------------------------------------------------------
def device_arrays(case: Case, device="cuda", logits=None, q=None) -> dict:
    """Device copies of a case's inputs, keyed like the decode path's
    constructor arguments.  bf16 arrays become torch.bfloat16 tensors with
    identical bits; fp8 codes stay uint8."""
    import torch

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    sp = case.spec
    d = dict(
        logits=dev(case.logits if logits is None else logits),
        row_starts=dev(case.row_starts), row_ends=dev(case.row_ends),
        ctx=sp.ctx, k=sp.k, num_shards=sp.shards, interleave=sp.interleave,
        q=bf16(case.q if q is None else q),
        cache=dev(case.cache) if sp.cache == "fp8" else bf16(case.cache),
        cache_scale=dev(np.array([case.cache_scale], dtype=np.float32)) if sp.cache == "fp8" else None,
        block_table=dev(case.block_table),
        row_req=dev(case.row_req), sm_scale=float(case.sm_scale), block_size=BLOCK,
    )
    if sp.prologue:
        d["prologue"] = dict(kv_c=bf16(case.kv_c), k_pe=bf16(case.k_pe), rms_w=bf16(case.rms_w),
                             eps=float(case.rms_eps), cos_sin=dev(case.cos_sin),
                             positions=dev(case.positions), slot_mapping=dev(case.slot_mapping))
        if sp.indexer:
            d["prologue"].update(
                index_k=bf16(case.index_k), index_w=bf16(case.index_w),
                index_eps=float(case.index_eps),
                index_cache=None if sp.pcp else dev(case.index_cache),
                index_cache_scale=None if sp.pcp else dev(np.array([case.index_scale],
                                                                   dtype=np.float32)))
        if sp.pcp:
            d["pcp_ranks"] = sp.pcp
    return d


def redraw_logits_q(case: Case, index: int):
    """Another draw of the logits (shard-major) and q of a workload, from an
    independent seed; the cache, tables and row bounds stay the case's own.
    Used to rotate several input sets through a benchmark so that a step's
    inputs are not left in the on-chip caches by the previous step."""
    sp = case.spec
    rng = np.random.Generator(np.random.PCG64([sp.seed, 1000 + index]))
    g = _draw_logits(sp, rng, case.row_starts, case.row_ends)
    q = _draw_bf16_normal(rng, case.q.shape, 1.0)
    return shard_layout(g, sp.shards, sp.interleave, SENTINEL), q
