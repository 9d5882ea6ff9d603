"""One DCP decode step of the DSA path over device-resident buffers.

The step is the sequence of library calls the decode-context-parallel path
makes ([A]: PR #46076 report, 实现拆解 items 1-5; [C]: PR #52046 report,
关键源码片段), with every shard emulated as a slice of one buffer:

  fused_rmsnorm_rope (optional: new K rows materialised and inserted; in the
  sequence-sharded (PCP) form each rank materialises its rows, the rows are
  gathered and cache_insert writes them all)
  -> topk_select (all shards, one launch; writes the gathered candidates)
  -> merge_candidates + convert_index (all shards; one launch, merge_convert)
  -> sparse_mla_decode (all shards, one launch) -> lse_combine.

Only sequencing and buffer ownership live here; the arithmetic is in the HIP
kernels behind ``libdsa.so``.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import (topk_select, merge_candidates, convert_index, merge_convert, sparse_mla_decode,
               lse_combine, fused_rmsnorm_rope, cache_insert)


@dataclasses.dataclass
class Prologue:
    kv_c: torch.Tensor          # [T][512] bf16
    k_pe: torch.Tensor          # [T][64] bf16
    rms_w: torch.Tensor         # [512] bf16
    eps: float
    cos_sin: torch.Tensor       # [n_pos][64] fp32
    positions: torch.Tensor     # [T] int32
    slot_mapping: torch.Tensor  # [T] int64
    # indexer-key branch of the same launch (all None: not run)
    index_k: Optional[torch.Tensor] = None            # [T][128] bf16
    index_w: Optional[torch.Tensor] = None            # [128] bf16
    index_eps: float = 1e-6
    index_cache: Optional[torch.Tensor] = None        # [slots][128] fp8 e4m3 codes
    index_cache_scale: Optional[torch.Tensor] = None  # [1] fp32


class DecodePath:
    """Holds the inputs and every intermediate of one step on the GPU."""

    def __init__(self, *, logits: torch.Tensor, row_starts: Optional[torch.Tensor],
                 row_ends: Optional[torch.Tensor], ctx: int, k: int, num_shards: int,
                 interleave: int, q: torch.Tensor, cache: torch.Tensor,
                 cache_scale: Optional[torch.Tensor], block_table: torch.Tensor,
                 row_req: Optional[torch.Tensor], sm_scale: float, block_size: int = 64,
                 prologue=None, splits: Optional[int] = None, pcp_ranks: int = 0):
        self.logits, self.row_starts, self.row_ends = logits, row_starts, row_ends
        self.ctx, self.k, self.S, self.I = ctx, k, num_shards, interleave
        self.q, self.cache, self.cache_scale = q, cache, cache_scale
        self.block_table, self.row_req = block_table, row_req
        self.sm_scale, self.block_size = sm_scale, block_size
        if isinstance(prologue, dict):
            prologue = Prologue(**prologue)
        self.prologue = prologue
        # pcp_ranks > 0: the sequence-sharded (PCP) prologue -- each rank
        # materialises its slice of the new K rows into the gathered buffer
        # (the all-gather, in place), then every row is inserted
        self.pcp_ranks = pcp_ranks
        # the merged global ids are written out only when wanted: the
        # per-shard slot lists the attention reads are derived without them
        self.want_ids = True
        dev = logits.device
        R, H = q.shape[0], q.shape[1]
        S = num_shards
        if splits is None:   # enough workgroups to cover the 256 CUs
            blocks = R * S * ((H + 127) // 128)
            splits = max(1, min(8, -(-256 // blocks)))
        # the combine merges at most 64 partials per (row, head)
        splits = max(1, min(splits, 64 // S))
        self.splits = splits
        self.cand = torch.empty((R, S * k, 2), dtype=torch.float32, device=dev)
        self.local_idx = torch.empty((S, R, k), dtype=torch.int32, device=dev)
        self.ids = torch.empty((R, k), dtype=torch.int32, device=dev)
        self.slots = torch.empty((S, R, k), dtype=torch.int32, device=dev)
        self.counts = torch.empty((S, R), dtype=torch.int32, device=dev)
        self.pout = torch.empty((S * splits, R, H, 512), dtype=torch.bfloat16, device=dev)
        self.plse = torch.empty((S * splits, R, H), dtype=torch.float32, device=dev)
        self.out = torch.empty((R, H, 512), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((R, H), dtype=torch.float32, device=dev)
        self.index_k_out = None
        if prologue is not None:
            T = prologue.kv_c.shape[0]
            self.kv_c_out = torch.empty((T, 512), dtype=torch.bfloat16, device=dev)
            self.k_pe_out = torch.empty((T, 64), dtype=torch.bfloat16, device=dev)
            if prologue.index_k is not None:
                self.index_k_out = torch.empty((T, 128), dtype=torch.bfloat16, device=dev)

    # -- steps ---------------------------------------------------------------
    def run_prologue(self, stream=None):
        p = self.prologue
        ix = p.index_k is not None
        if self.pcp_ranks <= 0:
            fused_rmsnorm_rope(p.kv_c, p.k_pe, p.rms_w, p.eps, p.cos_sin, p.positions,
                               kv_c_out=self.kv_c_out, k_pe_out=self.k_pe_out,
                               cache=self.cache, cache_scale=self.cache_scale,
                               slot_mapping=p.slot_mapping, index_k=p.index_k,
                               index_w=p.index_w, index_eps=p.index_eps,
                               index_k_out=self.index_k_out, index_cache=p.index_cache,
                               index_cache_scale=p.index_cache_scale, stream=stream)
            return
        # sequence-sharded: every rank materialises its rows (the indexer key
        # too, with no indexer-cache insert: the indexer takes the materialised
        # keys), the rows are gathered, and the replicated cache is updated
        T = p.kv_c.shape[0]
        bounds = [T * r // self.pcp_ranks for r in range(self.pcp_ranks + 1)]
        for a, b in zip(bounds[:-1], bounds[1:]):   # rank r materialises rows [a, b)
            if b > a:
                fused_rmsnorm_rope(p.kv_c[a:b], p.k_pe[a:b], p.rms_w, p.eps, p.cos_sin,
                                   p.positions[a:b], kv_c_out=self.kv_c_out[a:b],
                                   k_pe_out=self.k_pe_out[a:b],
                                   index_k=p.index_k[a:b] if ix else None, index_w=p.index_w,
                                   index_eps=p.index_eps,
                                   index_k_out=self.index_k_out[a:b] if ix else None,
                                   stream=stream)
        cache_insert(self.kv_c_out, self.k_pe_out, self.cache, p.slot_mapping,
                     cache_scale=self.cache_scale, stream=stream)

    def run_topk(self, stream=None, with_local_idx=False, logits=None):
        topk_select(self.logits if logits is None else logits, self.k, ctx=self.ctx,
                    num_shards=self.S, interleave=self.I, row_starts=self.row_starts,
                    row_ends=self.row_ends, local_idx=self.local_idx if with_local_idx else None,
                    cand=self.cand, want_local_idx=with_local_idx, stream=stream)

    def run_merge(self, stream=None):
        merge_candidates(self.cand, self.k, id_bound=self.ctx, ids=self.ids, stream=stream)

    def run_convert(self, stream=None):
        convert_index(self.ids, self.block_table, block_size=self.block_size, num_shards=self.S,
                      interleave=self.I, row_req=self.row_req, slots=self.slots,
                      counts=self.counts, stream=stream)

    def run_merge_convert(self, stream=None):
        merge_convert(self.cand, self.k, self.block_table, id_bound=self.ctx,
                      block_size=self.block_size, num_shards=self.S, interleave=self.I,
                      row_req=self.row_req, ids=self.ids if self.want_ids else None,
                      want_ids=self.want_ids, slots=self.slots, counts=self.counts,
                      stream=stream)

    def run_attention(self, stream=None, q=None):
        sparse_mla_decode(self.q if q is None else q, self.cache, self.slots, self.counts,
                          sm_scale=self.sm_scale, splits=self.splits,
                          cache_scale=self.cache_scale, out=self.pout,
                          lse=self.plse, stream=stream)

    def run_combine(self, stream=None):
        lse_combine(self.pout, self.plse, out=self.out, lse_out=self.lse, stream=stream)

    def step(self, stream=None, with_local_idx=False):
        if self.prologue is not None:
            self.run_prologue(stream)
        self.run_topk(stream, with_local_idx)
        self.run_merge_convert(stream)
        self.run_attention(stream)
        self.run_combine(stream)
