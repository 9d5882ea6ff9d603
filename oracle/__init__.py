"""CPU oracle for the DSA sparse-attention path — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct NumPy (float64) statement of what each step
of the path computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call it.  The product path
(``sparse_attention_indexer_topk_amd``) never imports it, and this package
imports nothing from the product path: the two share no code.  Inputs come
from ``dsa_inputs`` as raw bits and are decoded here by this package's own
format routines.

Sources (the pages are HTML-extracted reports of three vLLM pull requests):

* "PR #46076 [Attention][DSA] support dcp for FLASHINFER_MLA_SPARSE"
  (prhub report) — decode context parallel (DCP) top-K merge, index
  conversion, LSE base normalisation;
* "PR #40996 DCP supports hybrid attention" (prhub report) — rank-invariant
  collective gating, block-table width under DCP;
* "PR #52046" (prhub report, DSV3.2 prefill context parallel) — the fused
  RMSNorm + RoPE kernel, materialise/insert, combine of partials.

Module map:

* ``maps``      — shard ownership / local / global index maps, local counts;
* ``select``    — per-shard stable top-K with candidate packing, global
                  merge, global-to-local index conversion with compaction;
* ``attention`` — sparse MLA partial attention with base-e LSE, LSE combine;
* ``prologue``  — RMSNorm + interleaved-pair RoPE, cache insert; the same
                  for the indexer key (materialise, fp8 indexer-cache insert);
* ``formats``   — bf16 and fp8 e4m3 encode/decode written from their
                  definitions.

Every function is pinned by ``tests/test_oracle_*.py`` against brute force,
closed forms, library special cases and the pages' worked example.  Results
that no such check can pin are marked "parity unpinned" where they occur.
"""
from .maps import owner, local, global_id, local_count
from .select import topk_select, merge_candidates, convert_index, unsharded_topk
from .attention import sparse_mla_partial, lse_combine, attention_over_ids
from .prologue import rmsnorm_rope, cache_insert, index_norm_rope, index_cache_insert
from . import formats

__all__ = [
    "owner", "local", "global_id", "local_count",
    "topk_select", "merge_candidates", "convert_index", "unsharded_topk",
    "sparse_mla_partial", "lse_combine", "attention_over_ids",
    "rmsnorm_rope", "cache_insert", "index_norm_rope", "index_cache_insert", "formats",
]
