"""Python binding of ``libdsa.so`` — the MI355X DSA sparse-attention library.

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI declared in ``include/dsa.h``.  PyTorch provides device
memory and the current stream; there is no CPU fallback — if the library is
missing or the tensors are not on the GPU the call raises.

Functions (same names as the C entry points without the ``dsa_`` prefix):
``topk_select``, ``merge_candidates``, ``convert_index``,
``sparse_mla_decode``, ``lse_combine``, ``fused_rmsnorm_rope``.
Outputs may be passed in (written in place) or are allocated and returned.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdsa.so")

DSA_OK = 0
DSA_ERR_INVALID_ARG = -1
DSA_ERR_UNSUPPORTED_K = -2
DSA_ERR_UNSUPPORTED_DTYPE = -3
DSA_ERR_HIP = -4
DSA_BF16, DSA_FP32, DSA_FP8_E4M3 = 1, 2, 3

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F32 = ctypes.c_float

# C signatures (argument types), in header order
SIGNATURES = {
    "dsa_topk_select": [_P, _I64, _I64, _I32, _I32, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _P],
    "dsa_merge_candidates": [_P, _I32, _I32, _I32, _I32, _P, _P],
    "dsa_convert_index": [_P, _I32, _I32, _P, _I32, _P, _I64, _I64, _I32, _I32, _I32, _I32, _I32,
                          _P, _P, _P],
    "dsa_merge_convert": [_P, _I32, _I32, _I32, _I32, _P, _P, _I32, _P, _I64, _I64, _I32, _I32,
                          _I32, _I32, _I32, _P, _P, _P],
    "dsa_sparse_mla_decode": [_P, _I32, _I32, _P, _I32, _P, _I64, _P, _P, _I32, _I32, _I32, _F32,
                              _P, _P, _P],
    "dsa_lse_combine": [_P, _P, _I32, _I32, _I32, _I32, _P, _P, _P],
    "dsa_fused_rmsnorm_rope": [_P, _I64, _P, _I64, _I32, _P, _F32, _P, _I32, _P, _P, _P, _P, _I32, _P,
                               _P, _I64, _P],
    "dsa_cache_insert": [_P, _I64, _P, _I64, _I32, _P, _I32, _P, _P, _I64, _P],
    "dsa_last_error": [],
    "dsa_version": [],
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load ``libdsa.so`` (built in-tree); raise if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m sparse_attention_indexer_topk_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_char_p if name == "dsa_last_error" else ctypes.c_int
        _lib = L
    return _lib


class DSAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[status {status}] {message}")
        self.status = status


def _check(status: int):
    if status != DSA_OK:
        raise DSAError(status, lib().dsa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _need(t: torch.Tensor, name: str, dtype=None, last_contig=True):
    if not isinstance(t, torch.Tensor):
        raise RuntimeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise RuntimeError(f"{name} must be a GPU tensor (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise RuntimeError(f"{name} must be {dtype} (got {t.dtype})")
    if last_contig and t.dim() > 0 and t.stride(-1) != 1:
        raise RuntimeError(f"{name} must have a unit innermost stride")


def _bits16(t: torch.Tensor, name: str) -> torch.Tensor:
    """bf16 tensors may arrive as torch.bfloat16 or as raw int16/uint16 bits."""
    _need(t, name)
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise RuntimeError(f"{name} must be bf16 (got {t.dtype})")
    return t


def version() -> int:
    return lib().dsa_version()


# ---------------------------------------------------------------------------
def topk_select(logits: torch.Tensor, k: int, *, ctx: int, num_shards: int, interleave: int,
                row_starts: Optional[torch.Tensor] = None, row_ends: Optional[torch.Tensor] = None,
                shard_first: int = 0, local_idx: Optional[torch.Tensor] = None,
                cand: Optional[torch.Tensor] = None, want_local_idx: bool = True,
                want_cand: bool = True, stream=None):
    """Per-shard top-K + candidate pack.  ``logits``: [shard_count][rows][ld] fp32."""
    _need(logits, "logits", torch.float32)
    if logits.dim() != 3:
        raise RuntimeError("logits must be [shard_count][rows][ld]")
    count, rows, _ = logits.shape
    for name, t in (("row_starts", row_starts), ("row_ends", row_ends)):
        if t is not None:
            _need(t, name, torch.int32)
    dev = logits.device
    if local_idx is None and want_local_idx:
        local_idx = torch.empty((count, rows, k), dtype=torch.int32, device=dev)
    if cand is None and want_cand:
        cand = torch.empty((rows, num_shards * k, 2), dtype=torch.float32, device=dev)
    if local_idx is not None:
        _need(local_idx, "local_idx", torch.int32)
    if cand is not None:
        _need(cand, "cand", torch.float32)
    _check(lib().dsa_topk_select(
        _ptr(logits), logits.stride(1), logits.stride(0) if count > 1 else rows * logits.stride(1),
        rows, ctx, _ptr(row_starts), _ptr(row_ends), k, num_shards, interleave, shard_first, count,
        _ptr(local_idx), _ptr(cand), _stream(stream)))
    return local_idx, cand


def merge_candidates(cand: torch.Tensor, k: int, *, id_bound: int,
                     ids: Optional[torch.Tensor] = None, stream=None):
    """Global stable top-K over ``cand`` [rows][n_cand][2] fp32 -> ids [rows][k]."""
    _need(cand, "cand", torch.float32)
    if not cand.is_contiguous():
        raise RuntimeError("cand must be contiguous")
    rows, n_cand, _ = cand.shape
    if ids is None:
        ids = torch.empty((rows, k), dtype=torch.int32, device=cand.device)
    _need(ids, "ids", torch.int32)
    _check(lib().dsa_merge_candidates(_ptr(cand), rows, n_cand, k, id_bound, _ptr(ids),
                                      _stream(stream)))
    return ids


def merge_convert(cand: torch.Tensor, k: int, block_table: torch.Tensor, *, id_bound: int,
                  block_size: int, num_shards: int, interleave: int,
                  row_req: Optional[torch.Tensor] = None, shard_first: int = 0,
                  ids: Optional[torch.Tensor] = None, slots: Optional[torch.Tensor] = None,
                  counts: Optional[torch.Tensor] = None, want_ids: bool = True, stream=None):
    """merge_candidates then convert_index in one launch.

    cand [rows][n_cand][2] fp32 -> (ids [rows][k] or None, slots
    [shard_count][rows][k], counts [shard_count][rows]).
    """
    _need(cand, "cand", torch.float32)
    _need(block_table, "block_table", torch.int32)
    if not cand.is_contiguous():
        raise RuntimeError("cand must be contiguous")
    rows, n_cand, _ = cand.shape
    count, num_reqs, _ = block_table.shape
    if row_req is not None:
        _need(row_req, "row_req", torch.int32)
    if ids is None and want_ids:
        ids = torch.empty((rows, k), dtype=torch.int32, device=cand.device)
    if ids is not None:
        _need(ids, "ids", torch.int32)
    if slots is None:
        slots = torch.empty((count, rows, k), dtype=torch.int32, device=cand.device)
    if counts is None:
        counts = torch.empty((count, rows), dtype=torch.int32, device=cand.device)
    _need(slots, "slots", torch.int32)
    _need(counts, "counts", torch.int32)
    _check(lib().dsa_merge_convert(
        _ptr(cand), rows, n_cand, k, id_bound, _ptr(ids), _ptr(row_req), num_reqs,
        _ptr(block_table), block_table.stride(1),
        block_table.stride(0) if count > 1 else num_reqs * block_table.stride(1), block_size,
        num_shards, interleave, shard_first, count, _ptr(slots), _ptr(counts), _stream(stream)))
    return ids, slots, counts


def convert_index(ids: torch.Tensor, block_table: torch.Tensor, *, block_size: int,
                  num_shards: int, interleave: int, row_req: Optional[torch.Tensor] = None,
                  shard_first: int = 0, slots: Optional[torch.Tensor] = None,
                  counts: Optional[torch.Tensor] = None, stream=None):
    """ids [rows][k] -> slots [shard_count][rows][k], counts [shard_count][rows]."""
    _need(ids, "ids", torch.int32)
    _need(block_table, "block_table", torch.int32)
    if not ids.is_contiguous():
        raise RuntimeError("ids must be contiguous")
    rows, k = ids.shape
    count, num_reqs, _ = block_table.shape
    if row_req is not None:
        _need(row_req, "row_req", torch.int32)
    if slots is None:
        slots = torch.empty((count, rows, k), dtype=torch.int32, device=ids.device)
    if counts is None:
        counts = torch.empty((count, rows), dtype=torch.int32, device=ids.device)
    _need(slots, "slots", torch.int32)
    _need(counts, "counts", torch.int32)
    _check(lib().dsa_convert_index(
        _ptr(ids), rows, k, _ptr(row_req), num_reqs, _ptr(block_table), block_table.stride(1),
        block_table.stride(0) if count > 1 else num_reqs * block_table.stride(1), block_size,
        num_shards, interleave, shard_first, count, _ptr(slots), _ptr(counts), _stream(stream)))
    return slots, counts


def sparse_mla_decode(q: torch.Tensor, cache: torch.Tensor, slots: torch.Tensor,
                      counts: Optional[torch.Tensor], *, sm_scale: float, splits: int = 1,
                      cache_scale: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      stream=None):
    """q [rows][heads][576] bf16; cache [...][576] bf16 or uint8 (fp8 e4m3 codes);
    slots [n_parts][rows][k]; returns out [n_parts*splits][rows][heads][512]
    bf16 and lse [n_parts*splits][rows][heads] fp32 (split-K partials of part p
    are p*splits .. p*splits + splits - 1)."""
    _bits16(q, "q")
    _need(cache, "cache")
    _need(slots, "slots", torch.int32)
    if not (q.is_contiguous() and cache.is_contiguous() and slots.is_contiguous()):
        raise RuntimeError("q, cache and slots must be contiguous")
    rows, heads, _ = q.shape
    n_parts, _, k = slots.shape
    if cache.dtype in (torch.uint8, torch.float8_e4m3fn):
        cdt = DSA_FP8_E4M3
        if cache_scale is None:
            raise RuntimeError("an fp8 cache needs cache_scale")
        _need(cache_scale, "cache_scale", torch.float32)
    else:
        _bits16(cache, "cache")
        cdt = DSA_BF16
    num_slots = cache.numel() // 576
    if counts is not None:
        _need(counts, "counts", torch.int32)
    if out is None:
        out = torch.empty((n_parts * splits, rows, heads, 512), dtype=torch.bfloat16,
                          device=q.device)
    if lse is None:
        lse = torch.empty((n_parts * splits, rows, heads), dtype=torch.float32, device=q.device)
    _bits16(out, "out")
    _need(lse, "lse", torch.float32)
    _check(lib().dsa_sparse_mla_decode(
        _ptr(q), rows, heads, _ptr(cache), cdt, _ptr(cache_scale), num_slots, _ptr(slots),
        _ptr(counts), k, n_parts, int(splits), float(sm_scale), _ptr(out), _ptr(lse),
        _stream(stream)))
    return out, lse


def lse_combine(part_out: torch.Tensor, part_lse: torch.Tensor, *,
                out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None,
                want_lse: bool = True, stream=None):
    """part_out [n_parts][rows][heads][dim] bf16, part_lse [n_parts][rows][heads]."""
    _bits16(part_out, "part_out")
    _need(part_lse, "part_lse", torch.float32)
    if not (part_out.is_contiguous() and part_lse.is_contiguous()):
        raise RuntimeError("partials must be contiguous")
    n_parts, rows, heads, dim = part_out.shape
    if out is None:
        out = torch.empty((rows, heads, dim), dtype=torch.bfloat16, device=part_out.device)
    if lse_out is None and want_lse:
        lse_out = torch.empty((rows, heads), dtype=torch.float32, device=part_out.device)
    _check(lib().dsa_lse_combine(_ptr(part_out), _ptr(part_lse), n_parts, rows, heads, dim,
                                 _ptr(out), _ptr(lse_out), _stream(stream)))
    return out, lse_out


def fused_rmsnorm_rope(kv_c: torch.Tensor, k_pe: torch.Tensor, rms_w: torch.Tensor, eps: float,
                       cos_sin: torch.Tensor, positions: torch.Tensor, *,
                       kv_c_out: Optional[torch.Tensor] = None,
                       k_pe_out: Optional[torch.Tensor] = None,
                       cache: Optional[torch.Tensor] = None,
                       cache_scale: Optional[torch.Tensor] = None,
                       slot_mapping: Optional[torch.Tensor] = None, stream=None):
    """RMSNorm(kv_c) + RoPE(k_pe); writes the given outputs and/or inserts into
    ``cache`` at ``slot_mapping``.  Returns (kv_c_out, k_pe_out)."""
    _bits16(kv_c, "kv_c")
    _bits16(k_pe, "k_pe")
    _bits16(rms_w, "rms_w")
    _need(cos_sin, "cos_sin", torch.float32)
    _need(positions, "positions", torch.int32)
    T = kv_c.shape[0]
    cdt, num_slots = 0, 0
    if slot_mapping is not None:
        _need(slot_mapping, "slot_mapping", torch.int64)
        if cache is None:
            raise RuntimeError("slot_mapping needs a cache")
        cdt = DSA_FP8_E4M3 if cache.dtype in (torch.uint8, torch.float8_e4m3fn) else DSA_BF16
        num_slots = cache.numel() // 576
    _check(lib().dsa_fused_rmsnorm_rope(
        _ptr(kv_c), kv_c.stride(0), _ptr(k_pe), k_pe.stride(0), T, _ptr(rms_w), float(eps),
        _ptr(cos_sin), cos_sin.shape[0], _ptr(positions), _ptr(kv_c_out), _ptr(k_pe_out),
        _ptr(cache), cdt, _ptr(cache_scale), _ptr(slot_mapping), num_slots, _stream(stream)))
    return kv_c_out, k_pe_out


def cache_insert(kv_c: torch.Tensor, k_pe: torch.Tensor, cache: torch.Tensor,
                 slot_mapping: torch.Tensor, *, cache_scale: Optional[torch.Tensor] = None,
                 stream=None):
    """Write materialised K rows (kv_c [T][512], k_pe [T][64] bf16) into ``cache``
    at ``slot_mapping`` (bf16, or fp8 e4m3 scaled by ``cache_scale``)."""
    _bits16(kv_c, "kv_c")
    _bits16(k_pe, "k_pe")
    _need(slot_mapping, "slot_mapping", torch.int64)
    T = kv_c.shape[0]
    cdt = DSA_FP8_E4M3 if cache.dtype in (torch.uint8, torch.float8_e4m3fn) else DSA_BF16
    _check(lib().dsa_cache_insert(
        _ptr(kv_c), kv_c.stride(0), _ptr(k_pe), k_pe.stride(0), T, _ptr(cache), cdt,
        _ptr(cache_scale), _ptr(slot_mapping), cache.numel() // 576, _stream(stream)))


__all__ = ["lib", "version", "DSAError", "topk_select", "merge_candidates", "convert_index",
           "merge_convert", "sparse_mla_decode", "lse_combine", "fused_rmsnorm_rope",
           "cache_insert", "LIB_PATH", "SIGNATURES"]
