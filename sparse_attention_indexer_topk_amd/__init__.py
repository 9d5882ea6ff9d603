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
                              _P, _I32, _P, _P],
    "dsa_lse_combine": [_P, _I32, _P, _I32, _I32, _I32, _I32, _P, _P, _P],
    "dsa_fused_rmsnorm_rope": [_P, _I64, _P, _I64, _I32, _P, _F32, _P, _I32, _P, _P, _P, _P, _I32, _P,
                               _P, _I64, _P, _I64, _P, _F32, _P, _P, _P, _I64, _P],
    "dsa_cache_insert": [_P, _I64, _P, _I64, _I32, _P, _I32, _P, _P, _I64, _P],
    "dsa_launch_floor": [_I32, _I32, _P],
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


def _partial_dtype(t: torch.Tensor, name: str) -> int:
    """Partial outputs are bf16 (or its raw 16-bit bits) or fp32."""
    _need(t, name)
    if t.dtype == torch.float32:
        return DSA_FP32
    _bits16(t, name)
    return DSA_BF16


def _shape(t: torch.Tensor, name: str, shape):
    """``shape``: expected sizes, None = any."""
    if t.dim() != len(shape) or any(e is not None and a != e for a, e in zip(t.shape, shape)):
        want = "[" + "][".join("*" if e is None else str(e) for e in shape) + "]"
        raise RuntimeError(f"{name} must be {want} (got {list(t.shape)})")


def _contig(t: torch.Tensor, name: str):
    if not t.is_contiguous():
        raise RuntimeError(f"{name} must be contiguous")


def _row_major(t: torch.Tensor, name: str):
    """Rows may be strided (a leading dimension), elements of a row may not;
    the leading strides must not make rows overlap."""
    if t.dim() > 0 and t.stride(-1) != 1:
        raise RuntimeError(f"{name} must have a unit innermost stride")
    for d in range(t.dim() - 1):
        inner = t.stride(d + 1) * t.shape[d + 1] if d + 1 < t.dim() else 1
        if t.shape[d] > 1 and t.stride(d) < inner:
            raise RuntimeError(f"{name}: dimension {d} overlaps the next (stride {t.stride(d)})")


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise RuntimeError(f"tensors are on different devices: {sorted(map(str, devs))}")


def launch_floor(workgroups: int, threads: int, stream=None):
    """Launch an empty kernel of the given grid shape (a measurement helper)."""
    _check(lib().dsa_launch_floor(int(workgroups), int(threads), _stream(stream)))


def version() -> int:
    return lib().dsa_version()


# ---------------------------------------------------------------------------
# Every wrapper checks dtype, device, shape, length and contiguity against
# what the kernels index before it calls the library, so a mis-sized tensor
# raises here instead of becoming an out-of-bounds device access.

def _check_block_table(block_table: torch.Tensor):
    _need(block_table, "block_table", torch.int32)
    if block_table.dim() != 3:
        raise RuntimeError("block_table must be [shard_count][num_reqs][width]")
    # the kernels take the row stride as the table width
    if block_table.stride(1) != block_table.shape[2]:
        raise RuntimeError("block_table rows must be dense (row stride == width)")
    _row_major(block_table, "block_table")


def _bt_shard_stride(block_table: torch.Tensor) -> int:
    count, num_reqs, width = block_table.shape
    return block_table.stride(0) if count > 1 else num_reqs * width


def _check_slot_outputs(slots, counts, count, rows, k):
    _need(slots, "slots", torch.int32)
    _shape(slots, "slots", (count, rows, k))
    _contig(slots, "slots")
    if counts is not None:
        _need(counts, "counts", torch.int32)
        _shape(counts, "counts", (count, rows))
        _contig(counts, "counts")


def _check_cand(cand: torch.Tensor, name="cand"):
    _need(cand, name, torch.float32)
    if cand.dim() != 3 or cand.shape[2] != 2:
        raise RuntimeError(f"{name} must be [rows][n_cand][2] (got {list(cand.shape)})")
    _contig(cand, name)


def _check_row_vec(t, name, rows, dtype=torch.int32):
    if t is not None:
        _need(t, name, dtype)
        _shape(t, name, (rows,))
        _contig(t, name)


def _check_cache(cache: torch.Tensor):
    _need(cache, "cache")
    if cache.dim() < 1 or cache.shape[-1] != 576:
        raise RuntimeError(f"cache entries must be 576 wide (got {list(cache.shape)})")
    _contig(cache, "cache")
    if cache.dtype in (torch.uint8, torch.float8_e4m3fn):
        return DSA_FP8_E4M3
    _bits16(cache, "cache")
    return DSA_BF16


def _check_scale(cache_scale, cdt):
    if cdt == DSA_FP8_E4M3:
        if cache_scale is None:
            raise RuntimeError("an fp8 cache needs cache_scale")
        _need(cache_scale, "cache_scale", torch.float32)
        if cache_scale.numel() < 1:
            raise RuntimeError("cache_scale must hold one value")


def topk_select(logits: torch.Tensor, k: int, *, ctx: int, num_shards: int, interleave: int,
                row_starts: Optional[torch.Tensor] = None, row_ends: Optional[torch.Tensor] = None,
                shard_first: int = 0, local_idx: Optional[torch.Tensor] = None,
                cand: Optional[torch.Tensor] = None, want_local_idx: bool = True,
                want_cand: bool = True, stream=None):
    """Per-shard top-K + candidate pack.  ``logits``: [shard_count][rows][ld] fp32."""
    _need(logits, "logits", torch.float32)
    if logits.dim() != 3:
        raise RuntimeError("logits must be [shard_count][rows][ld]")
    _row_major(logits, "logits")
    # the kernel takes the row stride as the row length (and may read up to
    # it with 16-byte loads), so rows must be dense
    if logits.stride(1) != logits.shape[2]:
        raise RuntimeError("logits rows must be dense (row stride == ld)")
    count, rows, _ = logits.shape
    _check_row_vec(row_starts, "row_starts", rows)
    _check_row_vec(row_ends, "row_ends", rows)
    dev = logits.device
    if local_idx is None and want_local_idx:
        local_idx = torch.empty((count, rows, k), dtype=torch.int32, device=dev)
    if cand is None and want_cand:
        cand = torch.empty((rows, num_shards * k, 2), dtype=torch.float32, device=dev)
    if local_idx is not None:
        _need(local_idx, "local_idx", torch.int32)
        _shape(local_idx, "local_idx", (count, rows, k))
        _contig(local_idx, "local_idx")
    if cand is not None:
        _check_cand(cand)
        _shape(cand, "cand", (rows, num_shards * k, 2))
    _same_device(logits, row_starts, row_ends, local_idx, cand)
    _check(lib().dsa_topk_select(
        _ptr(logits), logits.stride(1), logits.stride(0) if count > 1 else rows * logits.stride(1),
        rows, ctx, _ptr(row_starts), _ptr(row_ends), k, num_shards, interleave, shard_first, count,
        _ptr(local_idx), _ptr(cand), _stream(stream)))
    return local_idx, cand


def merge_candidates(cand: torch.Tensor, k: int, *, id_bound: int,
                     ids: Optional[torch.Tensor] = None, stream=None):
    """Global stable top-K over ``cand`` [rows][n_cand][2] fp32 -> ids [rows][k]."""
    _check_cand(cand)
    rows, n_cand, _ = cand.shape
    if ids is None:
        ids = torch.empty((rows, k), dtype=torch.int32, device=cand.device)
    _need(ids, "ids", torch.int32)
    _shape(ids, "ids", (rows, k))
    _contig(ids, "ids")
    _same_device(cand, ids)
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
    _check_cand(cand)
    _check_block_table(block_table)
    rows, n_cand, _ = cand.shape
    count, num_reqs, _ = block_table.shape
    _check_row_vec(row_req, "row_req", rows)
    if ids is None and want_ids:
        ids = torch.empty((rows, k), dtype=torch.int32, device=cand.device)
    if ids is not None:
        _need(ids, "ids", torch.int32)
        _shape(ids, "ids", (rows, k))
        _contig(ids, "ids")
    if slots is None:
        slots = torch.empty((count, rows, k), dtype=torch.int32, device=cand.device)
    if counts is None:
        counts = torch.empty((count, rows), dtype=torch.int32, device=cand.device)
    _check_slot_outputs(slots, counts, count, rows, k)
    _same_device(cand, block_table, row_req, ids, slots, counts)
    _check(lib().dsa_merge_convert(
        _ptr(cand), rows, n_cand, k, id_bound, _ptr(ids), _ptr(row_req), num_reqs,
        _ptr(block_table), block_table.stride(1), _bt_shard_stride(block_table), block_size,
        num_shards, interleave, shard_first, count, _ptr(slots), _ptr(counts), _stream(stream)))
    return ids, slots, counts


def convert_index(ids: torch.Tensor, block_table: torch.Tensor, *, block_size: int,
                  num_shards: int, interleave: int, row_req: Optional[torch.Tensor] = None,
                  shard_first: int = 0, slots: Optional[torch.Tensor] = None,
                  counts: Optional[torch.Tensor] = None, stream=None):
    """ids [rows][k] -> slots [shard_count][rows][k], counts [shard_count][rows]."""
    _need(ids, "ids", torch.int32)
    if ids.dim() != 2:
        raise RuntimeError("ids must be [rows][k]")
    _contig(ids, "ids")
    _check_block_table(block_table)
    rows, k = ids.shape
    count, num_reqs, _ = block_table.shape
    _check_row_vec(row_req, "row_req", rows)
    if slots is None:
        slots = torch.empty((count, rows, k), dtype=torch.int32, device=ids.device)
    if counts is None:
        counts = torch.empty((count, rows), dtype=torch.int32, device=ids.device)
    _check_slot_outputs(slots, counts, count, rows, k)
    _same_device(ids, block_table, row_req, slots, counts)
    _check(lib().dsa_convert_index(
        _ptr(ids), rows, k, _ptr(row_req), num_reqs, _ptr(block_table), block_table.stride(1),
        _bt_shard_stride(block_table), block_size, num_shards, interleave, shard_first, count,
        _ptr(slots), _ptr(counts), _stream(stream)))
    return slots, counts


def sparse_mla_decode(q: torch.Tensor, cache: torch.Tensor, slots: torch.Tensor,
                      counts: Optional[torch.Tensor], *, sm_scale: float, splits: int = 1,
                      cache_scale: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      out_dtype: torch.dtype = torch.bfloat16, stream=None):
    """q [rows][heads][576] bf16; cache [...][576] bf16 or uint8 (fp8 e4m3 codes);
    slots [n_parts][rows][k]; returns out [n_parts*splits][rows][heads][512]
    and lse [n_parts*splits][rows][heads] fp32 (split-K partials of part p
    are p*splits .. p*splits + splits - 1).  out is bf16, or fp32 (the
    checking mode without the bf16 rounding) when out_dtype is torch.float32
    or a given `out` is fp32."""
    _bits16(q, "q")
    if q.dim() != 3 or q.shape[2] != 576:
        raise RuntimeError(f"q must be [rows][heads][576] (got {list(q.shape)})")
    _contig(q, "q")
    cdt = _check_cache(cache)
    _check_scale(cache_scale, cdt)
    _need(slots, "slots", torch.int32)
    if slots.dim() != 3:
        raise RuntimeError("slots must be [n_parts][rows][k]")
    _contig(slots, "slots")
    rows, heads, _ = q.shape
    n_parts, s_rows, k = slots.shape
    if s_rows != rows:
        raise RuntimeError(f"slots has {s_rows} rows, q has {rows}")
    num_slots = cache.numel() // 576
    if counts is not None:
        _need(counts, "counts", torch.int32)
        _shape(counts, "counts", (n_parts, rows))
        _contig(counts, "counts")
    P = n_parts * int(splits)
    if out is None:
        if out_dtype not in (torch.bfloat16, torch.float32):
            raise RuntimeError(f"out_dtype must be bf16 or fp32 (got {out_dtype})")
        out = torch.empty((P, rows, heads, 512), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((P, rows, heads), dtype=torch.float32, device=q.device)
    odt = _partial_dtype(out, "out")
    _shape(out, "out", (P, rows, heads, 512))
    _contig(out, "out")
    _need(lse, "lse", torch.float32)
    _shape(lse, "lse", (P, rows, heads))
    _contig(lse, "lse")
    _same_device(q, cache, slots, counts, cache_scale, out, lse)
    _check(lib().dsa_sparse_mla_decode(
        _ptr(q), rows, heads, _ptr(cache), cdt, _ptr(cache_scale), num_slots, _ptr(slots),
        _ptr(counts), k, n_parts, int(splits), float(sm_scale), _ptr(out), odt, _ptr(lse),
        _stream(stream)))
    return out, lse


def lse_combine(part_out: torch.Tensor, part_lse: torch.Tensor, *,
                out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None,
                want_lse: bool = True, stream=None):
    """part_out [n_parts][rows][heads][dim] bf16 (or fp32, the attention's
    checking mode), part_lse [n_parts][rows][heads]; out is bf16."""
    pdt = _partial_dtype(part_out, "part_out")
    _need(part_lse, "part_lse", torch.float32)
    if part_out.dim() != 4:
        raise RuntimeError("part_out must be [n_parts][rows][heads][dim]")
    _contig(part_out, "part_out")
    n_parts, rows, heads, dim = part_out.shape
    _shape(part_lse, "part_lse", (n_parts, rows, heads))
    _contig(part_lse, "part_lse")
    if out is None:
        out = torch.empty((rows, heads, dim), dtype=torch.bfloat16, device=part_out.device)
    if lse_out is None and want_lse:
        lse_out = torch.empty((rows, heads), dtype=torch.float32, device=part_out.device)
    _bits16(out, "out")
    _shape(out, "out", (rows, heads, dim))
    _contig(out, "out")
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32)
        _shape(lse_out, "lse_out", (rows, heads))
        _contig(lse_out, "lse_out")
    _same_device(part_out, part_lse, out, lse_out)
    _check(lib().dsa_lse_combine(_ptr(part_out), pdt, _ptr(part_lse), n_parts, rows, heads, dim,
                                 _ptr(out), _ptr(lse_out), _stream(stream)))
    return out, lse_out


def _check_rows_in(kv_c, k_pe):
    _bits16(kv_c, "kv_c")
    _bits16(k_pe, "k_pe")
    if kv_c.dim() != 2 or kv_c.shape[1] < 512:
        raise RuntimeError(f"kv_c must be [T][>=512] (got {list(kv_c.shape)})")
    if k_pe.dim() != 2 or k_pe.shape[1] < 64:
        raise RuntimeError(f"k_pe must be [T][>=64] (got {list(k_pe.shape)})")
    if k_pe.shape[0] != kv_c.shape[0]:
        raise RuntimeError(f"kv_c has {kv_c.shape[0]} rows, k_pe has {k_pe.shape[0]}")
    _row_major(kv_c, "kv_c")
    _row_major(k_pe, "k_pe")
    return kv_c.shape[0]


def fused_rmsnorm_rope(kv_c: Optional[torch.Tensor], k_pe: Optional[torch.Tensor],
                       rms_w: Optional[torch.Tensor], eps: float, cos_sin: torch.Tensor,
                       positions: torch.Tensor, *,
                       kv_c_out: Optional[torch.Tensor] = None,
                       k_pe_out: Optional[torch.Tensor] = None,
                       cache: Optional[torch.Tensor] = None,
                       cache_scale: Optional[torch.Tensor] = None,
                       slot_mapping: Optional[torch.Tensor] = None,
                       index_k: Optional[torch.Tensor] = None,
                       index_w: Optional[torch.Tensor] = None, index_eps: float = 1e-6,
                       index_k_out: Optional[torch.Tensor] = None,
                       index_cache: Optional[torch.Tensor] = None,
                       index_cache_scale: Optional[torch.Tensor] = None, stream=None):
    """Latent branch: RMSNorm(kv_c) + RoPE(k_pe), materialised into the given
    outputs and/or inserted into ``cache`` at ``slot_mapping``.  Indexer
    branch: the 128-wide indexer key normed and roped, materialised into
    ``index_k_out`` and/or inserted into the fp8 ``index_cache`` (only with a
    slot mapping).  Returns (kv_c_out, k_pe_out, index_k_out)."""
    _need(cos_sin, "cos_sin", torch.float32)
    _shape(cos_sin, "cos_sin", (None, 64))
    _contig(cos_sin, "cos_sin")
    _need(positions, "positions", torch.int32)
    if positions.dim() != 1:
        raise RuntimeError("positions must be [T]")
    _contig(positions, "positions")
    T = positions.shape[0]
    latent = (kv_c_out is not None or k_pe_out is not None
              or (slot_mapping is not None and cache is not None))
    indexer = index_k_out is not None or (slot_mapping is not None and index_cache is not None)
    if slot_mapping is not None:
        _check_row_vec(slot_mapping, "slot_mapping", T, torch.int64)
        if cache is None and index_cache is None:
            raise RuntimeError("slot_mapping needs a cache")
    if latent:
        if _check_rows_in(kv_c, k_pe) != T:
            raise RuntimeError(f"kv_c has {kv_c.shape[0]} rows, positions {T}")
        _bits16(rms_w, "rms_w")
        _shape(rms_w, "rms_w", (512,))
        _contig(rms_w, "rms_w")
    for name, t, w in (("kv_c_out", kv_c_out, 512), ("k_pe_out", k_pe_out, 64),
                       ("index_k_out", index_k_out, 128)):
        if t is not None:
            _bits16(t, name)
            _shape(t, name, (T, w))
            _contig(t, name)
    cdt, num_slots = 0, 0
    if slot_mapping is not None and cache is not None:
        cdt = _check_cache(cache)
        _check_scale(cache_scale, cdt)
        num_slots = cache.numel() // 576
    index_ld, index_slots = 0, 0
    if indexer:
        _bits16(index_k, "index_k")
        if index_k.dim() != 2 or index_k.shape[0] != T or index_k.shape[1] < 128:
            raise RuntimeError(f"index_k must be [T][>=128] (got {list(index_k.shape)})")
        _row_major(index_k, "index_k")
        index_ld = index_k.stride(0)
        _bits16(index_w, "index_w")
        _shape(index_w, "index_w", (128,))
        _contig(index_w, "index_w")
    if slot_mapping is not None and index_cache is not None:
        _need(index_cache, "index_cache")
        if index_cache.dtype not in (torch.uint8, torch.float8_e4m3fn) or index_cache.shape[-1] != 128:
            raise RuntimeError("index_cache must hold 128 fp8 e4m3 codes per slot")
        _contig(index_cache, "index_cache")
        _check_scale(index_cache_scale, DSA_FP8_E4M3)
        index_slots = index_cache.numel() // 128
    _same_device(kv_c if latent else None, k_pe if latent else None, rms_w if latent else None,
                 cos_sin, positions, kv_c_out, k_pe_out, cache, cache_scale, slot_mapping,
                 index_k if indexer else None, index_w if indexer else None, index_k_out,
                 index_cache, index_cache_scale)
    _check(lib().dsa_fused_rmsnorm_rope(
        _ptr(kv_c) if latent else None, kv_c.stride(0) if latent else 0,
        _ptr(k_pe) if latent else None, k_pe.stride(0) if latent else 0, T,
        _ptr(rms_w) if latent else None, float(eps), _ptr(cos_sin), cos_sin.shape[0],
        _ptr(positions), _ptr(kv_c_out), _ptr(k_pe_out), _ptr(cache), cdt, _ptr(cache_scale),
        _ptr(slot_mapping), num_slots, _ptr(index_k) if indexer else None, index_ld,
        _ptr(index_w) if indexer else None, float(index_eps), _ptr(index_k_out),
        _ptr(index_cache), _ptr(index_cache_scale), index_slots, _stream(stream)))
    return kv_c_out, k_pe_out, index_k_out


def cache_insert(kv_c: torch.Tensor, k_pe: torch.Tensor, cache: torch.Tensor,
                 slot_mapping: torch.Tensor, *, cache_scale: Optional[torch.Tensor] = None,
                 stream=None):
    """Write materialised K rows (kv_c [T][512], k_pe [T][64] bf16) into ``cache``
    at ``slot_mapping`` (bf16, or fp8 e4m3 scaled by ``cache_scale``)."""
    T = _check_rows_in(kv_c, k_pe)
    _check_row_vec(slot_mapping, "slot_mapping", T, torch.int64)
    cdt = _check_cache(cache)
    _check_scale(cache_scale, cdt)
    _same_device(kv_c, k_pe, cache, slot_mapping, cache_scale)
    _check(lib().dsa_cache_insert(
        _ptr(kv_c), kv_c.stride(0), _ptr(k_pe), k_pe.stride(0), T, _ptr(cache), cdt,
        _ptr(cache_scale), _ptr(slot_mapping), cache.numel() // 576, _stream(stream)))


__all__ = ["lib", "version", "DSAError", "topk_select", "merge_candidates", "convert_index",
           "merge_convert", "sparse_mla_decode", "lse_combine", "fused_rmsnorm_rope",
           "cache_insert", "launch_floor", "LIB_PATH", "SIGNATURES"]
