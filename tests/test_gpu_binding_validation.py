"""The binding refuses mis-shaped, mis-typed or strided tensors before it
calls the library: each bad call raises, and the output buffers it was given
keep their contents (no kernel ran)."""
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import sparse_attention_indexer_topk_amd as dsa  # noqa: E402

DEV = "cuda"
R, S, K, H = 3, 2, 512, 16
CTX = 2 * 1500


def i32(*shape, fill=-7):
    return torch.full(shape, fill, dtype=torch.int32, device=DEV)


def f32(*shape, fill=-7.0):
    return torch.full(shape, fill, dtype=torch.float32, device=DEV)


def bf(*shape):
    return torch.full(shape, 3.0, dtype=torch.bfloat16, device=DEV)


def untouched(*ts):
    torch.cuda.synchronize()
    for t in ts:
        if t is None:
            continue
        ref = -7 if t.dtype in (torch.int32, torch.int64) else (3.0 if t.dtype == torch.bfloat16 else -7.0)
        assert bool((t == ref).all()), "an output buffer changed: a kernel ran"


def raises(fn, *outs):
    print(f"[validation] {fn.__name__ if hasattr(fn, '__name__') else fn}", file=sys.stderr, flush=True)
    with pytest.raises(RuntimeError):
        fn()
    untouched(*outs)


def good_topk_args():
    return dict(logits=f32(S, R, CTX // S, fill=0.5), k=K, ctx=CTX, num_shards=S, interleave=1)


def test_topk_select_rejects_bad_shapes():
    a = good_topk_args()
    li, cand = i32(S, R, K), f32(R, S * K, 2)
    # wrong output shapes
    raises(lambda: dsa.topk_select(**a, local_idx=i32(S, R, K - 1), cand=cand), cand)
    raises(lambda: dsa.topk_select(**a, local_idx=li, cand=f32(R, S * K - 2, 2)), li)
    raises(lambda: dsa.topk_select(**a, local_idx=li, cand=f32(R + 1, S * K, 2)), li)
    # row bounds of the wrong length or dtype
    raises(lambda: dsa.topk_select(**a, row_ends=i32(R - 1, fill=10), local_idx=li, cand=cand),
           li, cand)
    raises(lambda: dsa.topk_select(**a, row_starts=torch.zeros(R, dtype=torch.int64, device=DEV),
                                   local_idx=li, cand=cand), li, cand)
    # strided rows, non-unit innermost stride, wrong dtype
    wide = f32(S, R, CTX, fill=0.5)
    raises(lambda: dsa.topk_select(**{**a, "logits": wide[:, :, :CTX // S]}, local_idx=li,
                                   cand=cand), li, cand)
    raises(lambda: dsa.topk_select(**{**a, "logits": wide[:, :, ::2]}, local_idx=li, cand=cand),
           li, cand)
    raises(lambda: dsa.topk_select(**{**a, "logits": a["logits"].double()}, local_idx=li,
                                   cand=cand), li, cand)
    # strided output
    raises(lambda: dsa.topk_select(**a, local_idx=i32(S, R, 2 * K)[:, :, ::2], cand=cand), cand)


def test_merge_and_convert_reject_bad_shapes():
    cand = f32(R, S * K, 2, fill=0.0)
    bt = i32(S, R, 24, fill=0)
    ids = i32(R, K)
    raises(lambda: dsa.merge_candidates(cand, K, id_bound=CTX, ids=i32(R, K + 1)))
    raises(lambda: dsa.merge_candidates(f32(R, S * K, 3), K, id_bound=CTX, ids=ids), ids)
    raises(lambda: dsa.merge_candidates(cand.transpose(0, 1), K, id_bound=CTX, ids=ids), ids)
    slots, counts = i32(S, R, K), i32(S, R)
    mc = dict(id_bound=CTX, block_size=64, num_shards=S, interleave=1)
    raises(lambda: dsa.merge_convert(cand, K, bt, **mc, ids=ids, slots=i32(S, R, K - 1),
                                     counts=counts), ids, counts)
    raises(lambda: dsa.merge_convert(cand, K, bt, **mc, ids=ids, slots=slots,
                                     counts=i32(S, R + 1)), ids, slots)
    raises(lambda: dsa.merge_convert(cand, K, bt, **mc, ids=ids, slots=slots, counts=counts,
                                     row_req=i32(R + 2, fill=0)), ids, slots, counts)
    raises(lambda: dsa.merge_convert(cand, K, i32(S, R, 48, fill=0)[:, :, :24], **mc, ids=ids,
                                     slots=slots, counts=counts), ids, slots, counts)
    raises(lambda: dsa.convert_index(ids, bt, block_size=64, num_shards=S, interleave=1,
                                     slots=i32(S + 1, R, K), counts=counts), counts)
    raises(lambda: dsa.convert_index(i32(R, 2 * K)[:, ::2], bt, block_size=64, num_shards=S,
                                     interleave=1, slots=slots, counts=counts), slots, counts)


def test_attention_and_combine_reject_bad_shapes():
    q = bf(R, H, 576)
    cache = bf(4, 64, 576)
    slots, counts = i32(S, R, K, fill=0), i32(S, R, fill=0)
    out, lse = bf(S, R, H, 512), f32(S, R, H)
    kw = dict(sm_scale=1 / 24)
    raises(lambda: dsa.sparse_mla_decode(bf(R, H, 512), cache, slots, counts, **kw, out=out,
                                         lse=lse), out, lse)
    raises(lambda: dsa.sparse_mla_decode(q, bf(4, 64, 512), slots, counts, **kw, out=out,
                                         lse=lse), out, lse)
    raises(lambda: dsa.sparse_mla_decode(q, cache, i32(S, R + 1, K, fill=0), None, **kw, out=out,
                                         lse=lse), out, lse)
    raises(lambda: dsa.sparse_mla_decode(q, cache, slots, i32(S, R - 1, fill=0), **kw, out=out,
                                         lse=lse), out, lse)
    raises(lambda: dsa.sparse_mla_decode(q, cache, slots, counts, **kw, out=bf(S, R, H, 256),
                                         lse=lse), lse)
    raises(lambda: dsa.sparse_mla_decode(q, cache, slots, counts, **kw, splits=2, out=out,
                                         lse=lse), out, lse)
    raises(lambda: dsa.sparse_mla_decode(q, cache, slots, counts, **kw, out=out,
                                         lse=f32(S, R, H + 16)), out)
    raises(lambda: dsa.sparse_mla_decode(q, torch.zeros(4, 64, 576, dtype=torch.uint8, device=DEV),
                                         slots, counts, **kw, out=out, lse=lse), out, lse)
    raises(lambda: dsa.sparse_mla_decode(bf(R, 2 * H, 576)[:, ::2], cache, slots, counts, **kw,
                                         out=out, lse=lse), out, lse)
    o, l = bf(R, H, 512), f32(R, H)
    raises(lambda: dsa.lse_combine(out, f32(S, R, H + 1), out=o, lse_out=l), o, l)
    raises(lambda: dsa.lse_combine(out, lse, out=bf(R, H, 256), lse_out=l), l)
    raises(lambda: dsa.lse_combine(out, lse, out=o, lse_out=f32(R + 1, H)), o)


def test_prologue_rejects_bad_shapes():
    T = 4
    kv, pe, w = bf(T, 512), bf(T, 64), bf(512)
    cs, pos = f32(100, 64, fill=0.0), i32(T, fill=1)
    kvo, peo = bf(T, 512), bf(T, 64)
    cache = bf(2, 64, 576)
    sm = torch.full((T,), -7, dtype=torch.int64, device=DEV)
    raises(lambda: dsa.fused_rmsnorm_rope(kv, pe, w, 1e-6, cs, i32(T - 1, fill=1), kv_c_out=kvo,
                                          k_pe_out=peo), kvo, peo)
    raises(lambda: dsa.fused_rmsnorm_rope(kv, bf(T + 1, 64), w, 1e-6, cs, pos, kv_c_out=kvo,
                                          k_pe_out=peo), kvo, peo)
    raises(lambda: dsa.fused_rmsnorm_rope(kv, pe, bf(256), 1e-6, cs, pos, kv_c_out=kvo,
                                          k_pe_out=peo), kvo, peo)
    raises(lambda: dsa.fused_rmsnorm_rope(kv, pe, w, 1e-6, f32(100, 32), pos, kv_c_out=kvo,
                                          k_pe_out=peo), kvo, peo)
    raises(lambda: dsa.fused_rmsnorm_rope(kv, pe, w, 1e-6, cs, pos, kv_c_out=bf(T, 256),
                                          k_pe_out=peo), peo)
    raises(lambda: dsa.fused_rmsnorm_rope(kv, pe, w, 1e-6, cs, pos, kv_c_out=kvo,
                                          k_pe_out=bf(T - 1, 64)), kvo)
    raises(lambda: dsa.fused_rmsnorm_rope(kv, pe, w, 1e-6, cs, pos, kv_c_out=kvo, k_pe_out=peo,
                                          cache=cache, slot_mapping=sm[:T - 1]), kvo, peo)
    raises(lambda: dsa.fused_rmsnorm_rope(kv, pe, w, 1e-6, cs, pos, kv_c_out=kvo, k_pe_out=peo,
                                          cache=torch.zeros(2, 64, 576, dtype=torch.uint8,
                                                            device=DEV),
                                          slot_mapping=sm), kvo, peo, sm)
    raises(lambda: dsa.cache_insert(kv, pe, bf(2, 64, 512), sm), sm)
    raises(lambda: dsa.cache_insert(kv, pe, cache, sm[:2]), sm)
