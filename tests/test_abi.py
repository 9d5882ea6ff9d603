"""The C-ABI library loads, exports every entry point include/dsa.h declares,
and rejects invalid arguments on the host before any HIP call (these tests
run without a GPU: no call below reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import sparse_attention_indexer_topk_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

if not os.path.exists(dsa.LIB_PATH):
    pytest.skip("libdsa.so not built", allow_module_level=True)

L = dsa.lib()
OK, INV, BADK, BADT = 0, -1, -2, -3
FAKE = 0x10000   # a 64 KB-aligned non-null address; validation never dereferences it


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(dsa_\w+)\s*\(", text, re.M)))


def test_header_declares_the_six_path_calls():
    syms = declared_symbols()
    for name in ["dsa_topk_select", "dsa_merge_candidates", "dsa_convert_index",
                 "dsa_sparse_mla_decode", "dsa_lse_combine", "dsa_fused_rmsnorm_rope",
                 "dsa_last_error", "dsa_version"]:
        assert name in syms


def test_library_exports_every_declared_symbol():
    for name in declared_symbols():
        assert hasattr(L, name), name
        assert name in dsa.SIGNATURES, f"binding lacks a signature for {name}"


def test_version():
    assert L.dsa_version() >= 100


def topk(**kw):
    a = dict(logits=FAKE, ld=2048, stride=2 * 2048, rows=2, ctx=4096, rs=None, re=None, k=512,
             S=2, I=1, first=0, count=2, idx=FAKE, cand=FAKE)
    a.update(kw)
    return L.dsa_topk_select(a["logits"], a["ld"], a["stride"], a["rows"], a["ctx"], a["rs"],
                             a["re"], a["k"], a["S"], a["I"], a["first"], a["count"], a["idx"],
                             a["cand"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(k=100), BADK), (dict(k=4096), BADK), (dict(logits=None), INV),
    (dict(idx=None, cand=None), INV), (dict(rows=-1), INV), (dict(S=0), INV),
    (dict(S=17), INV), (dict(I=0), INV), (dict(first=1, count=2), INV), (dict(count=0), INV),
    (dict(ctx=-1), INV), (dict(ctx=(1 << 24) + 1), INV), (dict(ld=2047), INV),
    (dict(stride=100), INV), (dict(logits=FAKE + 2), INV),
])
def test_topk_select_rejects(kw, code):
    assert topk(**kw) == code
    assert L.dsa_last_error().decode().startswith("dsa_topk_select")


def test_topk_select_rows_zero_is_noop():
    assert topk(rows=0) == OK


def test_merge_rejects():
    m = L.dsa_merge_candidates
    assert m(FAKE, 2, 1024, 300, 4096, FAKE, None) == BADK
    assert m(None, 2, 1024, 512, 4096, FAKE, None) == INV
    assert m(FAKE, 2, 0, 512, 4096, FAKE, None) == INV
    assert m(FAKE, 2, 16 * 512 + 1, 512, 4096, FAKE, None) == INV
    assert m(FAKE, 2, 1024, 512, 0, FAKE, None) == INV
    assert m(FAKE, 2, 1024, 512, (1 << 24) + 1, FAKE, None) == INV
    assert m(FAKE, 0, 1024, 512, 4096, FAKE, None) == OK


def test_convert_rejects():
    c = L.dsa_convert_index
    base = [FAKE, 2, 512, None, 2, FAKE, 32, 64, 64, 2, 1, 0, 2, FAKE, FAKE, None]
    def call(**kw):
        a = list(base)
        idx = dict(ids=0, rows=1, k=2, nreq=4, bt=5, bt_ld=6, bt_stride=7, bs=8, S=9, I=10,
                   first=11, count=12, slots=13)
        for key, v in kw.items():
            a[idx[key]] = v
        return c(*a)
    assert call(rows=0) == OK
    assert call(k=7, rows=0) == BADK
    assert call(ids=None, rows=0) == INV
    assert call(nreq=0, rows=0) == INV
    assert call(bt_ld=0, rows=0) == INV
    assert call(bt_stride=10, rows=0) == INV
    assert call(bs=0, rows=0) == INV
    assert call(S=2, first=2, count=1, rows=0) == INV


def test_sparse_mla_decode_rejects():
    f = L.dsa_sparse_mla_decode
    def call(**kw):
        a = dict(q=FAKE, rows=0, heads=128, cache=FAKE, dt=dsa.DSA_BF16, scale=None, nslots=100,
                 slots=FAKE, counts=None, k=2048, parts=4, splits=1, sm=0.04, out=FAKE,
                 odt=dsa.DSA_BF16, lse=FAKE)
        a.update(kw)
        return f(a["q"], a["rows"], a["heads"], a["cache"], a["dt"], a["scale"], a["nslots"],
                 a["slots"], a["counts"], a["k"], a["parts"], a["splits"], a["sm"], a["out"],
                 a["odt"], a["lse"], None)
    assert call() == OK
    assert call(heads=24) == INV
    assert call(heads=0) == INV
    assert call(k=1000) == BADK
    assert call(dt=dsa.DSA_FP32) == BADT
    assert call(dt=dsa.DSA_FP8_E4M3) == INV           # fp8 without a scale
    assert call(dt=dsa.DSA_FP8_E4M3, scale=FAKE) == OK
    assert call(q=FAKE + 8) == INV
    assert call(parts=0) == INV
    assert call(splits=0) == INV
    assert call(splits=65) == INV
    assert call(splits=8) == OK
    assert call(rows=-3) == INV
    # workgroup count past 2^31 - 1 is refused before any launch
    assert call(rows=1 << 29, parts=4, heads=128) == INV
    assert call(rows=1 << 28, parts=4, splits=2, heads=128) == INV
    # partial outputs: bf16, or fp32 (the checking mode); nothing else
    assert call(odt=dsa.DSA_FP32) == OK
    assert call(odt=dsa.DSA_FP8_E4M3) == BADT
    assert call(odt=0) == BADT


def test_lse_combine_rejects():
    f = L.dsa_lse_combine
    B, F = dsa.DSA_BF16, dsa.DSA_FP32
    assert f(FAKE, B, FAKE, 4, 0, 128, 512, FAKE, None, None) == OK
    assert f(FAKE, F, FAKE, 4, 0, 128, 512, FAKE, None, None) == OK
    assert f(FAKE, dsa.DSA_FP8_E4M3, FAKE, 4, 0, 128, 512, FAKE, None, None) == BADT
    assert f(FAKE, B, FAKE, 0, 0, 128, 512, FAKE, None, None) == INV
    assert f(FAKE, B, FAKE, 65, 0, 128, 512, FAKE, None, None) == INV
    assert f(FAKE, B, FAKE, 4, 0, 128, 12, FAKE, None, None) == INV
    assert f(None, B, FAKE, 4, 0, 128, 512, FAKE, None, None) == INV


def test_fused_rmsnorm_rope_rejects():
    f = L.dsa_fused_rmsnorm_rope
    def call(**kw):
        a = dict(kv=FAKE, kvld=512, pe=FAKE, peld=64, T=0, w=FAKE, eps=1e-6, cs=FAKE, npos=10,
                 pos=FAKE, kvo=FAKE, peo=FAKE, cache=None, dt=0, scale=None, sm=None, nslots=0,
                 ik=None, ikld=0, iw=None, ieps=1e-6, iko=None, icache=None, iscale=None,
                 inslots=0)
        a.update(kw)
        return f(a["kv"], a["kvld"], a["pe"], a["peld"], a["T"], a["w"], a["eps"], a["cs"],
                 a["npos"], a["pos"], a["kvo"], a["peo"], a["cache"], a["dt"], a["scale"], a["sm"],
                 a["nslots"], a["ik"], a["ikld"], a["iw"], a["ieps"], a["iko"], a["icache"],
                 a["iscale"], a["inslots"], None)
    assert call() == OK
    # nothing to produce (three outputs and the slot mapping NULL): early
    # return, whatever the inputs are
    assert call(kvo=None, peo=None, T=5, kv=None, cs=None) == OK
    assert call(kvld=500) == INV
    assert call(peld=63) == INV
    assert call(w=None) == INV
    assert call(sm=FAKE) == INV                         # slot mapping without a cache
    assert call(sm=FAKE, cache=FAKE, dt=dsa.DSA_FP32) == BADT
    assert call(sm=FAKE, cache=FAKE, dt=dsa.DSA_FP8_E4M3) == INV   # no scale
    assert call(T=-1) == INV
    # indexer branch: runs when index_k_out is given, or an indexer cache and a
    # slot mapping; then its inputs and the cache's scale are required
    ik = dict(ik=FAKE, ikld=128, iw=FAKE, iko=FAKE)
    assert call(**ik) == OK
    assert call(kvo=None, peo=None, kv=None, pe=None, w=None, **ik) == OK   # indexer only
    assert call(**{**ik, "ik": None}) == INV
    assert call(**{**ik, "iw": None}) == INV
    assert call(**{**ik, "ikld": 100}) == INV
    assert call(**{**ik, "ikld": 129}) == INV
    assert call(sm=FAKE, icache=FAKE, **ik) == INV                  # no indexer-cache scale
    assert call(sm=FAKE, icache=FAKE, iscale=FAKE, inslots=64, **ik) == OK
    # an indexer cache without a slot mapping is not written: the branch needs
    # no inputs when index_k_out is NULL too
    assert call(icache=FAKE, iscale=None) == OK


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(RuntimeError):
        dsa.topk_select(torch.zeros(2, 2, 2048), 512, ctx=4096, num_shards=2, interleave=1)
    with pytest.raises(RuntimeError):
        dsa.merge_candidates(torch.zeros(2, 1024, 2), 512, id_bound=4096)
