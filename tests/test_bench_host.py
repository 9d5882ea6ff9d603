"""Host-side checks of bench.py (no GPU): the single-GPU rule, the
algorithmic byte and flop counts behind the roofline line, and the lookup of
the counter-measured traffic."""
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def _case(rows, heads, shards, k, cache="bf16", pool_blocks=32768):
    # only the latent pool's element count and width are read
    pool = types.SimpleNamespace(size=pool_blocks * 64 * 576, itemsize=1 if cache == "fp8" else 2)
    return types.SimpleNamespace(rows=rows, heads=heads, S=shards, k=k, cache_dtype=cache,
                                 cache=pool)


def test_decode_attention_bytes_and_flops():
    # decode workload: 64 rows x 4 shards, every row selects k = 2048 tokens
    c = _case(64, 128, 4, 2048)
    counts_total = 64 * 2048
    b, u, f = bench.attention_traffic(c, counts_total)
    q = 64 * 128 * 576 * 2
    rows = counts_total * 1152
    slots = counts_total * 4 + 4 * 64 * 4
    partials = 4 * 64 * 128 * (512 * 2 + 4)
    assert b == u == q + rows + slots + partials == 194_642_944   # 2.4 GB pool: no reuse
    assert f == counts_total * 128 * (576 + 512) * 2
    # an fp8 cache moves half the bytes per gathered row
    b8, _, _ = bench.attention_traffic(_case(64, 128, 4, 2048, "fp8"), counts_total)
    assert b - b8 == counts_total * 576


def test_prefill_pool_in_infinity_cache_counts_once():
    # prefill chunk: 8192 rows, one request whose 512-block pool (37.7 MB) fits
    # the 256 MB Infinity Cache, so HBM delivers the pool once
    c = _case(8192, 128, 4, 2048, pool_blocks=512)
    counts_total = 8192 * 1024        # any total far above the pool's 32768 rows
    b, u, f = bench.attention_traffic(c, counts_total)
    pool = 512 * 64 * 576 * 2
    assert b - u == counts_total * 1152 - pool
    # flops over HBM-unique bytes exceed the ridge: the MFMA roof binds
    assert f / (bench.BF16_PEAK_TFLOPS * 1e12) > u / (bench.HBM_PEAK_GBS * 1e9)


def test_topk_and_merge_bytes():
    c = _case(64, 128, 4, 2048)
    n_valid = 64 * 32768
    tk, mg = bench.topk_traffic(c, n_valid, fused=False)
    assert tk == n_valid * 4 + 64 * 4 * 2048 * 8
    assert mg == 64 * 4 * 2048 * 8 + 64 * 2048 * 4
    _, mg_fused = bench.topk_traffic(c, n_valid, fused=True)
    assert mg_fused - mg == 4 * 64 * 2048 * 4 + 4 * 64 * 4


def test_measured_traffic_follows_the_kernel_source(tmp_path, monkeypatch):
    import hashlib
    src = tmp_path / "sparse_attention_indexer_topk_amd" / "csrc" / "sparse_mla_decode.hip"
    src.parent.mkdir(parents=True)
    src.write_bytes(b"kernel v1")
    prof = tmp_path / "profiles"
    prof.mkdir()
    sha = hashlib.sha256(b"kernel v1").hexdigest()
    (prof / "decode_hbm_traffic.md").write_text(
        f"    sparse_mla_decode traffic_bytes_per_launch=123456 source_sha256={sha}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("decode") == 123456
    assert bench.measured_traffic("long") is None        # no summary for that workload
    src.write_bytes(b"kernel v2")                          # the kernel changed since
    assert bench.measured_traffic("decode") is None
