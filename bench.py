#!/usr/bin/env python3
"""Benchmark of the DSA sparse-attention decode path on one MI355X.

One step = one pass of the whole path over one batch of the decode workload
(64 rows, 32768-token context, 4 shards, k = 2048, 128 heads, bf16 latent
cache): per-shard top-K + candidate pack -> merge -> index conversion ->
sparse MLA decode (all shards) -> LSE combine.  Inputs are resident in HBM
before timing starts; four independently drawn (logits, q) sets rotate
through the steps so a step does not find its inputs or its gathered rows
in the on-chip caches left by the previous step.

Prints ONE JSON line.  `value` = decode tokens/s of the whole path (one query
token per row).  Inside the timed steps the only HIP events (recorded on the
launch stream) bracket the attention launch, whose average duration gives the
roofline of that dominant kernel; a separate pass with events between every
launch gives the per-kernel breakdown and the top-K and decode halves of the
metric.  The CPU oracle is timed on the host for comparison.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer top-K rows/s + sparse-MLA decode tokens/s at 32k ctx, k=2048; % roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode",
                   choices=["decode", "tiny", "long", "prefill", "fp8"])
    p.add_argument("--sets", type=int, default=4, help="rotating input sets")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--att-stride", type=int, default=10,
                   help="bracket the attention launch with HIP events on every this-many-th "
                        "timed step (each event pair drains the queue and costs ~4 us of step time)")
    p.add_argument("--pcp", type=int, default=0,
                   help="prologue in sequence-sharded form over this many ranks "
                        "(materialise per rank, gather, insert)")
    p.add_argument("--no-merge-ids", action="store_true",
                   help="merge_convert writes only the slot lists and counts, not the merged "
                        "global ids (nothing downstream reads them)")
    p.add_argument("--unfused", action="store_true",
                   help="merge_candidates and convert_index as two launches")
    p.add_argument("--cpu-seconds", type=float, default=8.0,
                   help="oracle time per CPU-baseline mode (single thread, all threads)")
    p.add_argument("--splits", type=int, default=None,
                   help="pieces each shard's token list is cut into for the attention "
                        "(default: enough workgroups to cover the CUs)")
    p.add_argument("--launch-floor", action="store_true",
                   help="only launch empty kernels with the grid shapes of the decode step's "
                        "kernels (30 each), for a kernel trace of the launch floor")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB device copy (3 times), the reference "
                        "for scaling the HBM byte counters of a profile")
    return p.parse_args()


def calibrate_copy():
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n,
                      "dispatches": 3}), flush=True)


MALL_BYTES = 256 << 20   # MI355X Infinity Cache


def launch_floor_grids():
    """Empty launches with the grids of the decode workload's kernels (64 rows,
    4 shards, 128 heads): top-K and merge_convert 256 x 1024 threads, the
    attention 256 x 512, the combine 2048 x 256."""
    import torch
    import sparse_attention_indexer_topk_amd as dsa
    grids = {"topk_select / merge_convert": (256, 1024), "sparse_mla_decode": (256, 512),
             "lse_combine": (2048, 256)}
    for _ in range(30):
        for wg, nt in grids.values():
            dsa.launch_floor(wg, nt)
    torch.cuda.synchronize()
    print(json.dumps({"launch_floor": {k: {"workgroups": v[0], "threads": v[1], "launches": 30}
                                       for k, v in grids.items()}}), flush=True)


def attention_traffic(c, counts_total):
    """Algorithmic bytes and flops of one sparse_mla_decode launch.

    Returns (bytes per selection, HBM-unique bytes, flops).  The gathered
    latent rows count once per selection; when the whole latent pool fits the
    256 MB Infinity Cache (the prefill chunk: one request, 37.7 MB), repeated
    selections of a row are served on chip and the HBM-unique bytes count the
    pool once instead."""
    R, H, S, k = c.rows, c.heads, c.S, c.k
    entry = 576 if c.cache_dtype == "fp8" else 1152
    fixed = (R * H * 576 * 2                  # q, once per row and shard pass
             + counts_total * 4 + S * R * 4   # slot lists + counts
             + S * R * H * 512 * 2            # bf16 partial outputs
             + S * R * H * 4)                 # partial lse
    gathered = counts_total * entry
    pool = c.cache.size * c.cache.itemsize
    unique = fixed + (min(gathered, pool) if pool <= MALL_BYTES else gathered)
    flops = counts_total * H * (576 + 512) * 2
    return fixed + gathered, unique, flops


def topk_traffic(c, n_valid_logits, fused=True, ids=True):
    """Algorithmic bytes of topk_select and of the merge launch for one step
    (merge_convert also writes the slot lists and counts; ids=False: it does
    not write the merged ids)."""
    R, S, k = c.rows, c.S, c.k
    topk = n_valid_logits * 4 + R * S * k * 8         # logits read, candidates written
    merge = R * S * k * 8 + (R * k * 4 if ids else 0)  # candidates read, ids written
    if fused:
        merge += S * R * k * 4 + S * R * 4            # slots and counts written
    return topk, merge


def measured_traffic(workload):
    """HBM bytes per sparse_mla_decode launch from the committed counter
    summary of this workload, or None when there is none or the kernel source
    changed since the counters were taken."""
    import hashlib
    import re
    summary = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.md")
    src = os.path.join(ROOT, "sparse_attention_indexer_topk_amd", "csrc", "sparse_mla_decode.hip")
    try:
        text = open(summary).read()
        m = re.search(r"sparse_mla_decode traffic_bytes_per_launch=(\d+) source_sha256=([0-9a-f]+)",
                      text)
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    if not m or m.group(2) != sha:
        return None
    return int(m.group(1))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(c, seconds):
    """The oracle as it stands, on whole decode steps of the same workload,
    repeated until `seconds` have passed, in two modes: one BLAS thread, and
    every thread the BLAS library was given (the attention products are the
    only multi-threaded part; selection and conversion are NumPy loops)."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits

    rs = np.arange(c.rows)

    def run(limit):
        rows_done, t0 = 0, time.perf_counter()
        with threadpool_limits(limits=limit):
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
            while True:
                _, cand = oracle.topk_select(c.logits[:, rs], c.row_starts[rs], c.row_ends[rs],
                                             c.ctx, c.k, c.S, c.I)
                ids = oracle.merge_candidates(cand, c.k)
                slots, counts = oracle.convert_index(ids, c.row_req[rs], c.block_table, 64, c.S,
                                                     c.I)
                po, pl = oracle.sparse_mla_partial(c.q[rs], c.cache, c.cache_dtype,
                                                   c.cache_scale, slots, counts, c.sm_scale)
                oracle.lse_combine(po, pl)
                rows_done += len(rs)
                el = time.perf_counter() - t0
                if el >= seconds:
                    break
        return rows_done / el, rows_done, el, int(threads)

    v1, n1, e1, _ = run(1)
    vall, nall, eall, threads = run(None)
    return {"value": vall, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{nall // c.rows} whole steps of the {c.spec.name} workload "
                      f"({nall} rows, full path), float64 NumPy, {eall:.1f} s, "
                      f"{threads} BLAS threads",
            "single_thread": {"value": v1, "unit": "tokens/s", "cores": 1,
                              "sample": f"{n1 // c.rows} whole steps ({n1} rows), {e1:.1f} s"},
            "cpu_count": os.cpu_count(), "cpu_model": cpu_model()}


def main():
    a = parse()
    if a.calibrate_copy:
        calibrate_copy()
        return
    if a.launch_floor:
        launch_floor_grids()
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {a.gpus}): every shard is emulated "
              "as a slice of one buffer on a single MI355X; sharding across GPUs is described in "
              "the design notes, not benchmarked.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import dsa_inputs
    from sparse_attention_indexer_topk_amd.pipeline import DecodePath

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_gen = time.perf_counter()
    c = dsa_inputs.make(a.workload)
    arrays = dsa_inputs.device_arrays(c, device=dev)
    if a.pcp:
        if "prologue" not in arrays:
            print("--pcp needs a workload with a prologue (fp8)", file=sys.stderr)
            sys.exit(2)
        arrays["pcp_ranks"] = a.pcp
    if a.splits is not None:
        arrays["splits"] = a.splits
    path = DecodePath(**arrays)
    path.want_ids = a.unfused or not a.no_merge_ids
    logits_sets, q_sets = [path.logits], [path.q]
    for s in range(1, a.sets):
        lg, qq = dsa_inputs.redraw_logits_q(c, s)
        logits_sets.append(torch.from_numpy(lg).to(dev))
        q_sets.append(torch.from_numpy(qq.view(np.int16)).to(dev).view(torch.bfloat16))
    torch.cuda.synchronize()
    print(f"# inputs ready in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    if a.unfused:
        names = ["fused_rmsnorm_rope", "topk_select", "merge_candidates", "convert_index",
                 "sparse_mla_decode", "lse_combine"]
    else:
        names = ["fused_rmsnorm_rope", "topk_select", "merge_convert", "sparse_mla_decode",
                 "lse_combine"]
    if a.pcp:   # per-rank materialise launches + one insert
        names[0] = "prologue_pcp"

    def step(i, att_ev=None, all_ev=None):
        """One pass of the whole path.  att_ev: events around the attention
        launch only (the timed steps); all_ev: events between every launch
        (the per-kernel breakdown pass, outside the timed region)."""
        j = i % a.sets
        rec = (lambda n: all_ev[n].record(stream)) if all_ev is not None else (lambda n: None)
        n = 0
        rec(n)
        if path.prologue is not None:
            path.run_prologue()
        n += 1; rec(n)
        path.run_topk(logits=logits_sets[j])
        n += 1; rec(n)
        if a.unfused:
            path.run_merge()
            n += 1; rec(n)
            path.run_convert()
        else:
            path.run_merge_convert()
        n += 1; rec(n)
        if att_ev is not None: att_ev[0].record(stream)
        path.run_attention(q=q_sets[j])
        if att_ev is not None: att_ev[1].record(stream)
        n += 1; rec(n)
        path.run_combine()
        n += 1; rec(n)

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K whole steps; the only events in it bracket the attention
    # launch (the roofline's kernel) on every stride-th step.  An event pair
    # makes the queue drain before and after the launch, which costs about
    # 4 us of step time, so it samples the launches rather than wrapping each
    stride = max(1, a.att_stride)
    att_events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
                  for _ in range(0, a.steps, stride)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(a.warmup + i, att_ev=att_events[i // stride] if i % stride == 0 else None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / a.steps
    att_us = float(np.mean([e[0].elapsed_time(e[1]) for e in att_events])) * 1e3

    # per-kernel breakdown: a separate pass with events between all launches
    n_brk = min(a.steps, 50)
    brk = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
           for _ in range(n_brk)]
    for i in range(n_brk):
        step(i, all_ev=brk[i])
    torch.cuda.synchronize()
    kern_us = {n: float(np.mean([ev[j].elapsed_time(ev[j + 1]) for ev in brk])) * 1e3
               for j, n in enumerate(names)}
    if path.prologue is None:
        kern_us.pop(names[0])

    # algorithmic traffic of the last set's step (all sets have the same shape)
    counts_total = int(path.counts.sum().item())
    n_valid = 0
    for i in range(c.rows):
        n_valid += int(c.row_ends[i]) - int(c.row_starts[i])
    att_bytes, att_unique, att_flops = attention_traffic(c, counts_total)
    tk_bytes, mg_bytes = topk_traffic(c, n_valid, fused=not a.unfused,
                                      ids=a.unfused or not a.no_merge_ids)
    t_att = att_us * 1e-6
    att_tflops = att_flops / t_att / 1e12
    # the binding roof: HBM time of the bytes HBM must deliver vs MFMA time
    bound = ("hbm" if att_unique / (HBM_PEAK_GBS * 1e9) >= att_flops / (BF16_PEAK_TFLOPS * 1e12)
             else "mfma")
    att_gbs = att_unique / t_att / 1e9
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(att_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(att_gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(att_tflops, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(att_tflops / BF16_PEAK_TFLOPS, 4)}
    roof["traffic"] = measured_traffic(c.spec.name)
    roof["kernel"] = "sparse_mla_decode"
    roof["algorithmic_bytes"] = att_unique
    if att_unique != att_bytes:
        roof["bytes_per_selection"] = att_bytes
    roof["algorithmic_flops"] = att_flops
    roof["mfma_tflops"] = round(att_tflops, 1)

    # the metric's halves: top-K side = selection + merge (the fused launch
    # counted whole), decode side = conversion (when separate) + attention +
    # combine
    merge_key = "merge_candidates" if a.unfused else "merge_convert"
    t_topk = (kern_us["topk_select"] + kern_us[merge_key]) * 1e-6
    t_dec = (kern_us.get("convert_index", 0.0) + kern_us["sparse_mla_decode"] +
             kern_us["lse_combine"]) * 1e-6
    value = c.rows / (ms_per_step * 1e-3)
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": c.spec.name, "rows": c.rows, "ctx": c.ctx, "k": c.k,
                   "shards": c.S, "interleave": c.I, "heads": c.heads, "cache": c.cache_dtype,
                   "input_sets": a.sets, "merged_ids_written": bool(path.want_ids),
                   "attention_splits": path.splits,
                   **({"pcp_ranks": a.pcp} if a.pcp else {})},
        "topk_rows_per_s": round(c.rows / t_topk, 1),
        "decode_tokens_per_s": round(c.rows / t_dec, 1),
        "sparse_mla_decode_us_timed": round(att_us, 2),
        "attention_timed_launches": len(att_events),
        "kernel_us": {k: round(v, 2) for k, v in kern_us.items()},
        "topk_merge_hbm_frac": round((tk_bytes + mg_bytes) / (HBM_PEAK_GBS * 1e9) / t_topk, 4),
        "roofline": roof,
    }
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(c, a.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
