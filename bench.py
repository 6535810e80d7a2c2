#!/usr/bin/env python3
"""Benchmark of the paged KV write + paged decode hot path on one MI355X.

One step = pa_write_kv of the batch's new tokens, then paged decode attention
(the split-KV partial kernel and the partition merge) over the whole batch.
Default workload: Llama-3-8B attention shape in bf16 (B=64, H=32, KVH=8,
D=128, block size 16, context lengths U[1, 4096], shuffled blocks, 64 written
tokens).  Inputs are seeded synthetic tensors already resident in HBM.

By default a 1 GiB buffer is read before every step (outside the step's
timing events) so that the 256 MB last-level cache holds none of the KV rows
of the previous step.  The flush reads rather than writes: a written buffer
would leave dirty lines whose write-back would share the timed step's
bandwidth.  ``--hot`` skips the flush.

The timed step is one pa_decode_append call when the workload's write is
exactly one newest token per sequence (its partial kernel over the cached
tokens, then a merge that folds in and writes each new token: two kernels),
else the three kernels (write, partials, merge) launched one after another
on one stream; `three_kernel_step_us` reports the latter either way.  The
three-kernel step captured in a HIP graph and replayed is timed too
(`graph_step_us`): on this stack a replay takes longer than the launches.

Prints ONE JSON line.  `value` = KV bytes the decode must read (sum over
sequences of n_b * 2 * KVH * D * elem) / mean step time, in GB/s (10^9 B/s).
`roofline.achieved` takes the distinct rows instead (`kv_unique_bytes_per_step`:
a block shared by several tables counts once), the bytes HBM must deliver;
the two differ only for the prefix-shared workload, which by default decodes
with pa_decode_shared_prefix and its 2048-token common prefix as the hint
(`--shared-tokens 0`: plain pa_decode).

``--config prefix_serving_host`` times the host block manager (no GPU): 4096
requests sharing a 1024-token system prompt are admitted (prefix matching and
allocation), run 128 decode steps of batched appends (each step's
slot_mapping), and are freed; `value` = appended tokens/s.

``--config write_65536_bf16`` times pa_write_kv alone at a prefill-sized
token count: 65,536 tokens (16 prompts of 4096) with the Llama-3-8B shape
(KVH 8, D 128, bs 16) into shuffled blocks; `value` = bytes moved (K and V rows
read and written, plus the slots) / mean kernel time, in GB/s.

``--config prefill_8b_bf16`` times the paged prefill instead: one step =
pa_write_kv of every sequence's new chunk, then pa_prefill (causal attention
of the chunk's queries over the sequence's paged K/V), on the Llama-3-8B
shape with 8 sequences of U[0, 4096] cached tokens and U[512, 2048]-token
chunks.  `value` = algorithmic flops (4 * D * H per causally visible
(query, key) pair) / mean step time, in TFLOP/s; the roofline is the bf16
matrix-core peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, published
METRIC = "paged decode KV-read GB/s (% of HBM peak) + µs/step; write_kv GB/s"
PREFILL_METRIC = "paged prefill TFLOP/s (% of bf16 MFMA peak) + µs/step"
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "paged_kv_cache_70_amd", "csrc")
# the dominant kernel of each bench line ("bf16" / "f32": the decode partial
# kernel of that cache dtype; "write": the scatter write): its name in traces
# and its source file
PARTIAL_KERNELS = {"bf16": "decode_partial_mfma_kernel", "f32": "decode_partial_kernel", "write": "write_kv_kernel",
                   "prefill": "prefill_mfma_kernel"}
# where vLLM's cache layout runs another kernel (the bf16 decode and the
# prefill run the same templates with the layout as a parameter)
VLLM_KERNELS = {"f32": "decode_partial_vllm_kernel", "write": "write_kv_vllm_kernel"}
# the sources each kernel is compiled from (its file, the shared parameter
# structs, and the tile helpers the matrix-core kernels share)
_INTERNAL = os.path.join(CSRC, "pa_internal.h")
_TILE = os.path.join(CSRC, "pa_mfma_tile.h")
KERNEL_SRC = {"bf16": [os.path.join(CSRC, "pa_decode_mfma.hip"), _INTERNAL, _TILE],
              "f32": [os.path.join(CSRC, "pa_decode.hip"), _INTERNAL],
              "write": [os.path.join(CSRC, "pa_write.hip"), _INTERNAL],
              "prefill": [os.path.join(CSRC, "pa_prefill.hip"), _INTERNAL, _TILE]}


def _kernel_name(key: str, layout: str = "p09") -> str:
    """The dominant kernel of bench line `key` in cache layout `layout`."""
    return VLLM_KERNELS.get(key, PARTIAL_KERNELS[key]) if layout == "vllm" else PARTIAL_KERNELS[key]


def _traffic_file(key: str, workload: str, layout: str = "p09") -> str:
    """The committed counter summary of kernel `key` on `workload` (in vLLM's
    cache layout: a file of its own)."""
    suffix = "_vllm" if layout == "vllm" else ""
    return os.path.join(PROFILES, f"traffic_{_kernel_name(key, layout)}_{workload}{suffix}.json")


def _src_hash(key: str, layout: str = "p09") -> str:
    # the fp32 decode in vLLM's layout is compiled from the matrix-core kernel's file
    srcs = KERNEL_SRC["bf16"] if (key == "f32" and layout == "vllm") else KERNEL_SRC[key]
    h = hashlib.sha256()
    for path in srcs:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(workload: str, key: str, layout: str = "p09"):
    """HBM bytes per launch of the kernel `key` from the committed rocprofv3
    counter summary, if it was taken on this workload, in this cache layout,
    and on this kernel source."""
    try:
        with open(_traffic_file(key, workload, layout)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if (t.get("source_sha256_16") != _src_hash(key, layout) or t.get("workload") != workload
            or t.get("layout", "p09") != layout):
        return None
    return t.get("bytes_per_launch")

CALIB_TAG = "MulFunctor"        # torch.mul(src, 2.0, out=dst): the calibration copy


def _counter_rows(path: str, counter: str):
    """(kernel name, value) of every dispatch in a rocprofv3 --pmc CSV."""
    import csv
    with open(path, newline="") as f:
        return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in csv.DictReader(f)
                if r.get("Counter_Name") == counter]


def traffic_from_counters(fetch_csv: str, write_csv: str, workload: str, key: str,
                          calib_bytes: int, out_json: str, layout: str = "p09") -> dict:
    """HBM bytes per launch of the kernel `key` (in cache layout `layout`)
    from two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE;
    both in KiB per dispatch), each scaled by the same counter's reading for
    the calibration copy, which reads and writes calib_bytes."""
    kname = _kernel_name(key, layout)
    res = {"workload": workload, "kernel": kname, "layout": layout, "source_sha256_16": _src_hash(key, layout),
           "calibration_copy_bytes": calib_bytes}
    total = 0.0
    for key, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _counter_rows(path, key)
        kern = [v * 1024 for n, v in rows
                if n.startswith(kname) or f" {kname}<" in n or f"::{kname}<" in n or f"::{kname}(" in n]
        cal = [v * 1024 for n, v in rows if CALIB_TAG in n]
        if not kern or not cal:
            raise SystemExit(f"{path}: no {key} rows for {kname} ({len(kern)}) or the calibration copy ({len(cal)})")
        k_mean, c_mean = sum(kern) / len(kern), sum(cal) / len(cal)
        factor = calib_bytes / c_mean
        res[key.lower()] = {"dispatches": len(kern), "raw_bytes_per_launch": round(k_mean),
                            "calibration_raw_bytes": round(c_mean), "scale": round(factor, 5),
                            "bytes_per_launch": round(k_mean * factor)}
        total += k_mean * factor
    res["bytes_per_launch"] = round(total)
    with open(out_json, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    return res


def _calibration_copy(mib: int, dev, do_flush) -> None:
    """A plain fp32 copy of `mib` MiB, three times (torch.mul(src, 2.0,
    out=dst): reads and writes mib MiB): the reference reading that scales the
    HBM byte counters.  Nothing when mib is 0."""
    if not mib:
        return
    import torch
    src = torch.ones(mib << 18, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        do_flush()
        torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def _read_ceiling(nbytes: int, args, dev, do_flush) -> dict:
    """The streaming-read ceiling of nbytes on this device, in this process:
    pa_measure_read (16-byte loads, non-temporal like the decode's) over a
    buffer of that size, timed with events like the step (flushed before each
    read unless --hot), at a few workgroup counts per CU; the best is the
    ceiling."""
    import torch

    import paged_kv_cache_70_amd as pk
    nbytes = max(16, nbytes // 16 * 16)
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    res = {}
    for wpc in (1, 2, 4):
        for _ in range(max(2, args.warmup // 2)):
            do_flush()
            pk.measure_read(buf, sink, workgroups_per_cu=wpc)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for a, b in evs:
            do_flush()
            a.record()
            pk.measure_read(buf, sink, workgroups_per_cu=wpc)
            b.record()
        torch.cuda.synchronize()
        us = sum(a.elapsed_time(b) for a, b in evs) / len(evs) * 1e3
        res[wpc] = us
    del buf
    wpc = min(res, key=res.get)
    return {"GBps": round(nbytes / (res[wpc] * 1e-6) / 1e9, 1), "bytes": nbytes, "us": round(res[wpc], 2),
            "workgroups_per_cu": wpc, "nontemporal": True,
            "us_by_workgroups_per_cu": {str(k): round(v, 2) for k, v in res.items()},
            "what": "pa_measure_read: one pass of 16-byte non-temporal loads over a buffer of the step's distinct "
                    "KV bytes, one contiguous chunk per workgroup, events around the kernel, same flush as the "
                    "step; the best of 1, 2 and 4 workgroups per CU"}


def _mfma_ceiling(args, dev) -> dict:
    """The matrix-core ceiling on this device, in this process: pa_measure_mfma
    (independent bf16 32x32x16 products, no memory traffic) timed with events
    at one, two and four workgroups of 4 wavefronts per CU; the best is the ceiling."""
    import torch

    import paged_kv_cache_70_amd as pk
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    iters = 8192
    res = {}
    for wpc in (1, 2, 4):
        pk.measure_mfma(sink, iters, workgroups_per_cu=wpc)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
        torch.cuda.synchronize()
        flops = 0
        for a, b in evs:
            a.record()
            flops = pk.measure_mfma(sink, iters, workgroups_per_cu=wpc)
            b.record()
        torch.cuda.synchronize()
        us = sum(a.elapsed_time(b) for a, b in evs) / len(evs) * 1e3
        res[wpc] = (flops / (us * 1e-6) / 1e12, us)
    wpc = max(res, key=lambda k: res[k][0])
    return {"TFLOPS": round(res[wpc][0], 1), "workgroups_per_cu": wpc, "us": round(res[wpc][1], 2),
            "TFLOPS_by_workgroups_per_cu": {str(k): round(v[0], 1) for k, v in res.items()},
            "what": "pa_measure_mfma: 4 independent v_mfma_f32_32x32x16_bf16 chains per wavefront on register "
                    f"operands, {iters} rounds, events around the kernel; the best of 1, 2 and 4 workgroups of 4 "
                    "wavefronts per CU"}


def _cpu_baseline(w, budget_s: float):
    """The oracle (fp64 NumPy, untuned) on a bounded sample of the same
    workload: whole sequences in a fixed shuffled order, cycling through the
    batch again while less than budget_s of CPU work has been done, scaled to
    GB/s of KV rows read."""
    import numpy as np
    import oracle as O
    from synth import stored_np

    cfg = w.cfg
    kc, vc = stored_np(w.k_cache), stored_np(w.v_cache)
    q, tbl, lens = stored_np(w.q), stored_np(w.block_tables), stored_np(w.context_lens)
    elem = 4 if cfg.dtype == "f32" else 2
    row = 2 * cfg.num_kv_heads * cfg.head_dim * elem
    done, nbytes, t = 0, 0, 0.0
    order = np.random.default_rng(0).permutation(len(lens))
    while t < budget_s:
        b = int(order[done % len(order)])
        t0 = time.perf_counter()
        O.decode(q[b:b + 1], kc, vc, tbl[b:b + 1], lens[b:b + 1], w.scale, cfg.dtype)
        t += time.perf_counter() - t0
        nbytes += int(lens[b]) * row
        done += 1
    threads = 1
    try:
        from threadpoolctl import threadpool_info
        threads = max([1] + [int(i.get("num_threads", 1)) for i in threadpool_info()])
    except Exception:  # noqa: BLE001
        pass
    return {
        "value": round(nbytes / t / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} single-sequence decodes ({done / len(lens):.1f} passes over the {len(lens)} "
                  f"sequences, {nbytes / 1e6:.1f} MB of KV rows) in {t:.1f} s, fp64 NumPy; host has "
                  f"{len(os.sched_getaffinity(0))} usable cores",
    }


def _cpu_baseline_prefill(w, budget_s: float):
    """The oracle (fp64 NumPy, untuned) on a bounded sample of the prefill
    workload: whole sequences in a fixed shuffled order while less than
    budget_s of CPU work has been done, scaled to TFLOP/s of the same
    algorithmic flops."""
    import numpy as np
    import oracle as O
    from synth import stored_np

    cfg = w.cfg
    kc, vc = stored_np(w.k_cache).copy(), stored_np(w.v_cache).copy()
    O.write_kv(kc, vc, stored_np(w.k_new), stored_np(w.v_new), stored_np(w.slot_mapping))
    q, tbl, lens, qsl = stored_np(w.q), stored_np(w.block_tables), stored_np(w.context_lens), stored_np(w.query_start_loc)
    order = np.random.default_rng(0).permutation(len(lens))
    done, flops, t = 0, 0, 0.0
    while t < budget_s and done < 4 * len(lens):
        b = int(order[done % len(order)])
        s0, s1 = int(qsl[b]), int(qsl[b + 1])
        t0 = time.perf_counter()
        O.prefill(q[s0:s1], kc, vc, tbl[b:b + 1], lens[b:b + 1], np.array([0, s1 - s0]), w.scale, cfg.dtype)
        t += time.perf_counter() - t0
        L, n = s1 - s0, int(lens[b])
        flops += 4 * cfg.head_dim * cfg.num_heads * (L * (n - L) + L * (L + 1) // 2)
        done += 1
    threads = 1
    try:
        from threadpoolctl import threadpool_info
        threads = max([1] + [int(i.get("num_threads", 1)) for i in threadpool_info()])
    except Exception:  # noqa: BLE001
        pass
    return {
        "value": round(flops / t / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} single-sequence prefills of the {len(lens)} sequences ({flops / 1e9:.1f} GFLOP) "
                  f"in {t:.1f} s, fp64 NumPy; host has {len(os.sched_getaffinity(0))} usable cores",
    }


BM_METRIC = "host block manager: decode-step appends/s (+ prompt admissions/s, frees/s)"


def run_block_manager(args):
    """Host-only: the C++ block manager on a serving workload with a shared
    system prompt -- admit every request (prefix matching and allocation),
    run decode steps (one batched append per step: the step's slot_mapping),
    free everything.  The oracle runs a bounded sample of the same workload."""
    import numpy as np

    import paged_kv_cache_70_amd as pk
    import oracle.block_manager as OBM

    R, bs, system_len, steps = 4096, 16, 1024, 128
    rng = np.random.default_rng(7)
    system = rng.integers(0, 32000, system_len)
    suffix = rng.integers(64, 1025, R)
    prompts = [np.concatenate([system, rng.integers(0, 32000, int(n))]) for n in suffix]
    nb = sum((len(p) + steps + bs - 1) // bs for p in prompts)
    step_tokens = rng.integers(0, 32000, (steps, R))

    def run(bm, n_req, n_steps, batched):
        t0 = time.perf_counter()
        sids = [bm.add_sequence(p)[0] for p in prompts[:n_req]]
        t1 = time.perf_counter()
        for s in range(n_steps):
            if batched:
                bm.append_batch(sids, step_tokens[s, :n_req])
            else:
                for i, sid in enumerate(sids):
                    bm.append(sid, int(step_tokens[s, i]))
        t2 = time.perf_counter()
        for sid in sids:
            bm.free_sequence(sid)
        t3 = time.perf_counter()
        return t1 - t0, t2 - t1, t3 - t2

    for _ in range(max(args.warmup, 1)):
        run(pk.BlockManager(nb, bs), R, 4, True)
    times = [run(pk.BlockManager(nb, bs), R, steps, True) for _ in range(max(1, min(args.steps, 5)))]
    adm, app, fr = (min(t[i] for t in times) for i in range(3))
    res = {
        "metric": BM_METRIC,
        "value": round(R * steps / app, 1),
        "unit": "appended tokens/s",
        "n_gpus": 0,
        "steps": len(times),
        "warmup": max(args.warmup, 1),
        "ms_per_step": round(app / steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int64",
        "data": "synthetic (seeded token ids)",
        "config": {"workload": "prefix_serving_host", "requests": R, "block_size": bs,
                   "system_prompt_tokens": system_len, "suffix_tokens": [64, 1024], "decode_steps": steps,
                   "num_blocks": nb},
        "admissions_per_s": round(R / adm, 1),
        "prompt_tokens_per_s": round(sum(len(p) for p in prompts) / adm, 1),
        "frees_per_s": round(R / fr, 1),
        "ms_per_decode_step": round(app / steps * 1e3, 4),
        "timing": "best of the timed runs, host wall clock; one decode step = one batched append over every "
                  "request (its slot_mapping); each run uses a fresh manager",
        "roofline": None,
    }
    if not args.no_cpu_baseline:
        n_req, n_steps = 256, 16
        ta, tb, tc = run(OBM.BlockManager(nb, bs), n_req, n_steps, False)
        res["cpu_baseline"] = {
            "value": round(n_req * n_steps / tb, 1), "unit": "appended tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_req} requests, {n_steps} decode steps (Python oracle, one thread); admissions "
                      f"{n_req / ta:.1f}/s, frees {n_req / tc:.1f}/s",
        }
    print(json.dumps(res), flush=True)


def run_prefill(args, cfg):
    """Chunked-prefill step: write the chunks' K/V, then paged causal attention."""
    import torch

    import paged_kv_cache_70_amd as pk
    from synth import make_prefill

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = make_prefill(cfg, dev)
    T, H, D = w.q.shape
    kc, vc = w.k_cache, w.v_cache
    if args.layout == "vllm":
        from synth import to_vllm_layout
        kc, vc = to_vllm_layout(kc, vc)
    out = torch.empty_like(w.q)
    ws = pk.prefill_workspace(cfg.num_seqs, H, w.block_tables.shape[1], T, kc)
    flush = None if args.hot else torch.ones(1 << 28, dtype=torch.float32, device=dev)
    flush_sink = torch.zeros((), dtype=torch.float32, device=dev)

    def write():
        pk.write_kv(kc, vc, w.k_new, w.v_new, w.slot_mapping)

    def attend():
        pk.prefill(w.q, kc, vc, w.block_tables, w.context_lens, w.query_start_loc, w.scale,
                   out=out, workspace=ws)

    def do_flush():
        if flush is not None:
            torch.sum(flush, dim=0, out=flush_sink)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    _calibration_copy(args.copy_calibration, dev, do_flush)
    for _ in range(args.warmup):
        do_flush()
        write()
        attend()
    torch.cuda.synchronize()
    events = [(ev(), ev(), ev()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        do_flush()
        e = events[i]
        e[0].record()
        write()
        e[1].record()
        attend()
        e[2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = [e[0].elapsed_time(e[2]) * 1e3 for e in events]
    wr = [e[0].elapsed_time(e[1]) * 1e3 for e in events]
    ak = [e[1].elapsed_time(e[2]) * 1e3 for e in events]
    mean = lambda x: sum(x) / len(x)
    flops = w.flops()
    step_us, wr_us, ak_us = mean(st), mean(wr), mean(ak)
    value = flops / (step_us * 1e-6) / 1e12
    achieved = flops / (ak_us * 1e-6) / 1e12
    row = cfg.num_kv_heads * D * 2
    write_bytes = T * row * 2 * 2 + 8 * T
    res = {
        "metric": PREFILL_METRIC,
        "value": round(value, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_us / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) values, shuffled physical blocks)",
        "config": {
            "workload": cfg.name, "num_seqs": cfg.num_seqs, "num_heads": H, "num_kv_heads": cfg.num_kv_heads,
            "head_dim": D, "block_size": cfg.block_size, "cached_tokens": w.cached, "new_tokens": w.new,
            "query_tokens": T, "cache_layout": args.layout, "cache_flush_between_steps": flush is not None,
        },
        "flops_per_step": flops,
        "prefill_kernel_us": round(ak_us, 2),
        "write_us": round(wr_us, 2),
        "write_GBps": round(write_bytes / (wr_us * 1e-6) / 1e9, 2),
        "step_us_p10_p50_p90": [round(sorted(st)[min(len(st) - 1, int(q * len(st)))], 2) for q in (0.1, 0.5, 0.9)],
        "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 4),
        "timing": "step = events around the write and prefill kernels launched one after another; the "
                  "prefill kernel's share from the middle event",
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": _traffic(cfg.name, "prefill", args.layout),
            "kernel": "prefill_mfma_kernel",
        },
    }
    ceil = _mfma_ceiling(args, dev)
    res["mfma_ceiling_TFLOPS"] = ceil["TFLOPS"]
    res["frac_of_mfma_ceiling"] = round(achieved / ceil["TFLOPS"], 4)
    res["mfma_ceiling"] = ceil
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = _cpu_baseline_prefill(w, args.cpu_budget)
    print(json.dumps(res), flush=True)


def _cpu_baseline_write(w, budget_s: float):
    """The oracle's write (untuned: one token at a time) on the same
    workload, repeated while less than budget_s of CPU work has been done,
    scaled to GB/s of the same bytes."""
    import oracle as O
    from synth import stored_np

    kc, vc = stored_np(w.k_cache).copy(), stored_np(w.v_cache).copy()
    k, v, sl = stored_np(w.k_new), stored_np(w.v_new), stored_np(w.slot_mapping)
    done, t = 0, 0.0
    while t < budget_s:
        t0 = time.perf_counter()
        O.write_kv(kc, vc, k, v, sl)
        t += time.perf_counter() - t0
        done += 1
    return {
        "value": round(w.bytes_moved() * done / t / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{done} whole writes of the {w.slot_mapping.numel()} tokens in {t:.1f} s (Python loop "
                  f"over tokens, NumPy row copies); host has {len(os.sched_getaffinity(0))} usable cores",
    }


def run_write(args, cfg):
    """The paged KV write on its own, at a prefill-sized token count."""
    import torch

    import paged_kv_cache_70_amd as pk
    from synth import make_write

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = make_write(cfg, dev)
    kc, vc = w.k_cache, w.v_cache
    vllm = args.layout == "vllm"
    if vllm:
        from synth import to_vllm_layout
        kc, vc = to_vllm_layout(kc, vc)
    flush = None if args.hot else torch.ones(1 << 28, dtype=torch.float32, device=dev)
    flush_sink = torch.zeros((), dtype=torch.float32, device=dev)

    def write():
        pk.write_kv(kc, vc, w.k_new, w.v_new, w.slot_mapping)

    def do_flush():
        if flush is not None:
            torch.sum(flush, dim=0, out=flush_sink)

    _calibration_copy(args.copy_calibration, dev, do_flush)

    for _ in range(args.warmup):
        do_flush()
        write()
    torch.cuda.synchronize()
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        do_flush()
        events[i][0].record()
        write()
        events[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = [a.elapsed_time(b) * 1e3 for a, b in events]
    us = sum(st) / len(st)
    nbytes = w.bytes_moved()
    gbps = nbytes / (us * 1e-6) / 1e9
    T = w.slot_mapping.numel()
    res = {
        "metric": METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) values; 16 prompts' tokens into shuffled physical blocks)",
        "config": {
            "workload": cfg.name, "tokens": T, "valid_tokens": w.valid_tokens, "num_kv_heads": cfg.num_kv_heads,
            "head_dim": cfg.head_dim, "block_size": cfg.block_size, "num_blocks": kc.shape[0],
            "cache_layout": args.layout, "cache_flush_between_steps": flush is not None,
        },
        "bytes_per_step": nbytes,
        "write_us": round(us, 2),
        "step_us_p10_p50_p90": [round(sorted(st)[min(len(st) - 1, int(q * len(st)))], 2) for q in (0.1, 0.5, 0.9)],
        "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 4),
        "timing": "events around the write kernel alone; bytes = valid K and V rows read and written + 8 B "
                  "of slot per token",
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(gbps / HBM_PEAK_GBPS, 4),
            "traffic": _traffic(cfg.name, "write", args.layout),
            "kernel": "write_kv_vllm_kernel" if vllm else "write_kv_kernel",
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = _cpu_baseline_write(w, args.cpu_budget)
    print(json.dumps(res), flush=True)


def run_graph_compare(args, cfg):
    """Eager write + decode steps against the same step replayed from a HIP
    graph: steps bracketed by events after the flush (the bench's method),
    then back-to-back steps with no flush and no events (wall clock), which
    shows the host's enqueue cost.  Under rocprofv3 --kernel-trace the first
    warmup + steps step groups are eager and the last warmup + steps are
    replays (--trace-summary splits them so)."""
    import torch

    import paged_kv_cache_70_amd as pk
    from synth import make_workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = make_workload(cfg, dev)
    B, H, D = w.q.shape
    W = w.block_tables.shape[1]
    kc, vc = w.k_cache.clone(), w.v_cache.clone()
    ws = pk.new_workspace(B, H, W, kc)
    out = torch.empty_like(w.q)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.zeros((), dtype=torch.float32, device=dev)

    def step():
        pk.write_kv(kc, vc, w.k_new, w.v_new, w.slot_mapping)
        pk.decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, out=out, workspace=ws)

    def timed(fn):
        for _ in range(args.warmup):
            torch.sum(flush, dim=0, out=sink)
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for a, b in evs:
            torch.sum(flush, dim=0, out=sink)
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / len(evs) * 1e3

    eager = timed(step)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    graph = timed(g.replay)
    M = 200

    def wall(fn, sync):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(M):
            fn()
        if sync:
            torch.cuda.synchronize()
        t = (time.perf_counter() - t0) / M * 1e6
        torch.cuda.synchronize()
        return t

    res = {
        "config": {"workload": cfg.name},
        "step": "pa_write_kv + pa_decode",
        "eager_step_us": round(eager, 2), "graph_step_us": round(graph, 2),
        "back_to_back_us_per_step": {"eager": round(wall(step, True), 2), "graph": round(wall(g.replay, True), 2)},
        "host_enqueue_us_per_step": {"eager": round(wall(step, False), 2), "graph": round(wall(g.replay, False), 2)},
        "timing": "eager/graph_step_us: events around one step after a 1 GiB read flush, mean of --steps; "
                  "back-to-back: wall clock of 200 steps with no flush and no events; host enqueue: the same "
                  "without waiting for the GPU",
    }
    print(json.dumps(res), flush=True)


def trace_summary(csv_path: str, warmup: int, steps_timed: int) -> None:
    """Summary of a rocprofv3 --kernel-trace CSV of a --graph-compare run: the
    library's kernels from a write that follows a flush up to the next write
    form one step; of the flushed steps, the first warmup + steps are eager
    (the timed ones after the warm-up are summarised) and the last `steps`
    are the timed graph replays.  Prints, per kind, the time from the flush
    kernel's end to the step's first kernel, the gaps between the step's
    kernels, the step's span and each kernel's duration."""
    import csv
    rows = sorted(csv.DictReader(open(csv_path)), key=lambda r: int(r["Start_Timestamp"]))
    ks = [(r["Kernel_Name"].split("(")[0], int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows]
    steps = []
    for i, (n, a, b) in enumerate(ks):
        if "write_kv_kernel" in n and i > 0 and "reduce_kernel" in ks[i - 1][0]:
            j, st = i, []
            while j < len(ks) and "pa::" in ks[j][0] and (j == i or "write_kv_kernel" not in ks[j][0]):
                st.append(ks[j])
                j += 1
            steps.append((ks[i - 1][2], st))
    print("| step | steps | flush end -> first kernel (us) | gaps between the step's kernels (us) | "
          "first start -> last end (us) | kernel durations (us) |")
    print("|---|---|---|---|---|---|")
    for lab, sts in (("eager", steps[warmup:warmup + steps_timed]), ("graph replay", steps[-steps_timed:])):
        g0 = [st[0][1] - fe for fe, st in sts]
        span = [st[-1][2] - st[0][1] for fe, st in sts]
        inner = [y[1] - x[2] for fe, st in sts for x, y in zip(st, st[1:])]
        durs = {}
        for fe, st in sts:
            for n, a, b in st:
                durs.setdefault(n.replace("void ", "").split("<")[0], []).append(b - a)
        print(f"| {lab} | {len(sts)} | {sum(g0) / len(g0) / 1e3:.2f} | {sum(inner) / max(1, len(inner)) / 1e3:.2f} | "
              f"{sum(span) / len(span) / 1e3:.2f} | " +
              ", ".join(f"{k} {sum(v) / len(v) / 1e3:.2f}" for k, v in durs.items()) + " |")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="llama3_8b_bf16")
    ap.add_argument("--partition", type=int, default=0, help="tokens per split-KV partition (0 = library's choice)")
    ap.add_argument("--hot", action="store_true", help="do not flush the last-level cache between steps")
    ap.add_argument("--layout", choices=["p09", "vllm"], default="p09",
                    help="cache layout: P09's [NB, bs, KVH, D] (default) or vLLM's packed K [NB, KVH, D/x, bs, x] "
                         "with V [NB, KVH, D, bs] (bf16 decode, prefill and write configs)")
    ap.add_argument("--shared-tokens", type=int, default=-1,
                    help="decode with pa_decode_shared_prefix and this hint (default: the workload's common "
                         "prefix for prefix_shared_bf16, else 0 = pa_decode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replay timing")
    ap.add_argument("--step", choices=["auto", "append", "three"], default="auto",
                    help="decode step timed as the step: pa_decode_append (two kernels), or write + partial + "
                         "merge; auto takes the append step when the write is one newest token per sequence")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before the steps, run a plain fp32 copy of MIB MiB three times (the reference "
                         "reading for HBM byte counters)")
    ap.add_argument("--graph-compare", action="store_true",
                    help="time the write + decode step eagerly and replayed from a HIP graph (see run_graph_compare)")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="no GPU run: summarise a rocprofv3 kernel trace of a --graph-compare run")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU run: turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of a "
                         "--copy-calibration run into profiles/traffic_<kernel>_<workload>.json "
                         "(..._<workload>_vllm.json with --layout vllm)")
    args = ap.parse_args()

    if args.traffic_from:
        from synth import CONFIGS, PREFILL_CONFIGS, WRITE_CONFIGS
        if args.config in WRITE_CONFIGS:
            name, key = args.config, "write"
        elif args.config in PREFILL_CONFIGS:
            name, key = args.config, "prefill"
        else:
            name, key = CONFIGS[args.config].name, CONFIGS[args.config].dtype
        r = traffic_from_counters(*args.traffic_from, name, key,
                                  (args.copy_calibration or 256) << 20, _traffic_file(key, name, args.layout),
                                  args.layout)
        print(json.dumps(r))
        return

    if args.trace_summary:
        return trace_summary(args.trace_summary, args.warmup, args.steps)

    if args.config == "prefix_serving_host":
        return run_block_manager(args)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_70_amd as pk
    from synth import CONFIGS, make_workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    pk.load_library()
    from synth import PREFILL_CONFIGS, WRITE_CONFIGS
    if args.config in PREFILL_CONFIGS:
        return run_prefill(args, PREFILL_CONFIGS[args.config])
    if args.config in WRITE_CONFIGS:
        return run_write(args, WRITE_CONFIGS[args.config])
    if args.graph_compare:
        return run_graph_compare(args, CONFIGS[args.config])
    cfg = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = make_workload(cfg, dev)
    B, H, D = w.q.shape
    W = w.block_tables.shape[1]
    kc, vc = w.k_cache, w.v_cache
    if args.layout == "vllm":
        from synth import to_vllm_layout
        kc, vc = to_vllm_layout(kc, vc)
    P = args.partition or pk.partition_size(B, H, W, kc)
    ws = pk.new_workspace(B, H, W, kc, P)
    out = torch.empty_like(w.q)
    flush = None if args.hot else torch.ones(1 << 28, dtype=torch.float32, device=dev)
    flush_sink = torch.zeros((), dtype=torch.float32, device=dev)

    # pa_decode == pa_decode_partials then pa_decode_merge (same kernels); the
    # halves are called separately so that the partial kernel can be timed.
    def write():
        pk.write_kv(kc, vc, w.k_new, w.v_new, w.slot_mapping)

    shared = args.shared_tokens if args.shared_tokens >= 0 else (
        int(cfg.ctx[1]) if cfg.ctx[0] == "prefix" else 0)

    def partials():
        if shared:
            pk.decode_partials_shared_prefix(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, shared,
                                             out=out, workspace=ws, partition_size=P)
        else:
            pk.decode_partials(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, out=out,
                               workspace=ws, partition_size=P)

    def merge():
        pk.decode_merge(w.q, kc, w.block_tables, w.context_lens, out=out, workspace=ws,
                        partition_size=P)

    # The append step (pa_decode_append: the partial kernel over the cached
    # tokens, then one merge that folds in and writes each sequence's new
    # token) does the same work as write + decode when the write is exactly
    # one newest token (position n_b - 1) per sequence.
    bsz = cfg.block_size
    ctx_h = w.context_lens.cpu().to(torch.int64)
    tbl_h = w.block_tables.cpu().to(torch.int64)
    live = ctx_h > 0
    pos = (ctx_h - 1).clamp(min=0)
    newest = torch.where(live, tbl_h[torch.arange(B), pos // bsz] * bsz + pos % bsz, torch.full_like(ctx_h, -1))
    sm = w.slot_mapping.cpu()
    newest_write = (sm.numel() == int(live.sum()) and bool((sm >= 0).all())
                    and torch.equal(torch.sort(sm).values, torch.sort(newest[live]).values))
    if args.step == "append" and (not newest_write or not bool(live.all()) or shared):
        print(f"--step append needs a write of exactly one newest token per sequence and no shared-prefix hint; "
              f"{cfg.name}'s write is not that (use --step three or auto)", file=sys.stderr)
        sys.exit(2)
    use_append = args.step == "append" or (args.step == "auto" and not shared and newest_write)
    if use_append:
        row_of = {int(x): i for i, x in enumerate(sm.tolist())}
        idx = torch.tensor([row_of[int(x)] if x >= 0 else 0 for x in newest.tolist()], dtype=torch.int64,
                           device=dev)
        app_k, app_v = w.k_new.index_select(0, idx), w.v_new.index_select(0, idx)
        app_slots = newest.to(dev)
        cached = (ctx_h - live.to(torch.int64)).to(torch.int32).to(dev)
        aws = pk.new_append_workspace(B, H, W, kc, P)

    def append_step():
        pk.decode_append(w.q, kc, vc, app_k, app_v, app_slots, w.block_tables, cached, w.scale, out=out,
                         workspace=aws, partition_size=P)

    def do_flush():
        if flush is not None:
            torch.sum(flush, dim=0, out=flush_sink)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    _calibration_copy(args.copy_calibration, dev, do_flush)

    for _ in range(args.warmup):
        do_flush()
        write()
        partials()
        merge()
    torch.cuda.synchronize()

    # The timed steps: write + decode, bracketed by two events (the flush before
    # each step is outside them).
    events = [(ev(), ev()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        do_flush()
        events[i][0].record()
        write()
        partials()
        merge()
        events[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = [a.elapsed_time(b) * 1e3 for a, b in events]          # µs
    st3 = st
    if use_append:
        # the same steps as the append entry point: two kernels
        for _ in range(args.warmup):
            do_flush()
            append_step()
        aev = [(ev(), ev()) for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            do_flush()
            aev[i][0].record()
            append_step()
            aev[i][1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        st = [a.elapsed_time(b) * 1e3 for a, b in aev]

    # The same steps again, with events around each kernel: the partial kernel's
    # duration feeds the roofline; write and merge are reported beside it.
    kev = [(ev(), ev(), ev(), ev()) for _ in range(args.steps)]
    for i in range(args.steps):
        do_flush()
        e = kev[i]
        e[0].record()
        write()
        e[1].record()
        partials()
        e[2].record()
        merge()
        e[3].record()
    torch.cuda.synchronize()
    wr = [e[0].elapsed_time(e[1]) * 1e3 for e in kev]
    k2 = [e[1].elapsed_time(e[2]) * 1e3 for e in kev]
    k3 = [e[2].elapsed_time(e[3]) * 1e3 for e in kev]
    mean = lambda x: sum(x) / len(x)

    # The same step captured once in a HIP graph (the library enqueues only
    # kernels: no host synchronisation, allocation or memset) and replayed;
    # the flush stays outside.  Reported beside the step, not as the step.
    gst = []
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            write()
            partials()
            merge()                     # warm the capture stream once
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            write()
            partials()
            merge()
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            do_flush()
            graph.replay()
        gev = [(ev(), ev()) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            do_flush()
            gev[i][0].record()
            graph.replay()
            gev[i][1].record()
        torch.cuda.synchronize()
        gst = [a.elapsed_time(b) * 1e3 for a, b in gev]

    # Hot steps: the same step without the flush before it (the last-level
    # cache may still hold rows of the step before); reported beside the
    # flushed number, labelled as hot.
    hot = []
    if flush is not None:
        for _ in range(args.warmup):
            append_step() if use_append else (write(), partials(), merge())
        hev = [(ev(), ev()) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            hev[i][0].record()
            if use_append:
                append_step()
            else:
                write()
                partials()
                merge()
            hev[i][1].record()
        torch.cuda.synchronize()
        hot = [a.elapsed_time(b) * 1e3 for a, b in hev]

    def pct(x, q):
        s = sorted(x)
        return s[min(len(s) - 1, int(q * len(s)))]

    ceiling = _read_ceiling(w.kv_unique_bytes(), args, dev, do_flush)

    kv_bytes = w.kv_bytes()
    # the HBM roofline takes the distinct rows: a prefix block shared by many
    # tables is fetched from HBM once and then served from cache
    kv_unique = w.kv_unique_bytes()
    elem = 4 if cfg.dtype == "f32" else 2
    row = cfg.num_kv_heads * D * elem
    n_valid = int((w.slot_mapping >= 0).sum())
    write_bytes = n_valid * row * 2 * 2 + 8 * w.slot_mapping.numel()
    step_us = mean(st)
    wr_us, k2_us, k3_us = mean(wr), mean(k2), mean(k3)
    dec_us = k2_us + k3_us
    value = kv_bytes / (step_us * 1e-6) / 1e9
    achieved = kv_unique / (k2_us * 1e-6) / 1e9
    traffic = _traffic(cfg.name, cfg.dtype, args.layout)

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_us / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) values, shuffled physical blocks)",
        "config": {
            "workload": cfg.name, "num_seqs": B, "num_heads": H, "num_kv_heads": cfg.num_kv_heads,
            "head_dim": D, "block_size": cfg.block_size, "context_lens": list(cfg.ctx),
            "write_tokens": int(w.slot_mapping.numel()), "partition_size": P, "cache_layout": args.layout,
            "shared_prefix_hint_tokens": shared,
            "cache_flush_between_steps": flush is not None,
        },
        "hbm_frac_step": round(kv_unique / (step_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "hbm_frac_three_kernel_step": round(kv_unique / (mean(st3) * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "ceiling_GBps": ceiling["GBps"],
        "frac_of_ceiling": round(achieved / ceiling["GBps"], 4),
        "step_frac_of_ceiling": round(kv_unique / (step_us * 1e-6) / 1e9 / ceiling["GBps"], 4),
        "ceiling_read": ceiling,
        "hot_step_us": round(mean(hot), 2) if hot else None,
        "hot_hbm_frac_step": round(kv_unique / (mean(hot) * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4) if hot else None,
        "decode_us": round(dec_us, 2),
        "decode_kv_GBps": round(kv_bytes / (dec_us * 1e-6) / 1e9, 1),
        "partial_kernel_us": round(k2_us, 2),
        "merge_kernel_us": round(k3_us, 2),
        "step_us_p10_p50_p90": [round(pct(st, q), 2) for q in (0.1, 0.5, 0.9)],
        "step_kernels": "pa_decode_append (partial + merge-append)" if use_append else "write + partial + merge",
        "three_kernel_step_us": round(mean(st3), 2),
        "graph_step_us": round(mean(gst), 2) if gst else None,
        "write_us": round(wr_us, 2),
        "write_GBps": round(write_bytes / (wr_us * 1e-6) / 1e9, 2),
        "kv_bytes_per_step": kv_bytes,
        "kv_unique_bytes_per_step": kv_unique,
        "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 4),
        "timing": ("step = events around one pa_decode_append call (partial kernel over the cached tokens, "
                   "then a merge that folds in and writes each sequence's new token); three_kernel_step_us: "
                   "write, partial and merge kernels launched one after another" if use_append else
                   "step = events around the write, partial and merge kernels launched one after another") +
                  " (graph_step_us: the three-kernel step replayed from a HIP graph); per-kernel times from a "
                  "second pass with events around each kernel (each includes ~1-3 us of event/launch gap)",
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel": _kernel_name(cfg.dtype, args.layout),
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = _cpu_baseline(w, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
