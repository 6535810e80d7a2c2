"""Per-wavefront timeline of the bf16 persistent decode kernel.

Runs the partial kernel of one decode workload through ``libpaged_kv_timeline.so``
(the library with the persistent kernel built with -DPA_TIMELINE, made by
``paged_kv_cache_70_amd.build``) and summarises what it recorded: when each
wavefront entered, had its unit list and exited, on which die (XCC) it ran,
and when each unit started and ended.  s_memrealtime ticks at 100 MHz.

    python -m paged_kv_cache_70_amd.timeline llama3_8b_bf16 [--partition P] [--runs N]

Each run is preceded by a 1 GiB read flush, like the benchmark's steps.  The
prefix-shared workload runs with its common prefix as the shared-prefix hint.
Needs a GPU; the numbers are the instrumented build's (a few stores per unit
more than the library proper).
"""
from __future__ import annotations

import argparse
import ctypes
import os

import numpy as np

TICK_US = 0.01                 # s_memrealtime: 100 MHz
WAVE_BASE, UNIT_BASE, WORDS = 16, 32768, 1 << 16


def _pct(x, q):
    return float(np.percentile(x, q)) if len(x) else float("nan")


def summarise(buf: np.ndarray, lens: np.ndarray, P: int, D: int, shared_parts: int, events_us: float) -> list:
    """Lines describing one recorded run (buf: the 64-bit timeline words)."""
    nunit = int(buf[0])
    wv = buf[WAVE_BASE:UNIT_BASE].reshape(-1, 4)
    widx = np.nonzero(wv[:, 0])[0]
    wv = wv[widx]
    un = buf[UNIT_BASE:UNIT_BASE + 4 * min(nunit, 8000)].reshape(-1, 4)
    t0 = int(wv[:, 0].min())
    ts = lambda a: (a.astype(np.int64) - t0) * TICK_US
    entry, listed, exit_ = ts(wv[:, 0]), ts(wv[:, 1]), ts(wv[:, 2])
    xcc = (wv[:, 3] & 0xF).astype(int)
    ustart, uend = ts(un[:, 2]), ts(un[:, 3])
    b = (un[:, 1] >> 40).astype(int)
    p = ((un[:, 1] >> 24) & 0xFFFF).astype(int)
    ntok = np.minimum(lens[b], (p + 1) * P) - p * P
    ubytes = ntok * 2 * D * 2                       # K and V rows of one kv head, bf16
    wg = (un[:, 0] >> 8).astype(int)
    wave = (un[:, 0] & 0xFF).astype(int)
    NW = int((wv[0, 3] >> 8) & 0xFF)                # wavefronts per workgroup, as the kernel recorded it
    T = float(exit_.max())
    out = [f"events {events_us:.1f} us; kernel span (first entry to last exit) {T:.1f} us; wavefronts {len(wv)}, "
           f"units {nunit}; KV bytes streamed {ubytes.sum() / 1e6:.1f} MB ({ubytes.sum() / T / 1e3:.0f} GB/s over the span)",
           f"  entry: last at {entry.max():.2f} us; unit list ready at {listed.min():.2f}-{listed.max():.2f} us "
           f"(mean {listed.mean():.2f})",
           f"  wavefront exit: min {exit_.min():.1f}  p10 {_pct(exit_, 10):.1f}  p50 {_pct(exit_, 50):.1f}  "
           f"p90 {_pct(exit_, 90):.1f}  max {T:.1f} us",
           "  last exit per die: " + " ".join(f"{exit_[xcc == x].max():.1f}" for x in range(8) if (xcc == x).any())]
    wg_of = widx // NW
    ends = np.array([exit_[wg_of == g].max() for g in np.unique(wg_of)])
    firsts = np.array([exit_[wg_of == g].min() for g in np.unique(wg_of)])
    out.append(f"  workgroup end: min {ends.min():.1f}  p50 {_pct(ends, 50):.1f}  max {ends.max():.1f} us; "
               f"spread of wavefront exits inside a workgroup: mean {np.mean(ends - firsts):.1f} us ({NW} per workgroup)")
    dur = uend - ustart
    full = ntok == P
    if full.any():
        out.append(f"  full units ({int(full.sum())}): {dur[full].mean():.1f} us each (sd {dur[full].std():.1f}), "
                   f"{ubytes[full].mean() / dur[full].mean() / 1e3:.2f} GB/s per wavefront")
    # per wavefront with units: their order, and its busy time
    key = wg * NW + wave
    order = np.zeros(len(un), dtype=int)
    busy = []
    for k in np.unique(key):
        idx = np.nonzero(key == k)[0]
        idx = idx[np.argsort(ustart[idx])]
        order[idx] = np.arange(len(idx))
        busy.append(dur[idx].sum())
    busy = np.array(busy)
    tiles = np.maximum(1, (ntok + 15) // 16)
    per_tile = dur / tiles
    shared = p < shared_parts
    for name, m in (("shared", shared), ("private", ~shared)):
        for which, mo in (("first", order == 0), ("later", order > 0)):
            mm = m & mo
            if mm.any():
                out.append(f"  {name} units, {which} of their wavefront ({int(mm.sum())}): "
                           f"{np.median(per_tile[mm]):.2f} us per 16-token tile (median), {tiles[mm].mean():.1f} tiles")
    out.append(f"  wavefronts with units: {len(busy)} of {len(wv)}; their busy time: mean {busy.mean():.1f}  "
               f"p10 {_pct(busy, 10):.1f}  max {busy.max():.1f} us of the {T:.1f} us span")
    return out


def main(argv=None) -> None:
    import torch

    from . import api
    from .build import TIMELINE_LIB
    from synth import CONFIGS, make_workload

    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("config", choices=[k for k, c in CONFIGS.items() if c.dtype == "bf16"])
    ap.add_argument("--partition", type=int, default=0, help="tokens per partition (0: the library's choice)")
    ap.add_argument("--runs", type=int, default=3, help="recorded runs (after one warm-up run)")
    args = ap.parse_args(argv)

    lib = api.load_library(TIMELINE_LIB)
    if not hasattr(lib, "pa_timeline_read"):
        raise SystemExit(f"{TIMELINE_LIB} has no timeline: rebuild with `python -m paged_kv_cache_70_amd.build`")
    dev = torch.device("cuda:0")
    cfg = CONFIGS[args.config]
    w = make_workload(cfg, dev)
    B, H, D = w.q.shape
    W = w.block_tables.shape[1]
    P = args.partition or api.partition_size(B, H, W, w.k_cache)
    shared = int(cfg.ctx[1]) if cfg.ctx[0] == "prefix" else 0
    ws = api.new_workspace(B, H, W, w.k_cache, P)
    out = torch.empty_like(w.q)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.zeros((), dtype=torch.float32, device=dev)
    lens = w.context_lens.cpu().numpy().astype(np.int64)
    print(f"{args.config}: partition {P} tokens" + (f", shared-prefix hint {shared} tokens" if shared else ""),
          flush=True)

    def run():
        if shared:
            api.decode_partials_shared_prefix(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.scale,
                                              shared, out=out, workspace=ws, partition_size=P)
        else:
            api.decode_partials(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.scale, out=out,
                                workspace=ws, partition_size=P)

    buf = np.zeros(WORDS, dtype=np.uint64)
    for i in range(args.runs + 1):
        torch.sum(flush, dim=0, out=sink)
        if lib.pa_timeline_reset() != 0:
            raise SystemExit("pa_timeline_reset failed")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        run()
        b.record()
        torch.cuda.synchronize()
        if i == 0:
            continue
        if lib.pa_timeline_read(ctypes.c_void_p(buf.ctypes.data), buf.nbytes) != 0:
            raise SystemExit("pa_timeline_read failed")
        print(f"run {i}:")
        for line in summarise(buf, lens, P, D, (shared // P) if shared else 0, a.elapsed_time(b) * 1e3):
            print(line, flush=True)


if __name__ == "__main__":
    main()
