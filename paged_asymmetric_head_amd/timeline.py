"""Per-workgroup timelines of the split-KV kernel from the timeline build
(libdiffkv_attn_timeline.so, see diffkv_attn_timeline_buffer).

    python -m paged_asymmetric_head_amd.timeline batched_decode verify_long swa_sinks_fp8_p128

For each workload: the inputs are uploaded, the K/V pool is copied until the
copies exceed 1 GiB (each call reads a copy no earlier call left in the
caches), a few calls warm up, then each timed call runs alone (the stamp
buffer cleared before it, the stream synchronised after it) and every
workgroup that finished a chunk reports its eight real-time stamps (100 MHz).
Printed as Markdown: percentiles of each stamp over all workgroups of all
timed calls, from the call's first workgroup start; the span of each call;
and means by XCD (workgroup w runs on XCD w % 8 in dispatch order).
"""

import argparse
import math
import sys

import numpy as np
import torch

from . import binding as B
from .device import DeviceInputs
from .synth import workload

ENTRY = {"batched_decode": "decode", "batched_decode_sym": "decode", "tiny_decode": "decode",
         "verify_long": "verify", "swa_sinks_fp8_p1": "verify", "swa_sinks_fp8_p128": "verify"}
SLOTS = 8
PHASES = [(0, "start"), (1, "lengths in"), (2, "own key range known"), (3, "first K/V data in"),
          (4, "first tile done"), (5, "last round of the tile loop"), (6, "epilogue"),
          (7, "output stores issued")]
TICK_US = 0.01                      # the real-time counter runs at 100 MHz
PCT = (0, 10, 50, 90, 100)


def collect(name, calls_timed=4, warmup=3, max_workgroups=8192):
    """Stamps of every workgroup that finished a chunk, per timed call, in us
    from that call's first workgroup start: a list of (W, 8) arrays (0 where
    a workgroup did not pass a point, NaN for its start-relative value) and
    the workgroup index of each row."""
    inp = workload(name)
    dev = DeviceInputs(inp)
    pool = dev.k_cache.numel() * dev.k_cache.element_size() + dev.v_cache.numel() * dev.v_cache.element_size()
    copies = max(1, min(16, math.ceil((1 << 30) / pool)))
    caches = [(dev.k_cache, dev.v_cache)] + [(dev.k_cache.clone(), dev.v_cache.clone())
                                              for _ in range(copies - 1)]
    stream = torch.cuda.current_stream().cuda_stream
    calls = [dev.prepare(ENTRY[name], k_cache=k, v_cache=v, stream=stream) for k, v in caches]
    stamps = torch.zeros(max_workgroups * SLOTS, dtype=torch.int64, device=dev.device)
    if B.diffkv_attn_timeline_buffer(stamps) != B.OK:
        raise B.DiffKVError("the timeline build is not selected")
    for i in range(warmup):
        calls[i % copies]()
    torch.cuda.synchronize()
    out = []
    for i in range(calls_timed):
        stamps.zero_()
        torch.cuda.synchronize()
        calls[(warmup + i) % copies]()
        torch.cuda.synchronize()
        d = stamps.view(-1, SLOTS).cpu().numpy().astype(np.float64)
        wg = np.flatnonzero(d[:, 7] > 0)
        d = d[wg]
        t0 = d[:, 0].min()
        rel = np.where(d > 0, (d - t0) * TICK_US, np.nan)
        out.append((rel, wg))
    B.diffkv_attn_timeline_buffer(None)
    return out


def pct(x):
    x = x[~np.isnan(x)]
    if x.size == 0:
        return " | ".join("-" for _ in PCT)
    return " | ".join(f"{np.percentile(x, q):.2f}" for q in PCT)


def report(name, runs):
    rel = np.concatenate([r for r, _ in runs])
    wg = np.concatenate([w for _, w in runs])
    spans = np.array([np.nanmax(r[:, 7]) for r, _ in runs])
    lines = [f"### {name}: {len(runs)} calls, {rel.shape[0]} workgroup records", "",
             "| point | " + " | ".join(f"p{q}" for q in PCT) + " |",
             "|---|" + "---|" * len(PCT)]
    for k, label in PHASES:
        lines.append(f"| {k} {label} | {pct(rel[:, k])} |")
    lines.append(f"| span of the call (last store issued) | {pct(spans)} |")
    lines += ["", "| XCD | " + " | ".join(str(x) for x in range(8)) + " |", "|---|" + "---|" * 8]
    xcd = wg % 8
    for k, label in [(0, "start"), (3, "first K/V data in"), (7, "stores issued")]:
        lines.append(f"| mean {label} | " + " | ".join(
            f"{np.nanmean(rel[xcd == x, k]):.2f}" if (xcd == x).any() else "-" for x in range(8)) + " |")
    stream = rel[:, 7] - rel[:, 3]
    lines.append("| mean from first data to stores | " + " | ".join(
        f"{np.nanmean(stream[xcd == x]):.2f}" if (xcd == x).any() else "-" for x in range(8)) + " |")
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("workloads", nargs="+", choices=sorted(ENTRY))
    ap.add_argument("--calls", type=int, default=4)
    args = ap.parse_args(argv)
    B.select_library("timeline")
    for name in args.workloads:
        print(f"[timeline] {name}", file=sys.stderr, flush=True)
        print(report(name, collect(name, calls_timed=args.calls)), flush=True)


if __name__ == "__main__":
    main()
