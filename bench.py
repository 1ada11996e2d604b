#!/usr/bin/env python3
"""Throughput of the paged asymmetric-head attention path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-extra] [--no-cpu-baseline]

A step is one C-ABI call of the whole path (plan, block-table gather, FP8/bf16
load, QK^T, mask, online softmax, PV, split partials and merge) over one batch
of the seeded synthetic workload.  The headline workload is batched decode
(32 sequences of 8192..9216 tokens, 8 query heads on 1 KV head, page 128,
bf16 K/V); its metric is the KV bytes the visible keys occupy, read per
second from HBM.

The KV pool is replicated into enough copies ("layers") to exceed 1 GiB, and
consecutive steps read consecutive copies, so no step finds its keys in the
256 MB Infinity Cache or the L2.  Inputs are resident in HBM before timing.
The headline takes exactly W warmup steps; the other workloads warm up for
at least 80 ms of their own calls (a long kernel's first launches after a
pause run slower).

One JSON line is printed.  `value` and `ms_per_step` come from the timed
steps alone (HIP events around the K calls, nothing else on the stream).
`roofline` is the main attention kernel alone: a second pass of the same K
calls has the library's dispatch stamp each call's main kernel with its own
HIP events (the descriptor's profile_start / profile_stop).  Their mean, bounded by the step
time, is the kernel's duration `kernel_ms` (`kernel_ms_events` is the raw
mean, `kernel_ms_median` the median).  The stamping itself adds time between
launches, so the stamped pass's steps are not used for `value`.
`roofline.stream_read` (decode and verify) is the achievable-bandwidth
reference at the kernel's own byte count: a plain streaming read of that many
bytes in one launch, cold, timed the same way; `kernel_frac_of_stream` is the
attention kernel's rate as a fraction of it.
`cpu_baseline` times the FP64 oracle on the host's cores (every core of the
process's affinity set, one thread each, BLAS held to one thread) on a bounded
sample of the workload; every attention workload in `extra` carries its own.
`extra` carries the other workloads measured the same way (mixed_batch: one
serving step mixing a prefill chunk, verify blocks and decodes;
batched_decode_sym: the decode batch with symmetric 128/128 heads), the paged KV
write (diffkv_kv_write) on the decode and prefill token counts, and one GPU's
share of a two-way context split of the decode workload (diffkv_attn_partial
over half of every sequence's keys, and the diffkv_attn_combine merge), and a
sweep of the decode shape over context lengths (2K-64K tokens per sequence)
with the fit kernel time = a + bytes / B, and a sweep of the long-verify shape
over batch sizes (4-32 sequences at 40K-50K tokens).
"""

import argparse
import ctypes
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KV-read HBM GB/s (decode/verify) + prefill TFLOP/s, each as % of MI355X peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
ENTRY_OF = {"tiny_decode": "decode", "batched_decode": "decode", "verify_long": "verify",
            "swa_sinks_fp8_p1": "verify", "swa_sinks_fp8_p128": "verify",
            "chunked_prefill": "prefill", "mixed_batch": "mixed", "batched_decode_sym": "decode"}
HEADLINE = "batched_decode"
KERNEL_OF_ENTRY = {"decode": "split_attn_kernel", "verify": "split_attn_kernel",
                   "prefill": "prefill_attn_kernel",
                   "mixed": "split_attn_kernel + prefill_attn_kernel"}


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE,
                    choices=sorted(ENTRY_OF) + sorted(KV_WRITE_OF) + ["context_split_decode", "decode_sweep",
                                                                       "verify_sweep"],
                    help="attention workload for the headline line; a KV-write or context-split "
                         "name prints that measurement's own line instead")
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--extra-steps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target host time for the headline's oracle sample")
    ap.add_argument("--cpu-seconds-extra", type=float, default=4.0,
                    help="target host time for each other workload's oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (reads and writes 256 MiB), the "
                         "reference the HBM byte counters are scaled by")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter files (FETCH_SIZE, WRITE_SIZE) of a "
                         "--copy-calibration run into profiles/hbm_traffic.json and exit")
    return ap.parse_args()


class HipEvents:
    """hipEvent_t handles through the HIP runtime's C API (raw pointers)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        for fn in ("hipEventCreate", "hipEventRecord", "hipEventSynchronize", "hipEventElapsedTime",
                   "hipEventDestroy"):
            getattr(self.lib, fn).restype = ctypes.c_int

    def create(self):
        ev = ctypes.c_void_p()
        if self.lib.hipEventCreate(ctypes.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev.value

    def record(self, ev, stream):
        if self.lib.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)


def algorithmic_work(inp, q_lo=1, q_hi=None):
    """Bytes of the KV rows the visible keys occupy (each read once per
    (sequence, KV head)), (query row, visible key) pairs and their flops,
    over the sequences with q_lo <= q_len <= q_hi."""
    import numpy as np
    esize = 1 if inp.kv_dtype == "fp8" else 2
    keys = 0
    pairs = 0
    qctx = 0
    for b in range(inp.batch):
        L, n = int(inp.seq_lens[b]), int(inp.q_lens[b])
        if n < q_lo or (q_hi is not None and n > q_hi):
            continue
        p = L - n + np.arange(n)
        lo = np.maximum(0, p - inp.window + 1) if inp.window > 0 else np.zeros_like(p)
        keys += int(p.max() + 1 - lo.min())
        vis = int((p - lo + 1).sum())
        qctx += vis
        pairs += vis * inp.num_q_heads
    dqk, dv = inp.q.shape[2], inp.v_cache.shape[3]
    kv_bytes = keys * inp.num_kv_heads * (dqk + dv) * esize
    return {"kv_bytes": kv_bytes, "pairs": pairs, "flops": 2 * (dqk + dv) * pairs, "q_ctx": qctx}


_CODE_TOKENS = re.compile(r'"(?:\\.|[^"\\])*"|\'(?:\\.|[^\'\\])*\'|//[^\n]*|/\*.*?\*/|\s+', re.S)


def _code_only(text):
    """C++ source with comments dropped and whitespace runs collapsed
    (string and character literals kept), so editing a comment does not
    count as a kernel change."""
    def keep(m):
        t = m.group(0)
        return " " if t.startswith("//") or t.startswith("/*") or t.isspace() else t
    return re.sub(r"\s+", " ", _CODE_TOKENS.sub(keep, text)).strip()


def kernel_source_sha():
    """Identifies the kernels the counters were taken on: the code of the HIP
    sources and the public header, and the compile flags."""
    import glob
    from paged_asymmetric_head_amd.build import command
    h = hashlib.sha256()
    paths = sorted(p for p in glob.glob(os.path.join(ROOT, "paged_asymmetric_head_amd", "csrc", "*"))
                   if os.path.basename(p) != "stream_read.hip")
    paths.append(os.path.join(ROOT, "include", "diffkv_attn.h"))
    for path in paths:
        with open(path, encoding="utf-8") as f:
            h.update(os.path.basename(path).encode())
            h.update(_code_only(f.read()).encode())
    # Flags only: the compiler path, the output and the include directories
    # (which name the checkout's location) are left out.
    flags = [c for c in command("OUT")
             if not os.path.isabs(c) and c != "OUT" and "hipcc" not in c and not c.startswith("-I")]
    h.update(" ".join(flags).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload, sha):
    """HBM bytes per launch from the committed counter runs, if they were
    taken on the current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    rec = data.get(workload)
    if not rec or rec.get("source_sha") != sha:
        return None
    return rec.get("bytes_per_launch")


# Extra warmup, by time, for the workloads beside the headline: the chunked
# prefill kernel runs its first 15 or so launches after a pause up to 20%
# slower (2.44 ms falling to 2.07 ms over about 30 ms of back-to-back
# launches, also after 200 ms of other GPU work), so those measurements keep
# calling until this much time has passed.  The headline workload keeps
# exactly its W warmup steps.
EXTRA_WARM_MS = 80.0


def time_calls(calls, steps, warmup, events, stream, warm_ms=0.0):
    """Warm up (`warmup` calls, then more until `warm_ms` milliseconds have
    passed), then time exactly `steps` calls (rotating over `calls`) with a
    pair of HIP events around them and nothing else on the stream.  A second
    pass of the same calls has the library stamp each call's main kernel with
    its own pair of events at dispatch (the call's descriptor carries them
    for that one call; a call without a descriptor, the combine, is one
    kernel and is bracketed by the events on the stream instead); that
    stamping adds time between launches (the stamped pass's steps run longer),
    so the step time comes from the clean pass only.  Returns (total ms, wall
    seconds, sorted per-kernel ms, the stamped pass's total ms)."""
    import torch
    from paged_asymmetric_head_amd import binding as B
    n = len(calls)
    pairs = [(events.create(), events.create()) for _ in range(steps)]
    t0, t1, t2, t3 = (events.create() for _ in range(4))
    for i in range(warmup):
        calls[i % n]()
    torch.cuda.synchronize()
    t_end = time.perf_counter() + warm_ms / 1e3
    i = warmup
    while time.perf_counter() < t_end:
        calls[i % n]()
        torch.cuda.synchronize()
        i += 1
    # Timed region: exactly `steps` calls, nothing else on the stream.
    wall0 = time.perf_counter()
    events.record(t0, stream)
    for k in range(steps):
        calls[k % n]()
    events.record(t1, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = events.elapsed_ms(t0, t1)
    events.record(t2, stream)
    for k in range(steps):
        call = calls[k % n]
        desc = getattr(call, "desc", None)
        if desc is None:
            events.record(pairs[k][0], stream)
            call()
            events.record(pairs[k][1], stream)
        else:
            B.set_profile_events(desc, pairs[k][0], pairs[k][1])
            try:
                call()
            finally:
                B.set_profile_events(desc, None, None)
    events.record(t3, stream)
    torch.cuda.synchronize()
    kern = sorted(events.elapsed_ms(a, b) for a, b in pairs)
    return total_ms, wall, kern, events.elapsed_ms(t2, t3)


def kernel_ms_bounded(kern, step_ms):
    """The stamped kernels' mean duration, bounded by the clean pass's step
    time (a kernel cannot take longer than the call it belongs to; the stamps
    can add a little dispatch time), and the raw mean."""
    raw = sum(kern) / len(kern)
    return min(raw, step_ms), raw


def measure(name, steps, warmup, events, target_bytes=1 << 30, warm_ms=0.0):
    import torch
    from paged_asymmetric_head_amd import binding as B
    from paged_asymmetric_head_amd.device import DeviceInputs
    from paged_asymmetric_head_amd.synth import workload

    entry = ENTRY_OF[name]
    inp = workload(name)
    dev = DeviceInputs(inp)
    pool = dev.k_cache.numel() * dev.k_cache.element_size() + dev.v_cache.numel() * dev.v_cache.element_size()
    layers = max(1, min(16, math.ceil(target_bytes / pool)))
    caches = [(dev.k_cache, dev.v_cache)] + [(dev.k_cache.clone(), dev.v_cache.clone())
                                             for _ in range(layers - 1)]
    stream = torch.cuda.current_stream().cuda_stream
    calls = [dev.prepare(entry, k_cache=k, v_cache=v, stream=stream) for k, v in caches]
    total_ms, wall, kern, stamped_ms = time_calls(calls, steps, warmup, events, stream, warm_ms)
    out = calls[(steps - 1) % layers].out
    if not bool(torch.isfinite(out.float()).all()):
        raise RuntimeError(f"{name}: non-finite output")
    work = algorithmic_work(inp)
    d = dev.desc(entry)
    splits = B.diffkv_attn_num_splits(d, B.ENTRIES[entry], inp.window)
    return {
        "inp": inp, "entry": entry, "layers": layers, "splits": splits,
        "ms_per_step": total_ms / steps, "wall_ms_per_step": 1e3 * wall / steps,
        "kernel_ms_mean": kernel_ms_bounded(kern, total_ms / steps)[0],
        "kernel_ms_events": sum(kern) / len(kern), "kernel_ms_median": kern[len(kern) // 2],
        "stamped_ms_per_step": stamped_ms / steps,
        "work": work,
    }


# Paged KV write, measured on the token counts of two attention workloads:
# one new token per sequence (batched decode, bf16 cache) and a 4096-token
# chunk (chunked prefill, FP8 cache).
KV_WRITE_OF = {"kv_write_decode": "batched_decode", "kv_write_prefill": "chunked_prefill"}


def measure_kv_write(name, steps, warmup, events, target_bytes=1 << 30):
    """Time diffkv_kv_write; the algorithmic bytes are the bf16 rows read and
    the cache rows written (K 192 + V 128 values per token and KV head)."""
    import numpy as np
    import torch
    from paged_asymmetric_head_amd import binding as B
    from paged_asymmetric_head_amd.device import DeviceInputs, _to_device
    from paged_asymmetric_head_amd.synth import to_bf16_bits, workload

    inp = workload(KV_WRITE_OF[name])
    dev = DeviceInputs(inp)
    decode = inp.max_q_len == 1
    T, H = inp.total_q, inp.num_kv_heads
    rng = np.random.default_rng(2)
    pool = dev.k_cache.numel() * dev.k_cache.element_size() + dev.v_cache.numel() * dev.v_cache.element_size()
    layers = max(1, min(16, math.ceil(target_bytes / pool)))
    news = [(_to_device(to_bf16_bits(rng.standard_normal((T, H, 192), dtype=np.float32)), "cuda"),
             _to_device(to_bf16_bits(rng.standard_normal((T, H, 128), dtype=np.float32)), "cuda"))
            for _ in range(layers)]
    caches = [(dev.k_cache, dev.v_cache)] + [(dev.k_cache.clone(), dev.v_cache.clone())
                                             for _ in range(layers - 1)]
    stream = torch.cuda.current_stream().cuda_stream
    d = dev.desc("decode" if decode else "prefill")
    calls = [B.prepared_kv_write(d, kn, vn, kc, vc, dev.block_table, dev.seq_lens,
                                 None if decode else dev.q_lens, inp.k_scale, inp.v_scale, stream)
             for (kn, vn), (kc, vc) in zip(news, caches)]
    total_ms, wall, kern, _ = time_calls(calls, steps, warmup, events, stream)
    esize = 1 if inp.kv_dtype == "fp8" else 2
    nbytes = T * H * (inp.q.shape[2] + inp.v_cache.shape[3]) * (2 + esize)
    ms, ms_raw = kernel_ms_bounded(kern, total_ms / steps)
    achieved = nbytes / (ms * 1e-3) / 1e9
    step_ms = total_ms / steps
    return {"entry": "kv_write", "tokens": T, "num_kv_heads": H, "kv_dtype": inp.kv_dtype,
            "page_size": inp.page_size, "ms_per_step": round(step_ms, 5),
            "gbs": round(nbytes / (step_ms * 1e-3) / 1e9, 1), "layers": layers,
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": None, "kernel": "kv_write_kernel", "kernel_ms": round(ms, 5),
                         "kernel_ms_events": round(ms_raw, 5), "work_per_launch": nbytes}}


def measure_context_split(steps, warmup, events, parts=2, target_bytes=1 << 30):
    """One GPU's share of a context split of the batched-decode workload: the
    partial over the first of `parts` page-aligned key ranges of every
    sequence (through a block table holding only that range's pages), and the
    owner's combine of `parts` partials."""
    import numpy as np
    import torch
    from paged_asymmetric_head_amd import binding as B
    from paged_asymmetric_head_amd.device import DeviceInputs, _to_device
    from paged_asymmetric_head_amd.synth import workload

    inp = workload("batched_decode")
    dev = DeviceInputs(inp)
    P = inp.page_size
    lo = np.zeros(inp.batch, dtype=np.int32)
    hi = np.array([min(int(L), (-(-int(L) // P) // parts) * P) for L in inp.seq_lens], dtype=np.int32)
    bt = np.full_like(inp.block_table, -1)
    for b in range(inp.batch):
        bt[b, :(int(hi[b]) + P - 1) // P] = inp.block_table[b, :(int(hi[b]) + P - 1) // P]
    bt_d = _to_device(bt.astype(np.int32), "cuda")
    lo_d, hi_d = _to_device(lo, "cuda"), _to_device(hi, "cuda")
    pool = dev.k_cache.numel() * dev.k_cache.element_size() + dev.v_cache.numel() * dev.v_cache.element_size()
    layers = max(1, min(16, math.ceil(target_bytes / pool)))
    caches = [(dev.k_cache, dev.v_cache)] + [(dev.k_cache.clone(), dev.v_cache.clone())
                                             for _ in range(layers - 1)]
    rows = inp.total_q * inp.num_q_heads
    out_parts = torch.zeros((parts, rows, 128), dtype=torch.float32, device="cuda")
    lse_parts = torch.zeros((parts, rows), dtype=torch.float32, device="cuda")
    d = dev.desc("verify")
    ws, nbytes = dev.workspace_for("verify")
    stream = torch.cuda.current_stream().cuda_stream
    calls = [B.prepared_partial(d, dev.q, k, v, bt_d, dev.seq_lens, dev.q_lens, lo_d, hi_d,
                                inp.window, inp.k_scale, inp.v_scale, inp.softmax_scale,
                                out_parts[0], lse_parts[0], None, ws, nbytes, stream)
             for k, v in caches]
    total_ms, _, kern, _ = time_calls(calls, steps, warmup, events, stream)
    out = torch.empty((rows, 128), dtype=torch.bfloat16, device="cuda")
    comb = [B.prepared_combine(parts, rows, inp.num_q_heads, out_parts, lse_parts, dev.sinks, out,
                               None, stream)]
    c_total, _, c_kern, _ = time_calls(comb, steps, warmup, events, stream)
    kv_bytes = (int(hi.astype(np.int64).sum() - lo.sum()) * inp.num_kv_heads
                * (inp.q.shape[2] + inp.v_cache.shape[3]) * 2)
    ms, ms_raw = kernel_ms_bounded(kern, total_ms / steps)
    achieved = kv_bytes / (ms * 1e-3) / 1e9
    return {"entry": "partial+combine", "workload": "batched_decode", "parts": parts,
            "partial_ms_per_step": round(total_ms / steps, 5),
            "combine_ms_per_step": round(c_total / steps, 5),
            "combine_kernel_ms": round(kernel_ms_bounded(c_kern, c_total / steps)[0], 5),
            "layers": layers,
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                         "kernel": "split_attn_kernel (context partial)", "kernel_ms": round(ms, 5),
                         "kernel_ms_events": round(ms_raw, 5), "work_per_launch": kv_bytes}}


# Launch shapes tried for the streaming-read reference: (workgroups, loads
# in flight per thread).
STREAM_SHAPES = [(b, u) for b in (512, 1024, 2048, 4096, 8192) for u in (4, 8)]

# Decode context sweep: the batched-decode shape (32 sequences, Hq 8 / Hkv 1,
# QK 192 / V 128, page 128, bf16) at these lower bounds of the context range
# [L, 9L/8], to fit time = a + bytes / B over context length.
SWEEP_CONTEXTS = (2048, 8192, 16384, 32768, 65536)


def _random_paged_call(lens, q_len, rng, gen, stream, target_bytes, shuffle=True):
    """Prepared C-ABI calls (decode for q_len 1, verify otherwise) over random
    bf16 K/V drawn on the device, Hq 8 / Hkv 1, QK 192 / V 128, page 128, the
    pages in a random permutation, replicated into enough copies to pass
    target_bytes; returns (calls, output tensor, KV bytes of the visible keys)."""
    import numpy as np
    import torch
    from paged_asymmetric_head_amd import binding as B
    hq, hkv, dqk, dv, P = 8, 1, 192, 128, 128
    batch = len(lens)
    pages = (lens + P - 1) // P
    num_pages = int(pages.sum())
    stride = int(-(-int(lens.max()) // P))
    perm = (rng.permutation(num_pages) if shuffle else np.arange(num_pages)).astype(np.int32)
    bt = np.full((batch, stride), -1, dtype=np.int32)
    off = 0
    for b in range(batch):
        bt[b, :pages[b]] = perm[off:off + pages[b]]
        off += int(pages[b])
    pool = num_pages * P * hkv * (dqk + dv) * 2
    layers = max(1, min(16, math.ceil(target_bytes / pool)))
    caches = [(torch.randn((num_pages, P, hkv, dqk), generator=gen, device="cuda").to(torch.bfloat16),
               torch.randn((num_pages, P, hkv, dv), generator=gen, device="cuda").to(torch.bfloat16))
              for _ in range(layers)]
    total_q = batch * q_len
    q = torch.randn((total_q, hq, dqk), generator=gen, device="cuda").to(torch.bfloat16)
    bt_d = torch.from_numpy(bt).cuda()
    lens_d = torch.from_numpy(lens).cuda()
    qlens_d = torch.full((batch,), q_len, dtype=torch.int32, device="cuda")
    out = torch.empty((total_q, hq, dv), dtype=torch.bfloat16, device="cuda")
    entry = "decode" if q_len == 1 else "verify"
    d = B.AttnDesc(batch=batch, num_q_heads=hq, num_kv_heads=hkv, head_dim_qk=dqk, head_dim_v=dv,
                   page_size=P, num_pages=num_pages, block_table_stride=stride,
                   max_seq_len=int(lens.max()), max_q_len=q_len, total_q=total_q, kv_dtype=B.KV_BF16,
                   force_num_splits=0)
    nbytes = B.diffkv_attn_workspace_bytes(d, B.ENTRIES[entry])
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    calls = [B.prepared_call(f"diffkv_attn_{entry}", d, q, k, v, bt_d, lens_d, qlens_d, 0, None, 1.0, 1.0,
                             1.0 / math.sqrt(dqk), out, None, None, ws, nbytes, stream)
             for k, v in caches]
    kv_bytes = int(lens.astype(np.int64).sum()) * hkv * (dqk + dv) * 2
    return calls, out, kv_bytes, layers


def _sweep_point(calls, out, kv_bytes, layers, steps, warmup, events, stream, label):
    import torch
    total_ms, _, kern, _ = time_calls(calls, steps, warmup, events, stream)
    if not bool(torch.isfinite(out.float()).all()):
        raise RuntimeError(f"{label}: non-finite output")
    ms = kernel_ms_bounded(kern, total_ms / steps)[0]
    return {"kv_bytes": kv_bytes, "kernel_ms": round(ms, 5), "step_ms": round(total_ms / steps, 5),
            "kernel_gbs": round(kv_bytes / (ms * 1e-3) / 1e9, 1),
            "frac": round(kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "layers": layers}


# Verify batch sweep: the long-verify shape (8-token blocks, contexts uniform
# in [40000, 50000], Hq 8 / Hkv 1, page 128, bf16) at these batch sizes.
VERIFY_SWEEP_BATCHES = (4, 8, 16, 32)


def measure_verify_sweep(steps, warmup, events, batches=VERIFY_SWEEP_BATCHES, target_bytes=1 << 30):
    """The verify kernel over batch sizes at 40K-50K tokens, for timing only
    (random bf16 K/V drawn on the device): where the start cost of one launch
    is spread over more bytes."""
    import numpy as np
    import torch
    rng = np.random.default_rng(12)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(12)
    stream = torch.cuda.current_stream().cuda_stream
    rows = []
    for batch in batches:
        lens = rng.integers(40000, 50001, size=batch).astype(np.int32)
        calls, out, kv_bytes, layers = _random_paged_call(lens, 8, rng, gen, stream, target_bytes)
        row = _sweep_point(calls, out, kv_bytes, layers, steps, warmup, events, stream, f"verify batch {batch}")
        rows.append({"batch": batch, **row})
        del calls, out
        torch.cuda.empty_cache()
    return {"shape": "q_len 8 (causal in the block), contexts uniform in [40000, 50000], Hq 8 / Hkv 1, "
                     "QK 192 / V 128, page 128, bf16",
            "data": "random bf16 K/V drawn on the device (timing only)", "points": rows}


def measure_decode_sweep(steps, warmup, events, contexts=SWEEP_CONTEXTS, target_bytes=1 << 30,
                         shuffle=True):
    """The decode kernel over context lengths, for timing only: K/V are random
    bf16 values drawn on the device (no parity check here; the seeded
    workloads are checked by the tests), pages in a random permutation, the
    same launch path and cold-cache rotation as the other workloads.  Returns
    per-context kernel times and the least-squares fit of kernel time =
    a + bytes / B."""
    import numpy as np
    import torch
    rng = np.random.default_rng(11)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    stream = torch.cuda.current_stream().cuda_stream
    rows = []
    for L0 in contexts:
        lens = rng.integers(L0, L0 + L0 // 8 + 1, size=32).astype(np.int32)
        calls, out, kv_bytes, layers = _random_paged_call(lens, 1, rng, gen, stream, target_bytes, shuffle)
        row = _sweep_point(calls, out, kv_bytes, layers, steps, warmup, events, stream, f"decode sweep at {L0}")
        rows.append({"context_lo": int(L0), **row})
        del calls, out
        torch.cuda.empty_cache()
    x = np.array([r["kv_bytes"] for r in rows], dtype=np.float64)
    y = np.array([r["kernel_ms"] * 1e-3 for r in rows], dtype=np.float64)
    slope, icept = np.polyfit(x, y, 1)
    # The streaming-read reference at the longest context's byte count.
    ref = stream_read_reference(rows[-1]["kv_bytes"], steps, events)
    ref["kernel_frac_of_stream"] = round(rows[-1]["kernel_gbs"] / ref["gbs"], 4)
    return {"shape": "batch 32, Hq 8 / Hkv 1, QK 192 / V 128, page 128, bf16, contexts uniform in [L, 9L/8]",
            "data": "random bf16 K/V drawn on the device (timing only)", "points": rows,
            "fit_kernel_ms": {"a_us": round(icept * 1e6, 2), "B_gbs": round(1.0 / slope / 1e9, 1)},
            "stream_read_longest": ref}



def stream_read_reference(nbytes, steps, events, target_bytes=1 << 30):
    """Achievable read bandwidth at one size: a plain grid-stride 16-byte read
    of `nbytes` (libdiffkv_stream.so), timed like the attention kernels (HIP
    events around each launch), cold in L2 and the Infinity Cache (copies
    walked in turn, more than 1 GiB in all); the fastest of a few launch
    shapes.  Context for the HBM fraction: what one launch of plain reads of
    that many bytes reaches on this GPU."""
    import torch
    path = os.path.join(ROOT, "paged_asymmetric_head_amd", "libdiffkv_stream.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    lib.diffkv_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_void_p]
    lib.diffkv_stream_read.restype = ctypes.c_int
    nbytes = nbytes // 16 * 16
    copies = max(2, math.ceil(target_bytes / nbytes) + 1)
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(i % 251) for i in range(copies)]
    sink = torch.empty(max(b for b, _ in STREAM_SHAPES) * 256, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    best = None
    for blocks, unroll in STREAM_SHAPES:
        def launch(k):
            st = lib.diffkv_stream_read(bufs[k % copies].data_ptr(), nbytes, sink.data_ptr(), blocks, unroll,
                                        stream)
            if st != 0:
                raise RuntimeError(f"diffkv_stream_read: status {st}")
        for k in range(5):
            launch(k)
        torch.cuda.synchronize()
        pairs = [(events.create(), events.create()) for _ in range(steps)]
        for k in range(steps):
            events.record(pairs[k][0], stream)
            launch(k)
            events.record(pairs[k][1], stream)
        torch.cuda.synchronize()
        ms = sum(events.elapsed_ms(a, b) for a, b in pairs) / steps
        if best is None or ms < best[2]:
            best = (blocks, unroll, ms)
    del bufs, sink
    torch.cuda.empty_cache()
    blocks, unroll, ms = best
    return {"bytes": nbytes, "kernel_ms": round(ms, 5), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "blocks": blocks, "loads_per_thread": unroll,
            "kernel": "stream_read_kernel (libdiffkv_stream.so)"}


def with_stream_reference(roof, steps, events):
    """Adds the streaming-read reference at the kernel's own byte count to an
    HBM-bound roofline record, and the kernel's fraction of it."""
    ref = stream_read_reference(roof["work_per_launch"], steps, events)
    ref["kernel_frac_of_stream"] = round(roof["achieved"] / ref["gbs"], 4)
    roof["stream_read"] = ref
    return roof


COPY_BYTES = 256 << 20


def copy_calibration():
    """A plain elementwise copy of known size: reads and writes COPY_BYTES."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()


def _counter_means(path, counter):
    """Mean per-dispatch value of one counter, by kernel name (rocprofv3 CSV)."""
    import csv
    import collections
    per = collections.defaultdict(float)
    names = {}
    for row in csv.DictReader(open(path)):
        if row["Counter_Name"] != counter:
            continue
        per[row["Dispatch_Id"]] += float(row["Counter_Value"])
        names[row["Dispatch_Id"]] = row["Kernel_Name"]
    by_kernel = collections.defaultdict(list)
    for d, v in per.items():
        by_kernel[names[d]].append(v)
    return {k: sum(v) / len(v) for k, v in by_kernel.items()}


def write_traffic(workload, fetch_csv, write_csv):
    """HBM bytes per launch of the main kernel from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by what the counter reads for the
    calibration copy (COPY_BYTES read and written)."""
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")
    kern = KERNEL_OF_ENTRY[ENTRY_OF[workload]]

    def pick(d, key):
        hits = [v for k, v in d.items() if key in k]
        if not hits:
            raise SystemExit(f"no dispatch of {key} in the counter file")
        return max(hits)

    copy_key = "AUnaryFunctor<float, float, float"   # torch.mul(src, 1.0, out=dst)
    f_factor = COPY_BYTES / (pick(fetch, copy_key) * 1024.0)
    w_factor = COPY_BYTES / (pick(write, copy_key) * 1024.0)
    rec = {"kernel": kern, "source_sha": kernel_source_sha(),
           "fetch_kib_raw": pick(fetch, kern), "write_kib_raw": pick(write, kern),
           "copy_fetch_factor": f_factor, "copy_write_factor": w_factor}
    rec["bytes_per_launch"] = int(rec["fetch_kib_raw"] * 1024 * f_factor + rec["write_kib_raw"] * 1024 * w_factor)
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    data[workload] = rec
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    print(json.dumps({workload: rec}))


MIXED_SPLIT_MAX_Q = 16     # mixed calls: q_len <= 16 on the split kernels, longer on prefill


def roofline(m, sha, name):
    w = m["work"]
    ms = m["kernel_ms_mean"]
    traffic = measured_traffic(name, sha)
    if m["entry"] == "mixed":
        # Two kernels in sequence: the time each part needs at its own bound
        # (KV bytes of the short sequences at HBM peak, flops of the long ones
        # at bf16 MFMA peak), summed, against the measured step.
        ws = algorithmic_work(m["inp"], q_hi=MIXED_SPLIT_MAX_Q)
        wp = algorithmic_work(m["inp"], q_lo=MIXED_SPLIT_MAX_Q + 1)
        bound_ms = 1e3 * (ws["kv_bytes"] / (HBM_PEAK_GBS * 1e9) + wp["flops"] / (BF16_PEAK_TFLOPS * 1e12))
        return {"bound": "hbm+mfma", "bound_ms": round(bound_ms, 5), "step_ms": round(m["ms_per_step"], 5),
                "frac": round(bound_ms / m["ms_per_step"], 4), "traffic": None,
                "kernel": KERNEL_OF_ENTRY["mixed"], "split_part_kv_bytes": ws["kv_bytes"],
                "prefill_part_flops": wp["flops"],
                "split_kernel_ms": round(ms, 5)}
    if m["entry"] == "prefill":
        achieved = w["flops"] / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                "traffic": traffic, "kernel": KERNEL_OF_ENTRY[m["entry"]],
                "kernel_ms": round(ms, 5), "kernel_ms_median": round(m["kernel_ms_median"], 5),
                "kernel_ms_events": round(m["kernel_ms_events"], 5), "work_per_launch": w["flops"]}
    achieved = w["kv_bytes"] / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": KERNEL_OF_ENTRY[m["entry"]], "kernel_ms": round(ms, 5),
            "kernel_ms_median": round(m["kernel_ms_median"], 5),
            "kernel_ms_events": round(m["kernel_ms_events"], 5), "work_per_launch": w["kv_bytes"]}


def summary(m, sha, name):
    w = m["work"]
    s = m["ms_per_step"] * 1e-3
    res = {"entry": m["entry"], "ms_per_step": round(m["ms_per_step"], 5),
           "kv_gbs": round(w["kv_bytes"] / s / 1e9, 1),
           "tflops": round(w["flops"] / s / 1e12, 2),
           "q_ctx_tokens_per_s": w["q_ctx"] / s, "splits": m["splits"], "layers": m["layers"],
           "roofline": roofline(m, sha, name)}
    return res


def _oracle_items(inp, entry):
    """The workload cut into oracle items: every sequence with at most 16 new
    tokens is one item (its tokens share one key range), longer ones are cut
    into 8-token groups.  Each item is (packed rows, KV bytes of the union of
    their visible keys, flops of their visible (row, key) pairs)."""
    import numpy as np
    esize = 1 if inp.kv_dtype == "fp8" else 2
    row_bytes = inp.num_kv_heads * (inp.q.shape[2] + inp.v_cache.shape[3]) * esize
    starts = np.concatenate([[0], np.cumsum(inp.q_lens)[:-1]])
    items = []
    for b in range(inp.batch):
        L, n = int(inp.seq_lens[b]), int(inp.q_lens[b])
        step = n if n <= 16 else 8
        for c0 in range(0, n, step):
            i = np.arange(c0, min(n, c0 + step))
            p = L - n + i
            lo = np.maximum(0, p - inp.window + 1) if inp.window > 0 else np.zeros_like(p)
            kv = int(p.max() + 1 - lo.min()) * row_bytes
            flops = 2 * (inp.q.shape[2] + inp.v_cache.shape[3]) * int((p - lo + 1).sum()) * inp.num_q_heads
            items.append((starts[b] + i, kv, flops))
    return items


def cpu_baseline(name, seconds):
    """The FP64 oracle on the host: the workload's items (see _oracle_items)
    in a fixed random order, one per thread on every core of the affinity set
    (BLAS held to one thread each), in rounds of one item per core until about
    `seconds` have passed; the rate is the sampled items' algorithmic work
    (KV bytes, or flops for the prefill and mixed workloads) over the time."""
    from concurrent.futures import ThreadPoolExecutor
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import paged_attention
    from oracle.parallel import host_cores
    from paged_asymmetric_head_amd.synth import workload

    inp = workload(name)
    entry = ENTRY_OF[name]
    args = inp.oracle_kwargs()
    items = _oracle_items(inp, entry)
    order = np.random.default_rng(0).permutation(len(items))
    cores = host_cores()
    done_kv = done_flops = n_items = n_tok = 0
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(max_workers=cores) as ex:
        t0 = time.perf_counter()
        k = 0
        while time.perf_counter() - t0 < seconds:
            rnd = [items[order[(k + j) % len(items)]] for j in range(cores)]
            list(ex.map(lambda it: paged_attention(**args, tokens=it[0]), rnd))
            for toks, kv, fl in rnd:
                done_kv += kv
                done_flops += fl
                n_tok += len(toks)
            n_items += len(rnd)
            k += cores
        dt = time.perf_counter() - t0
    if entry in ("prefill", "mixed"):
        val, unit = done_flops / dt / 1e12, "TFLOP/s"
    else:
        val, unit = done_kv / dt / 1e9, "GB/s"
    return {"value": round(val, 6), "unit": unit, "cores": cores, "kind": "oracle",
            "sample": f"{name}: {n_items} items ({n_tok} query tokens; an item is a sequence of up to "
                      f"16 new tokens or 8 tokens of a longer one; the workload has {len(items)}), all "
                      f"heads, in {dt:.1f} s: FP64 NumPy oracle, one thread per core on {cores} cores, "
                      f"BLAS threads 1 each"}


def main():
    args = parse_args()
    if args.traffic_from:
        write_traffic(args.workload, *args.traffic_from)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this attention path has no cross-GPU step; "
              "run it with --gpus 1 (see the sharding design notes).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    from paged_asymmetric_head_amd import binding as B
    B.load_library()
    sha = kernel_source_sha()
    events = HipEvents()

    name = args.workload
    if name not in ENTRY_OF:
        print(f"[bench] {name}: generating and measuring", file=sys.stderr, flush=True)
        res = (measure_kv_write(name, args.steps, args.warmup, events) if name in KV_WRITE_OF
               else measure_decode_sweep(args.steps, args.warmup, events) if name == "decode_sweep"
               else measure_verify_sweep(args.steps, args.warmup, events) if name == "verify_sweep"
               else measure_context_split(args.steps, args.warmup, events))
        print(json.dumps({"workload": name, "steps": args.steps, "warmup": args.warmup,
                          "kernel_source_sha": sha, **res}), flush=True)
        return
    print(f"[bench] {name}: generating and measuring", file=sys.stderr, flush=True)
    m = measure(name, args.steps, args.warmup, events,
                warm_ms=0.0 if name == HEADLINE else EXTRA_WARM_MS)
    head = summary(m, sha, name)
    inp = m["inp"]
    is_prefill = m["entry"] == "prefill"
    value = head["tflops"] if is_prefill else head["kv_gbs"]
    result = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s" if is_prefill else "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, "entry": m["entry"], "batch": inp.batch,
                   "q_len": int(inp.q_lens.max()), "context_max": int(inp.max_seq_len),
                   "num_q_heads": inp.num_q_heads, "num_kv_heads": inp.num_kv_heads,
                   "head_dim_qk": 192, "head_dim_v": 128, "page_size": inp.page_size,
                   "kv_dtype": inp.kv_dtype, "window": inp.window,
                   "sinks": inp.sinks is not None, "splits": m["splits"], "kv_copies": m["layers"],
                   "kv_bytes_per_step": m["work"]["kv_bytes"]},
        "q_ctx_tokens_per_s": head["q_ctx_tokens_per_s"],
        "wall_ms_per_step": round(m["wall_ms_per_step"], 5),
        "roofline": head["roofline"],
        "kernel_source_sha": sha,
    }
    del m
    if head["roofline"]["bound"] == "hbm":
        print(f"[bench] {name}: streaming-read reference", file=sys.stderr, flush=True)
        with_stream_reference(result["roofline"], args.steps, events)
    if not args.no_extra:
        extra = {}
        for other in ("verify_long", "swa_sinks_fp8_p1", "swa_sinks_fp8_p128", "chunked_prefill",
                      "mixed_batch", "batched_decode_sym"):
            if other == name:
                continue
            print(f"[bench] {other}: generating and measuring", file=sys.stderr, flush=True)
            mo = measure(other, args.extra_steps, 5, events, warm_ms=EXTRA_WARM_MS)
            extra[other] = summary(mo, sha, other)
            if not args.no_cpu_baseline:
                print(f"[bench] {other}: timing the CPU oracle", file=sys.stderr, flush=True)
                extra[other]["cpu_baseline"] = cpu_baseline(other, args.cpu_seconds_extra)
            if other == "verify_long":
                with_stream_reference(extra[other]["roofline"], args.extra_steps, events)
            del mo
            torch.cuda.empty_cache()
        for other in KV_WRITE_OF:
            print(f"[bench] {other}: generating and measuring", file=sys.stderr, flush=True)
            extra[other] = measure_kv_write(other, args.extra_steps, 5, events)
            torch.cuda.empty_cache()
        print("[bench] context_split_decode: generating and measuring", file=sys.stderr, flush=True)
        extra["context_split_decode"] = measure_context_split(args.extra_steps, 5, events)
        torch.cuda.empty_cache()
        print("[bench] decode_sweep: generating and measuring", file=sys.stderr, flush=True)
        extra["decode_sweep"] = measure_decode_sweep(args.extra_steps, 5, events)
        torch.cuda.empty_cache()
        print("[bench] verify_sweep: generating and measuring", file=sys.stderr, flush=True)
        extra["verify_sweep"] = measure_verify_sweep(args.extra_steps, 5, events)
        torch.cuda.empty_cache()
        result["extra"] = extra
    if args.copy_calibration:
        copy_calibration()
    if not args.no_cpu_baseline:
        print(f"[bench] {name}: timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(name, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
