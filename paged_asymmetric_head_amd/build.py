"""Builds libdiffkv_attn.so (the attention library), libdiffkv_attn_debug.so
(the same library with the device-side precondition checks compiled in,
-DDIFFKV_DEBUG), libdiffkv_attn_timeline.so (the same with per-workgroup
real-time stamps in the split-KV kernels, -DDIFFKV_TIMELINE) and
libdiffkv_stream.so (the streaming-read reference the benchmark quotes
beside HBM peak) in-tree with hipcc for gfx950.

    python -m paged_asymmetric_head_amd.build

Every run recompiles (no staleness check).  Packed-FP32 VALU forms are
switched off for the device pass.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUTPUT = os.path.join(HERE, "libdiffkv_attn.so")
DEBUG_OUTPUT = os.path.join(HERE, "libdiffkv_attn_debug.so")
TIMELINE_OUTPUT = os.path.join(HERE, "libdiffkv_attn_timeline.so")
SOURCES = [os.path.join(CSRC, "diffkv_attn.hip")]
STREAM_OUTPUT = os.path.join(HERE, "libdiffkv_stream.so")
STREAM_SOURCES = [os.path.join(CSRC, "stream_read.hip")]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def command(output=OUTPUT, extra=(), sources=SOURCES):
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}",
            *extra, "-o", output, *sources]


def _compile(output, sources, verbose, extra=()):
    tmp = output + ".tmp"
    cmd = command(tmp, extra=extra, sources=sources)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, output)


def build(verbose=False):
    """Compile the libraries; returns the attention library's path."""
    _compile(OUTPUT, SOURCES, verbose)
    _compile(DEBUG_OUTPUT, SOURCES, verbose, extra=("-DDIFFKV_DEBUG",))
    _compile(TIMELINE_OUTPUT, SOURCES, verbose, extra=("-DDIFFKV_TIMELINE",))
    _compile(STREAM_OUTPUT, STREAM_SOURCES, verbose)
    return OUTPUT


if __name__ == "__main__":
    print(build(verbose=True))
