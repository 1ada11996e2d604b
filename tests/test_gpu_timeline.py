"""The timeline build (libdiffkv_attn_timeline.so, -DDIFFKV_TIMELINE;
diffkv_attn_timeline_buffer): its split-KV kernels return the release
build's outputs bit for bit, and every workgroup that finishes a chunk
writes stamps in the order of the points it passes (balanced plan with a
merge, one-chunk launches through the tile loop and through the short-range
pass)."""

import numpy as np
import pytest
import torch

from paged_asymmetric_head_amd import binding as B
from paged_asymmetric_head_amd.device import DeviceInputs
from paged_asymmetric_head_amd.synth import make_paged_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # name, entry, forced splits, inputs
    ("planned decode", "decode", 0, dict(seq_lens=[3000, 4100, 900], q_lens=[1, 1, 1], num_q_heads=8,
                                         num_kv_heads=1, page_size=128, kv_dtype="bf16")),
    ("one-chunk verify", "verify", 1, dict(seq_lens=[700, 1300], q_lens=[8, 5], num_q_heads=8,
                                           num_kv_heads=1, page_size=16, kv_dtype="fp8")),
    ("short window", "verify", 0, dict(seq_lens=[5000, 9000, 700], q_lens=[4, 4, 4], num_q_heads=8,
                                       num_kv_heads=1, page_size=1, kv_dtype="fp8", window=128,
                                       sinks=True, write_align=1)),
]


def run(dev, entry, splits):
    call = dev.prepare(entry, force_num_splits=splits)
    call()
    torch.cuda.synchronize()
    return call.out.clone()


@pytest.mark.parametrize("i", range(len(CASES)), ids=[c[0].replace(" ", "_") for c in CASES])
def test_timeline_build_matches_release_and_orders_its_stamps(i):
    name, entry, splits, kw = CASES[i]
    print(f"[gpu] timeline build: {name}", flush=True)
    dev = DeviceInputs(make_paged_inputs(40 + i, **kw))
    want = run(dev, entry, splits)
    B.select_library("timeline")
    try:
        stamps = torch.zeros(8192 * 8, dtype=torch.int64, device="cuda")
        assert B.diffkv_attn_timeline_buffer(stamps) == B.OK
        got = run(dev, entry, splits)
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))
        s = stamps.view(-1, 8).cpu().numpy()
        rows = s[s[:, 7] > 0]
        assert len(rows) > 0
        for r in rows:
            seen = [int(x) for x in r if x != 0]
            assert seen == sorted(seen), r
            assert r[0] > 0 and r[1] >= r[0] and r[2] >= r[1] and r[3] >= r[2] and r[6] >= r[3], r
        # A buffer for one workgroup: the others skip their writes.
        small = torch.zeros(8, dtype=torch.int64, device="cuda")
        assert B.diffkv_attn_timeline_buffer(small) == B.OK
        assert torch.equal(run(dev, entry, splits).view(torch.int16), want.view(torch.int16))
        assert B.diffkv_attn_timeline_buffer(None) == B.OK
    finally:
        B.select_library("release")


def test_release_build_has_no_timeline():
    assert B.diffkv_attn_timeline_buffer(None) == B.UNSUPPORTED
