"""diffkv_attn_verify_noalloc (the verify entry on the library's static
per-device workspace, for callers that cannot allocate) against
diffkv_attn_verify on the same inputs, through the C ABI: bitwise the same
output, and within the tolerance of the FP64 oracle, on two calls in a row
(the second smaller, so stale partials of the first stay in the array)."""

import numpy as np
import pytest
import torch

from paged_asymmetric_head_amd import binding as B
from paged_asymmetric_head_amd.device import DeviceInputs
from paged_asymmetric_head_amd.synth import make_paged_inputs, workload
from parity import compare, to_np
from test_gpu_parity import oracle, say

pytestmark = pytest.mark.gpu


def noalloc(dev, lse=False):
    inp = dev.inp
    out = torch.empty((inp.total_q, inp.num_q_heads, 128), dtype=torch.bfloat16, device=dev.device)
    lse_t = torch.empty((inp.total_q, inp.num_q_heads), dtype=torch.float32,
                        device=dev.device) if lse else None
    B.diffkv_attn_verify_noalloc(dev.desc("verify"), dev.q, dev.k_cache, dev.v_cache, dev.block_table,
                                 dev.seq_lens, dev.q_lens, inp.window, dev.sinks, inp.k_scale,
                                 inp.v_scale, inp.softmax_scale, out, lse_t)
    return out, lse_t


def test_noalloc_matches_verify_on_two_calls():
    big = workload("verify_long")                         # 4 blocks of 8 at 40K-50K, split-KV
    small = make_paged_inputs(71, seq_lens=[3000, 1777, 90], q_lens=[8, 5, 3], num_q_heads=8,
                              num_kv_heads=1, page_size=16, kv_dtype="fp8", window=0, sinks=True)
    for tag, inp in (("verify_long", big), ("small", small)):
        dev = DeviceInputs(inp)
        d = dev.desc("verify")
        assert B.diffkv_attn_num_splits(d, B.ENTRY_VERIFY, inp.window) > 1   # uses the workspace
        say(f"noalloc {tag}: batch={inp.batch} total_q={inp.total_q}")
        got, got_lse = noalloc(dev, lse=True)
        ref, ref_lse, _ = dev.run("verify", lse=True)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), tag
        assert torch.equal(got_lse, ref_lse), tag
        compare(to_np(got), oracle(inp).out, f"noalloc {tag}")


def test_noalloc_rejects_a_workspace_beyond_the_array():
    d = B.AttnDesc(batch=4096, num_q_heads=32, num_kv_heads=2, head_dim_qk=192, head_dim_v=128,
                   page_size=128, num_pages=1, block_table_stride=400, max_seq_len=50000,
                   max_q_len=16, total_q=4096 * 16, kv_dtype=B.KV_FP8_E4M3, force_num_splits=0)
    with pytest.raises(B.DiffKVError, match="workspace"):
        B.diffkv_attn_verify_noalloc(d, 0, 0, 0, 0, 0, 0, 0, None, 1.0, 1.0, 1.0, 0)
