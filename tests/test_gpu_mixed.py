"""GPU parity of mixed batches (diffkv_attn_mixed): decode, verify and prefill
sequences in one call, against the FP64 oracle and against the single-kind
entries.  Sequences with q_len <= 16 take the split-KV kernels, longer ones
the prefill kernel; the choice is made on the device from q_lens.
"""

import numpy as np
import pytest
import torch

from paged_asymmetric_head_amd import binding as B
from paged_asymmetric_head_amd.device import DeviceInputs
from paged_asymmetric_head_amd.synth import make_paged_inputs, workload
from parity import compare, to_np
from test_gpu_parity import check_call, oracle, say

pytestmark = pytest.mark.gpu

MIXED = [
    # (page, seq_lens, q_lens, Hq, Hkv, window, sinks, kv)
    (16, [300, 40, 700, 17, 90], [1, 17, 64, 16, 5], 8, 1, 0, True, "bf16"),
    (1, [100, 260, 33], [33, 1, 8], 4, 2, 0, False, "fp8"),
    (128, [1000, 200, 129, 5000], [300, 1, 129, 16], 16, 1, 128, True, "fp8"),
    (64, [520, 64, 90], [200, 2, 90], 8, 2, 40, False, "bf16"),
    (32, [33, 34], [17, 16], 6, 3, 0, True, "fp8"),
]


def mixed_inputs(i, extra_pages=3):
    P, L, n, Hq, Hkv, W, sinks, kv = MIXED[i]
    return make_paged_inputs(300 + i, seq_lens=L, q_lens=n, num_q_heads=Hq, num_kv_heads=Hkv,
                             page_size=P, kv_dtype=kv, window=W, sinks=sinks,
                             extra_pages=extra_pages, write_align=P if W > 0 else None)


@pytest.mark.parametrize("i", range(len(MIXED)), ids=[f"m{i}" for i in range(len(MIXED))])
def test_mixed_parity(i):
    dev = DeviceInputs(mixed_inputs(i))
    check_call(dev, "mixed", f"m{i}")


@pytest.mark.parametrize("splits", [1, 3, 20])
def test_mixed_forced_splits(splits):
    dev = DeviceInputs(mixed_inputs(0))
    check_call(dev, "mixed", f"m0 splits={splits}", force_num_splits=splits)


def test_mixed_matches_single_entries_bitwise():
    """A batch of short sequences through mixed is the verify call; a batch of
    long ones is the prefill call; in a mixed batch, the long sequences' rows
    equal the prefill call's rows on the same inputs (their workgroups do not
    depend on the other sequences)."""
    short = make_paged_inputs(320, seq_lens=[900, 64, 300], q_lens=[8, 16, 1], num_q_heads=8,
                              num_kv_heads=1, page_size=16, kv_dtype="fp8", sinks=True)
    dev = DeviceInputs(short)
    say("mixed vs verify (all short)")
    a, _, _ = dev.run("mixed")
    b, _, _ = dev.run("verify")
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    long_ = make_paged_inputs(321, seq_lens=[900, 400], q_lens=[100, 17], num_q_heads=8,
                              num_kv_heads=1, page_size=16, kv_dtype="bf16", window=64)
    dev = DeviceInputs(long_)
    say("mixed vs prefill (all long)")
    a, _, _ = dev.run("mixed")
    b, _, _ = dev.run("prefill")
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    inp = mixed_inputs(0)
    dev = DeviceInputs(inp)
    say("mixed vs prefill on the long rows")
    a, _, _ = dev.run("mixed")
    b, _, _ = dev.run("prefill")
    torch.cuda.synchronize()
    r0 = np.concatenate([[0], np.cumsum(inp.q_lens)])
    for s in range(inp.batch):
        if inp.q_lens[s] > 16:
            assert torch.equal(a[r0[s]:r0[s + 1]], b[r0[s]:r0[s + 1]]), s


def test_mixed_batch_workload():
    """The full-size mixed step (a 4096-token chunk at 26K context, 4 verify
    blocks at 40K-50K, 32 decodes at 8K-9K; GQA 32/2, FP8, page 128): every
    row of the output against the oracle."""
    inp = workload("mixed_batch")
    dev = DeviceInputs(inp)
    check_call(dev, "mixed", "mixed_batch")


def test_mixed_graph_replay_reroutes_sequences():
    """One mixed call captured in a HIP graph, replayed after q_lens, seq_lens
    and block tables change in place so that sequences move between the
    split-KV and prefill kernels; every replay must match the oracle."""
    cfg = dict(num_q_heads=8, num_kv_heads=1, page_size=16, kv_dtype="bf16", sinks=True,
               max_seq_len=1200)
    q_sets = [[20, 4, 8], [4, 20, 8], [30, 1, 1], [1, 1, 30], [10, 11, 11]]
    base = make_paged_inputs(330, seq_lens=[900, 1100, 64], q_lens=q_sets[0], extra_pages=300,
                             **cfg)
    dev = DeviceInputs(base)
    d = dev.desc("mixed")
    d.max_q_len = 40
    ws_bytes = B.diffkv_attn_workspace_bytes(d, B.ENTRY_MIXED)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty((base.total_q, 8, 128), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.diffkv_attn_mixed(d, dev.q, dev.k_cache, dev.v_cache, dev.block_table, dev.seq_lens,
                            dev.q_lens, base.window, dev.sinks, base.k_scale, base.v_scale,
                            base.softmax_scale, out, None, None, ws, ws_bytes)
    rng = np.random.default_rng(7)
    for rep, ql in enumerate(q_sets[1:]):
        lens = [int(max(q, x)) for q, x in zip(ql, rng.integers(1, 1200, size=3))]
        inp = make_paged_inputs(340 + rep, seq_lens=lens, q_lens=ql,
                                extra_pages=base.num_pages - sum(-(-x // 16) for x in lens), **cfg)
        assert inp.num_pages == base.num_pages and inp.total_q == base.total_q
        inp.sinks = base.sinks
        dev.q.copy_(torch.from_numpy(inp.q.view(np.int16)))
        dev.k_cache.copy_(torch.from_numpy(inp.k_cache.view(np.int16)))
        dev.v_cache.copy_(torch.from_numpy(inp.v_cache.view(np.int16)))
        dev.block_table.copy_(torch.from_numpy(inp.block_table))
        dev.seq_lens.copy_(torch.from_numpy(inp.seq_lens))
        dev.q_lens.copy_(torch.from_numpy(inp.q_lens))
        torch.cuda.synchronize()
        say(f"mixed graph replay {rep}: q_lens={ql} seq_lens={lens}")
        g.replay()
        torch.cuda.synchronize()
        compare(to_np(out), oracle(inp).out, f"mixed graph replay {rep}")
        _ = (dev.q.float() * 2).sum().item()     # eager work between replays
