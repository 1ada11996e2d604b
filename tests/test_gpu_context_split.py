"""GPU parity of the context split: diffkv_attn_partial (one key range's share
of every row, fp32, no sink) against the oracle's attention_partial, and
partials of a partition of every sequence's keys merged by diffkv_attn_combine
against the unsplit oracle.  Each part reads through a block table of its own
in which the pages outside its range are -1, as on a GPU that holds only its
share of the sequence.
"""

import numpy as np
import pytest
import torch

from oracle import attention_partial, paged_attention
from paged_asymmetric_head_amd import binding as B
from paged_asymmetric_head_amd.device import DeviceInputs, _to_device
from paged_asymmetric_head_amd.synth import make_paged_inputs, workload
from parity import compare, to_np
from test_gpu_parity import LSE_ATOL, say

pytestmark = pytest.mark.gpu


def part_table(inp, lo, hi):
    """Block table with only the pages holding keys in [lo[b], hi[b]) kept."""
    bt = np.full_like(inp.block_table, -1)
    P = inp.page_size
    for b in range(inp.batch):
        if hi[b] > lo[b]:
            t0, t1 = lo[b] // P, (hi[b] - 1) // P + 1
            bt[b, t0:t1] = inp.block_table[b, t0:t1]
    return bt


def run_partial(dev, lo, hi, force_num_splits=0, count=False):
    inp = dev.inp
    d = dev.desc("verify", force_num_splits)
    ws, nbytes = dev.workspace_for("verify", force_num_splits)
    out = torch.empty((inp.total_q, inp.num_q_heads, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((inp.total_q, inp.num_q_heads), dtype=torch.float32, device="cuda")
    cnt = torch.empty((inp.total_q, inp.num_q_heads), dtype=torch.int32, device="cuda") if count else None
    bt = _to_device(part_table(inp, lo, hi).astype(np.int32), "cuda")
    B.diffkv_attn_partial(d, dev.q, dev.k_cache, dev.v_cache, bt, dev.seq_lens, dev.q_lens,
                          _to_device(np.asarray(lo, dtype=np.int32), "cuda"),
                          _to_device(np.asarray(hi, dtype=np.int32), "cuda"), inp.window,
                          inp.k_scale, inp.v_scale, inp.softmax_scale, out, lse, cnt, ws, nbytes)
    return out, lse, cnt


def oracle_partial(inp, lo, hi):
    a = inp.oracle_kwargs()
    a.pop("sinks")
    return attention_partial(**a, key_lo=lo, key_hi=hi)


def check_partial(dev, lo, hi, tag, **kw):
    inp = dev.inp
    say(f"{tag}: partial batch={inp.batch} P={inp.page_size} kv={inp.kv_dtype} lo={list(lo)} hi={list(hi)}")
    out, lse, cnt = run_partial(dev, lo, hi, count=True, **kw)
    torch.cuda.synchronize()
    ref = oracle_partial(inp, lo, hi)
    got_lse = lse.cpu().numpy().astype(np.float64)
    empty = ref.count == 0
    assert np.array_equal(cnt.cpu().numpy(), ref.count), f"{tag}: count"
    assert np.all(np.isneginf(got_lse[empty])), f"{tag}: empty rows need lse -inf"
    assert np.all(out.cpu().numpy()[empty] == 0.0), f"{tag}: empty rows need 0"
    np.testing.assert_allclose(got_lse[~empty], ref.lse[~empty], rtol=0, atol=LSE_ATOL)
    if (~empty).any():
        compare(out.cpu().numpy().astype(np.float64)[~empty], ref.out[~empty], tag)
    return out, lse


CASES = [
    # page, seq_lens, q_lens, Hq, Hkv, window, kv
    (16, [300, 40, 700, 17], [1, 8, 4, 16], 8, 1, 0, "bf16"),
    (1, [100, 260, 33], [3, 1, 8], 4, 2, 0, "fp8"),
    (128, [1000, 200, 5000], [4, 1, 8], 16, 1, 128, "fp8"),
    (64, [520, 64, 90], [2, 2, 9], 8, 2, 40, "bf16"),
]


@pytest.mark.parametrize("i", range(len(CASES)), ids=[f"c{i}" for i in range(len(CASES))])
def test_partial_parity(i):
    P, L, n, Hq, Hkv, W, kv = CASES[i]
    inp = make_paged_inputs(500 + i, seq_lens=L, q_lens=n, num_q_heads=Hq, num_kv_heads=Hkv,
                            page_size=P, kv_dtype=kv, window=W, extra_pages=3,
                            write_align=P if W > 0 else None)
    dev = DeviceInputs(inp)
    rng = np.random.default_rng(510 + i)
    first = [max(0, l - qn - W + 1) if W > 0 else 0 for l, qn in zip(L, n)]
    for rep in range(3):
        lo = [int(rng.integers(f, l)) for f, l in zip(first, L)]
        hi = [int(rng.integers(a + 1, l + 1)) for a, l in zip(lo, L)]
        if rep == 2:                     # empty ranges and single keys
            hi = [a if s % 2 == 0 else a + 1 for s, a in enumerate(lo)]
        check_partial(dev, lo, hi, f"c{i}/r{rep}")


@pytest.mark.parametrize("splits", [3, 20])
def test_partial_forced_splits(splits):
    inp = make_paged_inputs(520, seq_lens=[3000, 1777, 90], q_lens=[8, 5, 3], num_q_heads=8,
                            num_kv_heads=1, page_size=16, kv_dtype="bf16")
    check_partial(DeviceInputs(inp), [100, 0, 50], [2900, 1000, 51], f"partial splits={splits}",
                  force_num_splits=splits)


def combine_parts(dev, cuts):
    """Partials for the ranges cuts[s] .. cuts[s+1] of every sequence, merged."""
    inp = dev.inp
    outs, lses = [], []
    for s in range(len(cuts[0]) - 1):
        lo = [c[s] for c in cuts]
        hi = [c[s + 1] for c in cuts]
        o, l, _ = run_partial(dev, lo, hi)
        outs.append(o)
        lses.append(l)
    S = len(outs)
    rows = inp.total_q * inp.num_q_heads
    out_parts = torch.stack(outs).contiguous()
    lse_parts = torch.stack(lses).contiguous()
    out = torch.empty((inp.total_q, inp.num_q_heads, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((inp.total_q, inp.num_q_heads), dtype=torch.float32, device="cuda")
    B.diffkv_attn_combine(S, rows, inp.num_q_heads, out_parts, lse_parts, dev.sinks, out, lse)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("P,kv,W", [(16, "bf16", 0), (1, "fp8", 0), (128, "fp8", 0), (8, "bf16", 20)])
def test_partition_and_combine_equals_attention(P, kv, W):
    L = [300, 129, 64, 1000]
    inp = make_paged_inputs(530, seq_lens=L, q_lens=[4, 1, 8, 3], num_q_heads=8, num_kv_heads=2,
                            page_size=P, kv_dtype=kv, window=W, sinks=True, extra_pages=3,
                            write_align=P if W > 0 else None)
    dev = DeviceInputs(inp)
    cuts = [[0, 100, 100, 128, 300], [0, 1, 64, 129, 129], [0, 0, 32, 33, 64],
            [0, 250, 600, 999, 1000]]
    say(f"partition P={P} kv={kv} W={W}")
    out, lse = combine_parts(dev, cuts)
    ref = paged_attention(**inp.oracle_kwargs())
    compare(to_np(out), ref.out, f"partition P={P}")
    np.testing.assert_allclose(lse.cpu().numpy(), ref.lse, rtol=0, atol=LSE_ATOL)


@pytest.mark.parametrize("parts", [2, 4])
def test_batched_decode_split_across_parts(parts):
    """The batched-decode workload (32 x 8192..9216, page 128, bf16) with each
    sequence's keys cut into equal page-aligned parts, as across GPUs."""
    inp = workload("batched_decode")
    dev = DeviceInputs(inp)
    cuts = []
    for L in inp.seq_lens:
        pages = -(-int(L) // 128)
        edges = [min(int(L), (pages * s // parts) * 128) for s in range(parts)] + [int(L)]
        cuts.append(edges)
    say(f"batched_decode in {parts} parts")
    out, lse = combine_parts(dev, cuts)
    ref = paged_attention(**inp.oracle_kwargs())
    compare(to_np(out), ref.out, f"batched_decode/{parts}")
    np.testing.assert_allclose(lse.cpu().numpy(), ref.lse, rtol=0, atol=LSE_ATOL)
