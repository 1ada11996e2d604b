"""GPU parity: the HIP path against the FP64 oracle on the same seeded inputs.

Every call goes through the C ABI (libdiffkv_attn.so via the ctypes binding).
"""

import numpy as np
import pytest
import torch

from oracle import paged_attention
from paged_asymmetric_head_amd.synth import make_paged_inputs, workload
from paged_asymmetric_head_amd.device import DeviceInputs
from parity import compare, expected_counts, to_np

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def oracle(inp, **kw):
    args = inp.oracle_kwargs()
    args.update(kw)
    return paged_attention(**args)


def check_call(dev, entry, tag, tokens=None, **kw):
    inp = dev.inp
    say(f"{tag}: {entry} batch={inp.batch} total_q={inp.total_q} P={inp.page_size} "
        f"kv={inp.kv_dtype} W={inp.window} sinks={inp.sinks is not None} {kw}")
    out, lse, cnt = dev.run(entry, lse=True, count=True, **kw)
    torch.cuda.synchronize()
    ref = oracle(inp, tokens=tokens)
    rows = ref.tokens
    compare(to_np(out)[rows], ref.out, tag)
    np.testing.assert_allclose(to_np(lse)[rows], ref.lse, rtol=0, atol=2e-3)
    c = cnt.cpu().numpy()
    assert np.array_equal(c[rows], ref.count), f"{tag}: count differs from the oracle"
    assert np.array_equal(c, expected_counts(inp)), f"{tag}: count differs from the mask size"
    return out


# --- the five workloads ---------------------------------------------------------

FULL = [("tiny_decode", "decode"), ("batched_decode", "decode"), ("verify_long", "verify"),
        ("swa_sinks_fp8_p1", "verify"), ("swa_sinks_fp8_p128", "verify")]


@pytest.mark.parametrize("name,entry", FULL, ids=[n for n, _ in FULL])
def test_workload_parity(name, entry):
    inp = workload(name)
    dev = DeviceInputs(inp)
    check_call(dev, entry, name)


def test_chunked_prefill_parity_sampled_rows():
    inp = workload("chunked_prefill")
    dev = DeviceInputs(inp)
    rng = np.random.default_rng(55)
    tokens = np.unique(np.concatenate([[0, 1, 15, 16, 63, 64, 2047, 2048, 4031, 4094, 4095],
                                       rng.integers(0, 4096, 21)]))
    check_call(dev, "prefill", "chunked_prefill", tokens=tokens)


# --- tiny grid through every entry that accepts it --------------------------------

GRID = [
    # (page, seq_lens, q_len, Hq, Hkv, window, sinks, kv)
    (1, [5, 9], 1, 2, 1, 0, False, "bf16"),
    (16, [16, 17, 15, 1], 1, 8, 2, 0, True, "fp8"),
    (2, [7, 3], 2, 4, 2, 0, True, "bf16"),
    (4, [10, 17, 4], 3, 4, 1, 5, False, "fp8"),
    (16, [33, 40], 8, 4, 1, 16, True, "bf16"),
    (2, [12, 30], 5, 2, 2, 1, False, "bf16"),
    (8, [9, 23], 4, 16, 1, 70, True, "fp8"),
    (16, [48, 70], 7, 4, 4, 9, False, "fp8"),
    (1, [20], 6, 1, 1, 3, True, "bf16"),
    (128, [200, 129, 128, 127, 1], 1, 8, 1, 0, False, "bf16"),
    (64, [300, 65], 16, 8, 1, 0, True, "bf16"),
    (32, [130, 257], 12, 6, 3, 40, True, "fp8"),
    (256, [600, 255], 9, 16, 1, 0, False, "fp8"),
]


@pytest.mark.parametrize("case", GRID, ids=[f"g{i}" for i in range(len(GRID))])
def test_grid_all_entries(case):
    P, L, n, Hq, Hkv, W, sinks, kv = case
    inp = make_paged_inputs(200 + GRID.index(case), seq_lens=L, q_lens=n, num_q_heads=Hq,
                            num_kv_heads=Hkv, page_size=P, kv_dtype=kv, window=W, sinks=sinks,
                            extra_pages=3, write_align=P if W > 0 else None)
    dev = DeviceInputs(inp)
    entries = (["decode"] if n == 1 else []) + (["verify"] if n <= 16 else []) + ["prefill"]
    outs = [check_call(dev, e, f"g{GRID.index(case)}/{e}") for e in entries]
    for o in outs[1:]:
        compare(to_np(o), to_np(outs[0]), "cross-entry")


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 40])
def test_forced_split_counts(splits):
    inp = make_paged_inputs(77, seq_lens=[3000, 1777, 90], q_lens=[8, 5, 3], num_q_heads=8,
                            num_kv_heads=1, page_size=16, kv_dtype="bf16", sinks=True)
    dev = DeviceInputs(inp)
    check_call(dev, "verify", f"splits={splits}", force_num_splits=splits)


def test_run_to_run_bitwise_determinism_and_page_permutation():
    inp = make_paged_inputs(81, seq_lens=[5000, 4100, 70], q_lens=[4, 4, 4], num_q_heads=8,
                            num_kv_heads=1, page_size=16, kv_dtype="fp8", window=300, sinks=True,
                            write_align=16)
    dev = DeviceInputs(inp)
    a, _, _ = dev.run("verify")
    b, _, _ = dev.run("verify")
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # Move every physical page somewhere else and remap the table.
    perm = torch.randperm(inp.num_pages, generator=torch.Generator().manual_seed(3)).to(dev.device)
    k2 = torch.empty_like(dev.k_cache)
    v2 = torch.empty_like(dev.v_cache)
    k2[perm] = dev.k_cache
    v2[perm] = dev.v_cache
    bt = dev.block_table
    bt2 = torch.where(bt >= 0, perm[bt.clamp(min=0).long()].int(), bt)
    dev.k_cache, dev.v_cache = k2, v2
    c, _, _ = dev.run("verify", block_table=bt2)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


@pytest.mark.parametrize("entry", ["verify", "prefill"])
def test_fp8_values_pass_through_exactly(entry):
    """Window 1: each token sees only its own key, so out = V_p * v_scale.  With
    v_scale 1 and V rows holding every finite E4M3 code, the output must be
    the decoded codes bit for bit (each is exact in bf16)."""
    from oracle import decode_e4m3fn
    inp = make_paged_inputs(91, seq_lens=[9], q_lens=8, num_q_heads=2, num_kv_heads=1,
                            page_size=4, kv_dtype="fp8", window=1, write_align=4)
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]
    L, n = 9, 8
    rows = np.resize(codes, (n, 128))
    for i in range(n):
        pos = L - n + i
        inp.v_cache[inp.block_table[0, pos // 4], pos % 4, 0, :] = rows[i]
    inp.v_scale = 1.0
    dev = DeviceInputs(inp)
    say(f"fp8 pass-through via {entry}")
    out, _, _ = dev.run(entry)
    torch.cuda.synchronize()
    got = to_np(out)
    want = decode_e4m3fn(rows)
    for h in range(2):
        assert np.array_equal(got[:, h, :], want), "E4M3 decode is not exact on the GPU"


@pytest.mark.parametrize("q_len,hq,splits", [(1, 8, 0), (1, 8, 9), (4, 8, 5), (8, 8, 40)])
def test_workspace_reuse_across_calls(q_len, hq, splits):
    """One workspace, several calls with different sequence lengths inside the
    same descriptor bounds: the split partials and the arrival counters the
    last split uses to merge must leave the workspace ready for the next call
    (both the fused-merge and the merge-kernel paths)."""
    from paged_asymmetric_head_amd import binding as B
    entry = "decode" if q_len == 1 else "verify"
    lens = [[3000, 2500, 700], [2999, 64, 3001], [1, 3001, 1500]]
    base = make_paged_inputs(61, seq_lens=lens[0], q_lens=q_len, num_q_heads=hq, num_kv_heads=1,
                             page_size=128, kv_dtype="bf16", max_seq_len=3001)
    dev0 = DeviceInputs(base)
    ws, nbytes = dev0.workspace_for(entry, splits)
    say(f"workspace reuse: {entry} q_len={q_len} splits={splits} ws={nbytes} "
        f"num_splits={B.diffkv_attn_num_splits(dev0.desc(entry, splits), B.ENTRIES[entry])}")
    for k, L in enumerate(lens):
        Lq = [max(x, q_len) for x in L]
        inp = make_paged_inputs(61 + k, seq_lens=Lq, q_lens=q_len, num_q_heads=hq, num_kv_heads=1,
                                page_size=128, kv_dtype="bf16", max_seq_len=3001)
        dev = DeviceInputs(inp)
        out, _, _ = dev.run(entry, force_num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        compare(to_np(out), oracle(inp).out, f"reuse call {k}")
