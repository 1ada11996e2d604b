"""GPU parity for symmetric 128/128 heads (the QK width the kernels also
build besides 192): every attention entry, forced splits, the KV write and
the context split, against the FP64 oracle on the same seeded inputs."""

import numpy as np
import pytest
import torch

from oracle import paged_attention, paged_kv_write
from paged_asymmetric_head_amd import binding as B
from paged_asymmetric_head_amd.device import DeviceInputs, _to_device
from paged_asymmetric_head_amd.synth import make_paged_inputs, to_bf16_bits, workload
from parity import compare, to_np
from test_gpu_parity import check_call, say
from test_gpu_context_split import combine_parts

pytestmark = pytest.mark.gpu

GRID = [
    # (page, seq_lens, q_len, Hq, Hkv, window, sinks, kv)
    (16, [300, 40, 700], 4, 8, 1, 0, True, "bf16"),
    (1, [100, 33], 1, 4, 2, 0, False, "fp8"),
    (128, [1000, 200], 8, 16, 1, 128, True, "fp8"),
    (64, [520, 90], 16, 8, 2, 40, False, "bf16"),
    (8, [70, 9, 33], 3, 2, 2, 5, True, "fp8"),
]


def sym_inputs(i, **kw):
    P, L, n, Hq, Hkv, W, sinks, kv = GRID[i]
    return make_paged_inputs(700 + i, seq_lens=L, q_lens=n, num_q_heads=Hq, num_kv_heads=Hkv,
                             page_size=P, kv_dtype=kv, window=W, sinks=sinks, extra_pages=3,
                             write_align=P if W > 0 else None, head_dim_qk=128, **kw)


@pytest.mark.parametrize("i", range(len(GRID)), ids=[f"s{i}" for i in range(len(GRID))])
def test_symmetric_all_entries(i):
    inp = sym_inputs(i)
    dev = DeviceInputs(inp)
    n = GRID[i][2]
    entries = (["decode"] if n == 1 else []) + (["verify"] if n <= 16 else []) + ["prefill", "mixed"]
    outs = [check_call(dev, e, f"s{i}/{e}") for e in entries]
    for o in outs[1:]:
        compare(to_np(o), to_np(outs[0]), "cross-entry")


@pytest.mark.parametrize("splits", [3, 40])
def test_symmetric_forced_splits(splits):
    inp = make_paged_inputs(710, seq_lens=[3000, 1777, 90], q_lens=[8, 5, 3], num_q_heads=8,
                            num_kv_heads=1, page_size=16, kv_dtype="bf16", sinks=True,
                            head_dim_qk=128)
    check_call(DeviceInputs(inp), "verify", f"sym splits={splits}", force_num_splits=splits)


def test_symmetric_chunked_prefill():
    inp = make_paged_inputs(711, seq_lens=[2600], q_lens=600, num_q_heads=32, num_kv_heads=2,
                            page_size=128, kv_dtype="fp8", head_dim_qk=128)
    check_call(DeviceInputs(inp), "prefill", "sym prefill", tokens=[0, 1, 255, 256, 300, 598, 599])


def test_symmetric_batched_decode_workload():
    inp = workload("batched_decode_sym")
    check_call(DeviceInputs(inp), "decode", "batched_decode_sym")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_symmetric_kv_write(kv_dtype):
    inp = make_paged_inputs(712, seq_lens=[300, 77, 129], q_lens=[5, 1, 129], num_q_heads=4,
                            num_kv_heads=2, page_size=16, kv_dtype=kv_dtype, extra_pages=3,
                            head_dim_qk=128)
    rng = np.random.default_rng(713)
    k_new = to_bf16_bits((rng.standard_normal((inp.total_q, 2, 128)) * 3).astype(np.float32))
    v_new = to_bf16_bits((rng.standard_normal((inp.total_q, 2, 128)) * 3).astype(np.float32))
    ks, vs = (inp.k_scale, inp.v_scale) if kv_dtype == "fp8" else (1.0, 1.0)
    dev = DeviceInputs(inp)
    say(f"sym kv_write {kv_dtype}")
    B.diffkv_kv_write(dev.desc("prefill"), _to_device(k_new, "cuda"), _to_device(v_new, "cuda"),
                      dev.k_cache, dev.v_cache, dev.block_table, dev.seq_lens, dev.q_lens, ks, vs)
    torch.cuda.synchronize()
    want = paged_kv_write(k_new, v_new, inp.k_cache, inp.v_cache, inp.block_table, inp.seq_lens,
                          inp.q_lens, kv_dtype=kv_dtype, k_scale=ks, v_scale=vs)
    for got, w in zip((dev.k_cache, dev.v_cache), want):
        g = got.cpu().numpy()
        g = g.view(np.uint16) if kv_dtype == "bf16" else g
        assert np.array_equal(g, w)


def test_symmetric_context_split():
    inp = make_paged_inputs(714, seq_lens=[300, 129, 1000], q_lens=[4, 1, 3], num_q_heads=8,
                            num_kv_heads=2, page_size=16, kv_dtype="fp8", sinks=True, extra_pages=3,
                            head_dim_qk=128)
    dev = DeviceInputs(inp)
    say("sym context split")
    out, lse = combine_parts(dev, [[0, 100, 128, 300], [0, 1, 64, 129], [0, 250, 999, 1000]])
    ref = paged_attention(**inp.oracle_kwargs())
    compare(to_np(out), ref.out, "sym context split")
