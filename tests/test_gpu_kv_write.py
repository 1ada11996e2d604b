"""GPU parity of the paged KV write: the HIP kernel against the oracle, byte for byte.

Every call goes through the C ABI (diffkv_kv_write via the ctypes binding).
The caches start NaN-filled or holding a generated workload, so a stray or
missing write shows up as a byte difference anywhere in either pool.
"""

import numpy as np
import pytest
import torch

from oracle import paged_attention, paged_kv_write
from paged_asymmetric_head_amd import binding as B
from paged_asymmetric_head_amd.device import DeviceInputs, _to_device
from paged_asymmetric_head_amd.synth import make_paged_inputs, to_bf16_bits, workload
from parity import compare, to_np

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def desc_for(inp, *, decode=False, num_pages=None):
    return B.AttnDesc(batch=inp.batch, num_q_heads=inp.num_q_heads, num_kv_heads=inp.num_kv_heads,
                      head_dim_qk=192, head_dim_v=128, page_size=inp.page_size,
                      num_pages=inp.num_pages if num_pages is None else num_pages,
                      block_table_stride=inp.block_table_stride, max_seq_len=inp.max_seq_len,
                      max_q_len=1 if decode else inp.max_q_len, total_q=inp.total_q,
                      kv_dtype=B.KV_FP8_E4M3 if inp.kv_dtype == "fp8" else B.KV_BF16,
                      force_num_splits=0)


def cache_np(t, kv_dtype):
    a = t.cpu().numpy()
    return a.view(np.uint16) if kv_dtype == "bf16" else a


def gpu_write(inp, k_new, v_new, k_cache, v_cache, ks, vs, *, block_table=None, decode=False):
    """One diffkv_kv_write call on device copies; returns the caches as numpy."""
    bt = inp.block_table if block_table is None else block_table
    kc, vc = _to_device(k_cache, "cuda"), _to_device(v_cache, "cuda")
    B.diffkv_kv_write(desc_for(inp, decode=decode), _to_device(k_new, "cuda"),
                      _to_device(v_new, "cuda"), kc, vc,
                      _to_device(bt.astype(np.int32), "cuda"),
                      _to_device(inp.seq_lens.astype(np.int32), "cuda"),
                      None if decode else _to_device(inp.q_lens.astype(np.int32), "cuda"),
                      float(ks), float(vs))
    torch.cuda.synchronize()
    return cache_np(kc, inp.kv_dtype), cache_np(vc, inp.kv_dtype)


def new_rows(seed, T, hkv, scale=3.0, specials=False):
    """Seeded bf16 rows for the new tokens; with specials, NaN, +-inf, -0 and
    values below the smallest E4M3 subnormal are planted at fixed places."""
    rng = np.random.default_rng(seed)
    k = (rng.standard_normal((T, hkv, 192)) * scale).astype(np.float32)
    v = (rng.standard_normal((T, hkv, 128)) * scale).astype(np.float32)
    if specials:
        for a in (k, v):
            f = a.reshape(-1)
            f[0:7] = [np.nan, -np.nan, np.inf, -np.inf, -0.0, 1e-30, -1e-30]
            f[-5:] = [np.nan, 6e4, -6e4, 2.0 ** -130, -(2.0 ** -140)]
    return to_bf16_bits(k), to_bf16_bits(v)


def check_caches(got, want, tag):
    for name, g, w in zip(("k_cache", "v_cache"), got, want):
        diff = np.argwhere(g != w)
        assert diff.size == 0, f"{tag}: {name} differs at {len(diff)} bytes, first {diff[:4].tolist()}"


CASES = [(P, dt) for dt in ("bf16", "fp8") for P in (1, 16, 128)]


@pytest.mark.parametrize("P,kv_dtype", CASES, ids=[f"p{P}_{dt}" for P, dt in CASES])
def test_kv_write_matches_oracle(P, kv_dtype):
    """Ragged new-token counts (1 .. 129, crossing pages at every size), two
    KV heads, a pool with spare pages; whole caches compared byte for byte."""
    inp = make_paged_inputs(71, seq_lens=[300, 77, 129, 1000, 16], q_lens=[5, 1, 129, 37, 16],
                            num_q_heads=4, num_kv_heads=2, page_size=P, kv_dtype=kv_dtype,
                            extra_pages=3)
    k_new, v_new = new_rows(72, inp.total_q, 2, specials=True)
    ks, vs = (inp.k_scale, inp.v_scale) if kv_dtype == "fp8" else (1.0, 1.0)
    say(f"kv_write p{P} {kv_dtype} total_q={inp.total_q}")
    got = gpu_write(inp, k_new, v_new, inp.k_cache, inp.v_cache, ks, vs)
    want = paged_kv_write(k_new, v_new, inp.k_cache, inp.v_cache, inp.block_table, inp.seq_lens,
                          inp.q_lens, kv_dtype=kv_dtype, k_scale=ks, v_scale=vs)
    check_caches(got, want, f"p{P}_{kv_dtype}")
    assert not np.array_equal(want[0], inp.k_cache)


@pytest.mark.parametrize("scale", [1.0, 0.37, 0.125, 3e-3, 300.0])
def test_fp8_codes_for_every_bf16_value(scale):
    """All 65536 bf16 codes (NaNs, infinities, subnormals included) through
    the encoder at scales that are exact, inexact, clamping and flushing."""
    T = 512
    inp = make_paged_inputs(5, seq_lens=[600], q_lens=[T], num_q_heads=1, num_kv_heads=1,
                            page_size=16, kv_dtype="fp8")
    every = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    k_new = np.concatenate([every, every[::2]]).reshape(T, 1, 192)
    v_new = every[np.random.default_rng(6).permutation(65536)].reshape(T, 1, 128)
    say(f"kv_write every bf16 code, scale {scale}")
    got = gpu_write(inp, k_new, v_new, inp.k_cache, inp.v_cache, scale, scale)
    want = paged_kv_write(k_new, v_new, inp.k_cache, inp.v_cache, inp.block_table, inp.seq_lens,
                          inp.q_lens, kv_dtype="fp8", k_scale=scale, v_scale=scale)
    check_caches(got, want, f"every_code_{scale}")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_kv_write_decode_without_q_lens(kv_dtype):
    """One new token per sequence (q_lens NULL), page 128, 33 sequences."""
    lens = [int(x) for x in np.random.default_rng(8).integers(1, 2000, 33)]
    inp = make_paged_inputs(9, seq_lens=lens, q_lens=1, num_q_heads=8, num_kv_heads=1,
                            page_size=128, kv_dtype=kv_dtype)
    k_new, v_new = new_rows(10, inp.total_q, 1)
    ks, vs = (inp.k_scale, inp.v_scale) if kv_dtype == "fp8" else (1.0, 1.0)
    say(f"kv_write decode {kv_dtype}")
    got = gpu_write(inp, k_new, v_new, inp.k_cache, inp.v_cache, ks, vs, decode=True)
    want = paged_kv_write(k_new, v_new, inp.k_cache, inp.v_cache, inp.block_table, inp.seq_lens,
                          inp.q_lens, kv_dtype=kv_dtype, k_scale=ks, v_scale=vs)
    check_caches(got, want, f"decode_{kv_dtype}")


def test_kv_write_skips_tokens_whose_page_is_out_of_range():
    """Sequence 1's pages for its new tokens point past the pool or are -1:
    nothing is written for it; the others are written as the oracle does."""
    inp = make_paged_inputs(12, seq_lens=[200, 300, 150], q_lens=[9, 40, 20], num_q_heads=4,
                            num_kv_heads=1, page_size=16, kv_dtype="fp8", extra_pages=2)
    k_new, v_new = new_rows(13, inp.total_q, 1)
    bt = inp.block_table.copy()
    L, n = int(inp.seq_lens[1]), int(inp.q_lens[1])
    for t in range((L - n) // 16, (L - 1) // 16 + 1):
        bt[1, t] = inp.num_pages + 7 if t % 2 else -1
    say("kv_write out-of-range pages")
    got = gpu_write(inp, k_new, v_new, inp.k_cache, inp.v_cache, inp.k_scale, inp.v_scale,
                    block_table=bt)
    keep = [0, 2]
    rows = np.concatenate([np.arange(0, 9), np.arange(49, 69)])
    want = paged_kv_write(k_new[rows], v_new[rows], inp.k_cache, inp.v_cache, bt[keep],
                          inp.seq_lens[keep], inp.q_lens[keep], kv_dtype="fp8",
                          k_scale=inp.k_scale, v_scale=inp.v_scale)
    check_caches(got, want, "out_of_range")


@pytest.mark.parametrize("kv_dtype,entry", [("bf16", "verify"), ("fp8", "verify"),
                                            ("fp8", "prefill")])
def test_write_then_attention(kv_dtype, entry):
    """The written caches feed the attention kernels: new tokens written by
    the HIP path into NaN slots, then attention over them, against the
    oracle's attention over the oracle's write."""
    inp = make_paged_inputs(14, seq_lens=[700, 131, 64, 900], q_lens=[8, 4, 2, 7], num_q_heads=8,
                            num_kv_heads=1, page_size=16, kv_dtype=kv_dtype, window=128,
                            sinks=True)
    k_new, v_new = new_rows(15, inp.total_q, 1, scale=1.0)
    kc, vc = inp.k_cache.copy(), inp.v_cache.copy()
    nan = np.iinfo(kc.dtype).max
    for b in range(inp.batch):
        L, n = int(inp.seq_lens[b]), int(inp.q_lens[b])
        for p in range(L - n, L):
            kc[inp.block_table[b, p // 16], p % 16] = nan
            vc[inp.block_table[b, p // 16], p % 16] = nan
    ks, vs = (inp.k_scale, inp.v_scale) if kv_dtype == "fp8" else (1.0, 1.0)
    say(f"write then {entry} {kv_dtype}")
    dev = DeviceInputs(inp)
    dev.k_cache, dev.v_cache = _to_device(kc, "cuda"), _to_device(vc, "cuda")
    B.diffkv_kv_write(desc_for(inp), _to_device(k_new, "cuda"), _to_device(v_new, "cuda"),
                      dev.k_cache, dev.v_cache, dev.block_table, dev.seq_lens, dev.q_lens, ks, vs)
    out, _, _ = dev.run(entry)
    torch.cuda.synchronize()
    kw, vw = paged_kv_write(k_new, v_new, kc, vc, inp.block_table, inp.seq_lens, inp.q_lens,
                            kv_dtype=kv_dtype, k_scale=ks, v_scale=vs)
    check_caches((cache_np(dev.k_cache, kv_dtype), cache_np(dev.v_cache, kv_dtype)), (kw, vw),
                 f"write_{entry}_{kv_dtype}")
    args = inp.oracle_kwargs()
    args.update(k_cache=kw, v_cache=vw)
    ref = paged_attention(**args)
    compare(to_np(out), ref.out, f"write_then_{entry}_{kv_dtype}")


def test_kv_write_chunked_prefill_size():
    """The chunked-prefill chunk at its full size: 4096 new tokens after
    26624 cached, two KV heads, page 128, FP8, byte for byte."""
    inp = workload("chunked_prefill")
    k_new, v_new = new_rows(16, inp.total_q, inp.num_kv_heads)
    say(f"kv_write chunked_prefill total_q={inp.total_q}")
    got = gpu_write(inp, k_new, v_new, inp.k_cache, inp.v_cache, inp.k_scale, inp.v_scale)
    want = paged_kv_write(k_new, v_new, inp.k_cache, inp.v_cache, inp.block_table, inp.seq_lens,
                          inp.q_lens, kv_dtype="fp8", k_scale=inp.k_scale, v_scale=inp.v_scale)
    check_caches(got, want, "chunked_prefill")
