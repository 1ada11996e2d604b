"""Pins of the KV-write oracle and its FP8 encoder (CPU only).

Each pin checks the oracle against something other than itself: torch's own
float8_e4m3fn cast (a library routine), worked closed forms of the format,
the round trip through the definition-based decoder, the seeded generator's
own paging code (synth.py, which builds the caches the attention tests use),
and brute-force dense attention over the logical rows.
"""

import math

import numpy as np
import pytest
import torch

from oracle import decode_bf16, decode_e4m3fn, encode_e4m3fn, paged_attention, paged_kv_write
from paged_asymmetric_head_amd.synth import make_paged_inputs, to_bf16_bits


def _torch_e4m3(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_encoder_matches_torch_cast_on_every_bf16_value_in_range():
    f = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    x = f[np.isfinite(f) & (np.abs(f) <= 448)]
    assert x.size > 30000
    np.testing.assert_array_equal(encode_e4m3fn(x), _torch_e4m3(x))


def test_encoder_matches_torch_cast_on_random_float32():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.uniform(-448, 448, 500_000), rng.standard_normal(300_000) * 3,
                        rng.standard_normal(200_000) * 1e-2]).astype(np.float32)
    np.testing.assert_array_equal(encode_e4m3fn(x), _torch_e4m3(x))


def test_encoder_closed_forms():
    cases = {
        448.0: 0x7E, -448.0: 0xFE,            # largest finite
        2.0 ** -9: 0x01,                       # smallest subnormal
        2.0 ** -10: 0x00,                      # halfway to zero: tie to the even code 0
        3 * 2.0 ** -10: 0x02,                  # halfway between codes 1 and 2: even
        2.0 ** -6: 0x08,                       # smallest normal
        1.0: 0x38, 1.0625: 0x38,               # tie between 1.0 (0x38) and 1.125 (0x39): even
        1.1875: 0x3A,                          # tie between 1.125 (0x39) and 1.25 (0x3A): even
        464.0: 0x7E, 500.0: 0x7E, 1e30: 0x7E,  # clamped to 448
    }
    x = np.array(list(cases), dtype=np.float32)
    np.testing.assert_array_equal(encode_e4m3fn(x), np.array(list(cases.values()), dtype=np.uint8))
    zeros = encode_e4m3fn(np.array([0.0, -0.0], dtype=np.float32))      # the sign bit is kept
    np.testing.assert_array_equal(zeros, np.array([0x00, 0x80], dtype=np.uint8))
    special = encode_e4m3fn(np.array([np.inf, -np.inf, np.nan, -np.nan], dtype=np.float32))
    np.testing.assert_array_equal(special, np.array([0x7E, 0xFE, 0x7F, 0xFF], dtype=np.uint8))


def test_encoder_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    np.testing.assert_array_equal(encode_e4m3fn(decode_e4m3fn(codes).astype(np.float32)), codes)


@pytest.mark.parametrize("P", [1, 16, 128])
def test_bf16_write_rebuilds_the_generators_cache(P):
    """Clearing the new tokens' slots and writing their logical rows back
    must give the generator's cache byte for byte (its paging is its own)."""
    inp = make_paged_inputs(31, seq_lens=[300, 77, 129], q_lens=[5, 1, 129], num_q_heads=4,
                            num_kv_heads=2, page_size=P, kv_dtype="bf16", extra_pages=3)
    B = inp.batch
    k_new = np.concatenate([inp.logical_k[b][-int(inp.q_lens[b]):] for b in range(B)])
    v_new = np.concatenate([inp.logical_v[b][-int(inp.q_lens[b]):] for b in range(B)])
    kc, vc = inp.k_cache.copy(), inp.v_cache.copy()
    for b in range(B):        # clear the new tokens' slots (NaN fill, as unused slots hold)
        L, n = int(inp.seq_lens[b]), int(inp.q_lens[b])
        for p in range(L - n, L):
            kc[inp.block_table[b, p // P], p % P] = 0xFFFF
            vc[inp.block_table[b, p // P], p % P] = 0xFFFF
    assert not np.array_equal(kc, inp.k_cache)
    kw, vw = paged_kv_write(k_new, v_new, kc, vc, inp.block_table, inp.seq_lens, inp.q_lens,
                            kv_dtype="bf16")
    np.testing.assert_array_equal(kw, inp.k_cache)
    np.testing.assert_array_equal(vw, inp.v_cache)


def _fp8_write_case(seed, P):
    rng = np.random.default_rng(seed)
    inp = make_paged_inputs(seed, seq_lens=[260, 40, 131], q_lens=[7, 40, 3], num_q_heads=8,
                            num_kv_heads=1, page_size=P, kv_dtype="fp8", extra_pages=2)
    T = inp.total_q
    k_new = to_bf16_bits((rng.standard_normal((T, 1, 192)) * 3).astype(np.float32))
    v_new = to_bf16_bits((rng.standard_normal((T, 1, 128)) * 3).astype(np.float32))
    return inp, k_new, v_new


@pytest.mark.parametrize("P", [1, 16, 128])
def test_fp8_write_codes_slots_and_untouched_bytes(P):
    inp, k_new, v_new = _fp8_write_case(41, P)
    ks, vs = np.float32(0.0125), np.float32(0.02)
    kw, vw = paged_kv_write(k_new, v_new, inp.k_cache, inp.v_cache, inp.block_table, inp.seq_lens,
                            inp.q_lens, kv_dtype="fp8", k_scale=ks, v_scale=vs)
    # codes: torch's cast of the float32 quotient; slots: the generator's
    # logical -> physical map, recovered from where it wrote each logical row
    written = np.zeros(kw.shape[:2], dtype=bool)
    r0 = 0
    for b in range(inp.batch):
        L, n = int(inp.seq_lens[b]), int(inp.q_lens[b])
        start = int(inp.written_start[b])
        for i in range(n):
            p = L - n + i
            # the generator stored logical row p - start at this slot
            where = np.argwhere(np.all(inp.k_cache == inp.logical_k[b][p - start][None, None], axis=(2, 3)))
            assert len(where) >= 1
            page, slot = where[0]
            k = np.clip(decode_bf16(k_new[r0 + i]).astype(np.float32) / ks, -448, 448)
            v = np.clip(decode_bf16(v_new[r0 + i]).astype(np.float32) / vs, -448, 448)
            np.testing.assert_array_equal(kw[page, slot], _torch_e4m3(k))
            np.testing.assert_array_equal(vw[page, slot], _torch_e4m3(v))
            written[page, slot] = True
        r0 += n
    np.testing.assert_array_equal(kw[~written], inp.k_cache[~written])
    np.testing.assert_array_equal(vw[~written], inp.v_cache[~written])


def test_written_rows_are_what_attention_then_reads():
    """After the write, the attention oracle through the block table equals
    brute-force dense attention over the logical rows (new rows decoded from
    the codes just written), so the write puts each row where a read finds it."""
    inp, k_new, v_new = _fp8_write_case(43, 16)
    ks, vs = np.float32(inp.k_scale), np.float32(inp.v_scale)    # the cache's per-tensor scales
    kw, vw = paged_kv_write(k_new, v_new, inp.k_cache, inp.v_cache, inp.block_table, inp.seq_lens,
                            inp.q_lens, kv_dtype="fp8", k_scale=ks, v_scale=vs)
    args = inp.oracle_kwargs()
    args.update(k_cache=kw, v_cache=vw, k_scale=float(ks), v_scale=float(vs))
    res = paged_attention(**args)
    r0 = 0
    for b in range(inp.batch):
        L, n = int(inp.seq_lens[b]), int(inp.q_lens[b])
        start = int(inp.written_start[b])
        K = decode_e4m3fn(inp.logical_k[b][:, 0]) * float(inp.k_scale)
        V = decode_e4m3fn(inp.logical_v[b][:, 0]) * float(inp.v_scale)
        Kn = decode_e4m3fn(encode_e4m3fn(decode_bf16(k_new[r0:r0 + n, 0]).astype(np.float32) / ks)) * float(ks)
        Vn = decode_e4m3fn(encode_e4m3fn(decode_bf16(v_new[r0:r0 + n, 0]).astype(np.float32) / vs)) * float(vs)
        K = np.concatenate([K[:L - n - start], Kn])
        V = np.concatenate([V[:L - n - start], Vn])
        for i in range(n):
            p = L - n + i
            for h in range(inp.num_q_heads):
                q = decode_bf16(inp.q[r0 + i, h])
                x = [inp.softmax_scale * math.fsum(q * K[j]) for j in range(p - start + 1)]
                m = max(x)
                e = [math.exp(v - m) for v in x]
                den = math.fsum(e)
                ref = np.array([math.fsum(e[j] * V[j, d] for j in range(len(e))) / den for d in range(128)])
                np.testing.assert_allclose(res.out[r0 + i, h], ref, rtol=1e-12, atol=1e-12)
        r0 += n
