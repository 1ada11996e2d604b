"""Pins of the FP64 oracle against things other than itself (CPU only).

* brute force on tiny inputs (logical arrays, explicit mask, fsum loops),
* torch's scaled_dot_product_attention in float64 (library routine),
* closed forms (equal scores give the mean of V; the sink relation; a single
  visible key returns that key's value),
* invariants (page permutation, split merge, verify == decodes, NaN tails).
"""

import math

import numpy as np
import pytest
import torch

from oracle import paged_attention, decode_bf16, decode_e4m3fn
from paged_asymmetric_head_amd.synth import make_paged_inputs, workload
from brute import brute_force, lib_decode


def run(inp, **kw):
    args = inp.oracle_kwargs()
    args.update(kw)
    return paged_attention(**args)


def rel(a, b):
    return np.max(np.abs(a - b) / np.maximum(np.abs(b), 1e-300))


# --- codecs ------------------------------------------------------------------

def test_e4m3fn_all_codes_match_torch_and_spec_points():
    codes = np.arange(256, dtype=np.uint8)
    ours = decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[~np.isnan(ours)], ref[~np.isnan(ref)])
    # Points fixed by the format's definition.
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6 and ours[0x38] == 1.0
    assert ours[0x00] == 0.0 and ours[0x80] == 0.0 and math.copysign(1, ours[0x80]) == -1
    assert np.sum(np.isnan(ours)) == 2


def test_bf16_all_codes_match_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = decode_bf16(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert decode_bf16(np.array([0x3F80], dtype=np.uint16))[0] == 1.0


# --- brute force grid ---------------------------------------------------------

GRID = [
    # (page, seq_lens, q_len, Hq, Hkv, window, sinks, kv)
    (1, [5, 9], 1, 2, 1, 0, False, "bf16"),
    (2, [7, 3], 2, 4, 2, 0, True, "bf16"),
    (3, [10, 17, 4], 3, 4, 1, 5, False, "fp8"),
    (16, [16, 17, 15, 1], 1, 8, 2, 0, True, "fp8"),
    (16, [33, 40], 8, 4, 1, 16, True, "bf16"),
    (2, [12, 30], 5, 2, 2, 1, False, "bf16"),
    (3, [9, 23], 4, 16, 1, 70, True, "fp8"),
    (16, [48, 70], 7, 4, 4, 9, False, "fp8"),
    (1, [20], 6, 1, 1, 3, True, "bf16"),
]


@pytest.mark.parametrize("case", GRID, ids=[f"g{i}" for i in range(len(GRID))])
def test_oracle_matches_brute_force(case):
    P, L, n, Hq, Hkv, W, sinks, kv = case
    inp = make_paged_inputs(100 + GRID.index(case), seq_lens=L, q_lens=n, num_q_heads=Hq,
                            num_kv_heads=Hkv, page_size=P, kv_dtype=kv, window=W, sinks=sinks,
                            extra_pages=3, write_align=P if W > 0 else None)
    res = run(inp)
    bo, bl, bc = brute_force(inp)
    assert np.all(np.isfinite(res.out))
    assert np.array_equal(res.count, bc)
    np.testing.assert_allclose(res.out, bo, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(res.lse, bl, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("kv,W,sinks", [("bf16", 0, True), ("fp8", 6, False)])
def test_oracle_symmetric_heads_match_brute_force(kv, W, sinks):
    """Symmetric 128/128 heads: the same definition with K as wide as V."""
    inp = make_paged_inputs(150 + W, seq_lens=[30, 17], q_lens=[4, 2], num_q_heads=4,
                            num_kv_heads=2, page_size=4, kv_dtype=kv, window=W, sinks=sinks,
                            extra_pages=2, write_align=4 if W > 0 else None, head_dim_qk=128)
    assert inp.q.shape[2] == 128 and inp.k_cache.shape[3] == 128
    res = run(inp)
    bo, bl, bc = brute_force(inp)
    assert np.array_equal(res.count, bc)
    np.testing.assert_allclose(res.out, bo, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(res.lse, bl, rtol=1e-12, atol=1e-13)


def test_oracle_row_subset_matches_full():
    inp = make_paged_inputs(7, seq_lens=[40, 55, 23], q_lens=[3, 6, 2], num_q_heads=8,
                            num_kv_heads=2, page_size=4, kv_dtype="bf16", window=11, sinks=True)
    full = run(inp)
    sub = run(inp, tokens=[10, 1, 4])
    assert list(sub.tokens) == [1, 4, 10]
    # The key range (and so the summation length) differs: equal to rounding.
    np.testing.assert_allclose(sub.out, full.out[[1, 4, 10]], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(sub.lse, full.lse[[1, 4, 10]], rtol=1e-14)
    assert np.array_equal(sub.count, full.count[[1, 4, 10]])


# --- library routine: scaled_dot_product_attention ------------------------------

@pytest.mark.parametrize("kv,W", [("bf16", 0), ("fp8", 0), ("bf16", 13), ("fp8", 6)])
def test_oracle_matches_sdpa_float64(kv, W):
    inp = make_paged_inputs(31, seq_lens=[45, 64, 28], q_lens=[4, 8, 1], num_q_heads=8,
                            num_kv_heads=2, page_size=8, kv_dtype=kv, window=W,
                            write_align=8 if W else None)
    res = run(inp)
    G = 4
    ks = inp.k_scale if kv == "fp8" else 1.0
    vs = inp.v_scale if kv == "fp8" else 1.0
    q = torch.from_numpy(inp.q.view(np.int16)).view(torch.bfloat16).double()
    r0 = 0
    for b in range(inp.batch):
        L, n, st = int(inp.seq_lens[b]), int(inp.q_lens[b]), int(inp.written_start[b])
        K = np.zeros((L, 2, 192))
        V = np.zeros((L, 2, 128))
        K[st:] = lib_decode(inp.logical_k[b], kv) * ks
        V[st:] = lib_decode(inp.logical_v[b], kv) * vs
        Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0)   # [Hq, L, 192]
        Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0)
        Qt = q[r0:r0 + n].permute(1, 0, 2)                                       # [Hq, n, 192]
        pos = torch.arange(L - n, L)[:, None]
        j = torch.arange(L)[None, :]
        mask = j <= pos
        if W > 0:
            mask = mask & (pos - j < W)
        ref = torch.nn.functional.scaled_dot_product_attention(
            Qt, Kt, Vt, attn_mask=mask, scale=inp.softmax_scale)                   # [Hq, n, 128]
        got = torch.from_numpy(res.out[r0:r0 + n]).permute(1, 0, 2)
        torch.testing.assert_close(got, ref, rtol=1e-12, atol=1e-12)
        r0 += n


# --- closed forms ----------------------------------------------------------------

def _zero_keys(inp):
    inp.k_cache = np.where(np.isnan(decode_bf16(inp.k_cache)) if inp.kv_dtype == "bf16"
                           else np.isnan(decode_e4m3fn(inp.k_cache)), inp.k_cache,
                           np.zeros_like(inp.k_cache))
    return inp


@pytest.mark.parametrize("sinks", [False, True])
def test_equal_scores_give_mean_of_visible_values(sinks):
    inp = make_paged_inputs(5, seq_lens=[30, 12], q_lens=[3, 2], num_q_heads=4, num_kv_heads=1,
                            page_size=4, kv_dtype="bf16", window=7, sinks=sinks, write_align=4)
    _zero_keys(inp)
    res = run(inp)
    r0 = 0
    for b in range(inp.batch):
        L, n, st = int(inp.seq_lens[b]), int(inp.q_lens[b]), int(inp.written_start[b])
        V = lib_decode(inp.logical_v[b], "bf16")
        for i in range(n):
            p = L - n + i
            lo = max(0, p - 7 + 1)
            vis = V[lo - st:p + 1 - st, 0]
            for h in range(4):
                expect = vis.sum(axis=0) / (vis.shape[0] + (math.exp(float(inp.sinks[h])) if sinks else 0))
                np.testing.assert_allclose(res.out[r0 + i, h], expect, rtol=1e-12, atol=1e-14)
                assert res.count[r0 + i, h] == p + 1 - lo
        r0 += n


def test_sink_closed_form_and_limits():
    base = dict(seq_lens=[50, 19], q_lens=[4, 2], num_q_heads=4, num_kv_heads=2, page_size=8,
                kv_dtype="fp8", window=0)
    inp = make_paged_inputs(9, sinks=True, **base)
    with_sink = run(inp)
    no_sink = run(inp, sinks=None)
    s = inp.sinks.astype(np.float64)
    factor = 1.0 + np.exp(s[None, :] - no_sink.lse)
    np.testing.assert_allclose(with_sink.out, no_sink.out / factor[..., None], rtol=1e-12, atol=1e-15)
    # lse excludes the sink.
    np.testing.assert_allclose(with_sink.lse, no_sink.lse, rtol=1e-13)
    very_low = run(inp, sinks=np.full(4, -1e4))
    assert np.array_equal(very_low.out, no_sink.out)
    very_high = run(inp, sinks=np.full(4, 1e4))
    assert np.max(np.abs(very_high.out)) == 0.0


def test_single_visible_key_returns_its_value():
    # Window 1: each token sees only itself, so out equals its V row exactly.
    inp = make_paged_inputs(11, seq_lens=[9, 33], q_lens=[3, 5], num_q_heads=4, num_kv_heads=2,
                            page_size=4, kv_dtype="bf16", window=1, write_align=4)
    res = run(inp)
    r0 = 0
    for b in range(inp.batch):
        L, n, st = int(inp.seq_lens[b]), int(inp.q_lens[b]), int(inp.written_start[b])
        V = lib_decode(inp.logical_v[b], "bf16")
        for i in range(n):
            for h in range(4):
                assert np.array_equal(res.out[r0 + i, h], V[L - n + i - st, h // 2])
                assert res.count[r0 + i, h] == 1
        r0 += n
    # A one-token sequence, full attention.
    one = make_paged_inputs(12, seq_lens=[1], q_lens=1, num_q_heads=2, num_kv_heads=1,
                            page_size=16, kv_dtype="fp8")
    r = run(one)
    v = lib_decode(one.logical_v[0], "fp8")[0, 0] * one.v_scale
    assert np.array_equal(r.out[0, 0], v) and np.array_equal(r.out[0, 1], v)


def test_window_at_least_context_is_full_attention():
    a = make_paged_inputs(13, seq_lens=[20, 31], q_lens=[4, 2], num_q_heads=4, num_kv_heads=1,
                          page_size=4, kv_dtype="bf16", window=0)
    full = run(a)
    wide = run(a, window=31)
    assert np.array_equal(full.out, wide.out)


# --- invariants ------------------------------------------------------------------

def test_page_permutation_leaves_output_bitwise_unchanged():
    inp = make_paged_inputs(17, seq_lens=[41, 70, 9], q_lens=[2, 5, 1], num_q_heads=8,
                            num_kv_heads=2, page_size=4, kv_dtype="fp8", window=12, sinks=True,
                            extra_pages=5)
    a = run(inp)
    pi = np.random.default_rng(0).permutation(inp.num_pages)
    k2 = np.empty_like(inp.k_cache)
    v2 = np.empty_like(inp.v_cache)
    k2[pi] = inp.k_cache
    v2[pi] = inp.v_cache
    bt2 = np.where(inp.block_table >= 0, pi[np.maximum(inp.block_table, 0)], -1).astype(np.int32)
    b = run(inp, k_cache=k2, v_cache=v2, block_table=bt2)
    assert np.array_equal(a.out, b.out) and np.array_equal(a.lse, b.lse)


@pytest.mark.parametrize("split", [1, 2, 3, 7, "page"])
def test_split_merge_equals_unsplit(split):
    inp = make_paged_inputs(19, seq_lens=[61, 100, 17], q_lens=[4, 8, 1], num_q_heads=8,
                            num_kv_heads=1, page_size=16, kv_dtype="bf16", window=0, sinks=True)
    a = run(inp)
    b = run(inp, split=split)
    np.testing.assert_allclose(b.out, a.out, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(b.lse, a.lse, rtol=1e-13)


def test_verify_block_equals_sequence_of_decodes():
    n = 6
    inp = make_paged_inputs(23, seq_lens=[57], q_lens=n, num_q_heads=4, num_kv_heads=1,
                            page_size=8, kv_dtype="bf16", window=10, sinks=True, write_align=8)
    ver = run(inp)
    L = int(inp.seq_lens[0])
    for i in range(n):
        dec = run(inp, q=inp.q[i:i + 1], seq_lens=np.array([L - n + 1 + i]), q_lens=np.array([1]))
        np.testing.assert_allclose(dec.out[0], ver.out[i], rtol=1e-13, atol=1e-15)
        assert np.array_equal(dec.count[0], ver.count[i])


def test_nan_tails_never_reach_the_output():
    # The generator leaves every unused slot and page NaN; the window case also
    # leaves whole pages before the window unwritten.  Entries of pages that
    # must not be read are set to -1: the oracle raises if it touches one.
    inp = make_paged_inputs(29, seq_lens=[67, 130, 5], q_lens=[3, 4, 2], num_q_heads=4,
                            num_kv_heads=1, page_size=16, kv_dtype="fp8", window=20, sinks=True,
                            extra_pages=4, write_align=16)
    assert np.isnan(decode_e4m3fn(inp.k_cache)).any()
    bt = inp.block_table.copy()
    for b in range(inp.batch):
        L, n = int(inp.seq_lens[b]), int(inp.q_lens[b])
        first_page = max(0, L - n - 20 + 1) // 16
        bt[b, :first_page] = -1
    res = run(inp, block_table=bt)
    assert np.all(np.isfinite(res.out)) and np.all(np.isfinite(res.lse))
    ref = run(inp)
    assert np.array_equal(res.out, ref.out)


@pytest.mark.parametrize("which,split", [("k", None), ("v", None), ("k", 3), ("v", "page")])
def test_nan_in_a_visible_key_propagates(which, split):
    """The definition sums over every visible key, so a NaN in a visible K or V
    row makes every output row that sees it NaN (all query heads of that KV
    head), while rows that do not see it (earlier tokens of the causal block,
    other KV heads, other sequences) stay finite.  Only masked keys may be
    dropped; an oracle that zeroed every non-finite score would hide a kernel
    that silently skips NaN keys."""
    inp = make_paged_inputs(31, seq_lens=[40, 25], q_lens=[4, 2], num_q_heads=4, num_kv_heads=2,
                            page_size=8, kv_dtype="bf16", sinks=True)
    L, n, P = 40, 4, 8
    j = L - n + 2                                   # key of token 2: seen by tokens 2 and 3 only
    page, slot = inp.block_table[0, j // P], j % P
    cache = inp.k_cache if which == "k" else inp.v_cache
    cache[page, slot, 1, 5] = 0x7FC0                # NaN in KV head 1's row
    res = run(inp, split=split)
    bad = np.isnan(res.out).any(axis=2)             # [total_q, Hq]
    want = np.zeros_like(bad)
    want[2:4, 2:4] = True                           # tokens 2, 3 of sequence 0; heads of KV head 1
    assert np.array_equal(bad, want)
    if which == "v":                                # NaN in one V dim: only that dim
        assert np.isnan(res.out[2:4, 2:4, 5]).all()
        assert np.isfinite(np.delete(res.out[2:4, 2:4], 5, axis=2)).all()
    else:
        assert np.isnan(res.out[2:4, 2:4]).all() and np.isnan(res.lse[2:4, 2:4]).all()


def test_nan_partial_propagates_through_combine():
    from oracle import combine_partials
    outs = np.zeros((3, 2, 2, 4))
    lses = np.array([[[0.5, -np.inf], [1.0, 2.0]], [[np.nan, 0.0], [0.0, 0.0]],
                     [[-np.inf, -np.inf], [0.3, 0.1]]])
    out, lse = combine_partials(outs, lses, sinks=np.array([0.0, 1.0]))
    assert np.isnan(out[0, 0]).all() and np.isnan(lse[0, 0])
    assert np.isfinite(out[[0, 1, 1], [1, 0, 1]]).all()


@pytest.mark.parametrize("tokens_per_item", [1, 3, 64])
def test_parallel_runner_gives_the_rows_of_one_call(tokens_per_item):
    """oracle.parallel cuts the rows into groups on threads; every row must be
    the one a single paged_attention call gives (up to the rounding of the
    key-range length each group's products run over), counts exactly."""
    from oracle.parallel import paged_attention_parallel
    inp = make_paged_inputs(33, seq_lens=[300, 41, 150], q_lens=[20, 1, 7], num_q_heads=8,
                            num_kv_heads=2, page_size=16, kv_dtype="fp8", window=50, sinks=True,
                            write_align=16)
    ref = run(inp)
    par = paged_attention_parallel(**inp.oracle_kwargs(), tokens_per_item=tokens_per_item, workers=4)
    assert np.array_equal(par.tokens, ref.tokens) and np.array_equal(par.count, ref.count)
    np.testing.assert_allclose(par.out, ref.out, rtol=0, atol=1e-13)
    np.testing.assert_allclose(par.lse, ref.lse, rtol=0, atol=1e-13)
    sub = paged_attention_parallel(**inp.oracle_kwargs(), tokens=[27, 3, 0, 21], tokens_per_item=2)
    assert list(sub.tokens) == [0, 3, 21, 27]
    np.testing.assert_allclose(sub.out, ref.out[[0, 3, 21, 27]], rtol=0, atol=1e-13)


def test_oracle_rejects_unreadable_visible_page():
    inp = make_paged_inputs(3, seq_lens=[20], q_lens=1, num_q_heads=1, num_kv_heads=1,
                            page_size=4, kv_dtype="bf16")
    bt = inp.block_table.copy()
    bt[0, 2] = -1
    with pytest.raises(ValueError):
        run(inp, block_table=bt)


def test_planted_mistakes_are_caught():
    """Each pin above must fail for a plausible error; check the brute force
    disagrees with oracle outputs that carry one (mistakes planted on the CPU)."""
    inp = make_paged_inputs(41, seq_lens=[26, 19], q_lens=[3, 2], num_q_heads=4, num_kv_heads=2,
                            page_size=4, kv_dtype="fp8", window=9, sinks=True, write_align=4)
    bo, _, bc = brute_force(inp)
    good = run(inp)
    np.testing.assert_allclose(good.out, bo, rtol=1e-12, atol=1e-13)
    # wrong window (off by one), dropped sink, transposed GQA map, wrong scale
    variants = [run(inp, window=10).out, run(inp, sinks=None).out,
                run(inp, k_scale=inp.k_scale * 1.01).out]
    swapped = inp.q.copy()
    swapped[:, [0, 2]] = swapped[:, [2, 0]]
    variants.append(run(inp, q=swapped).out)
    for v in variants:
        assert not np.allclose(v, bo, rtol=1e-6, atol=1e-9)


def test_generator_is_deterministic_and_page_size_independent():
    a = make_paged_inputs(4, seq_lens=(300, 900), q_lens=[4] * 5, num_q_heads=8, num_kv_heads=1,
                          page_size=1, kv_dtype="fp8", window=128, sinks=True, write_align=128)
    b = make_paged_inputs(4, seq_lens=(300, 900), q_lens=[4] * 5, num_q_heads=8, num_kv_heads=1,
                          page_size=128, kv_dtype="fp8", window=128, sinks=True, write_align=128)
    assert np.array_equal(a.seq_lens, b.seq_lens) and np.array_equal(a.q, b.q)
    assert all(np.array_equal(x, y) for x, y in zip(a.logical_k, b.logical_k))
    ra, rb = run(a), run(b)
    assert np.array_equal(ra.out, rb.out)


def test_tiny_decode_workload_against_brute_force():
    inp = workload("tiny_decode")
    assert inp.num_pages == 32 and list(inp.seq_lens) == [37, 300]
    res = run(inp)
    bo, _, bc = brute_force(inp)
    np.testing.assert_allclose(res.out, bo, rtol=1e-12, atol=1e-13)
    assert np.array_equal(res.count, bc)
