"""Pins of the context-split oracle (CPU only): attention_partial (one key
range's share of every row, no sink) and combine_partials (log-sum-exp merge
with the sink joining once).

The pins check it against brute force on the generator's logical arrays
(explicit key lists, math.fsum, a library decoder), against the unsplit
oracle through a partition of every sequence's keys (cuts inside pages, on
page edges, empty parts), and against closed forms.
"""

import math

import numpy as np
import pytest

from oracle import attention_partial, combine_partials, paged_attention
from paged_asymmetric_head_amd.synth import make_paged_inputs
from brute import lib_decode, visible_matrix


def partial_args(inp):
    a = inp.oracle_kwargs()
    a.pop("sinks")
    return a


def brute_partial(inp, key_lo, key_hi):
    """Restricted attention from the logical rows: out [T, Hq, Dv], lse [T, Hq]."""
    Hq, G = inp.num_q_heads, inp.num_q_heads // inp.num_kv_heads
    q = lib_decode(inp.q, "bf16")
    ks = inp.k_scale if inp.kv_dtype == "fp8" else 1.0
    vs = inp.v_scale if inp.kv_dtype == "fp8" else 1.0
    out = np.zeros((inp.total_q, Hq, 128))
    lse = np.full((inp.total_q, Hq), -np.inf)
    row = 0
    for b in range(inp.batch):
        L, n, start = int(inp.seq_lens[b]), int(inp.q_lens[b]), int(inp.written_start[b])
        K = lib_decode(inp.logical_k[b], inp.kv_dtype) * ks
        V = lib_decode(inp.logical_v[b], inp.kv_dtype) * vs
        vis = visible_matrix(L, n, inp.window)
        for i in range(n):
            keys = [j for j in range(L) if vis[i, j] and key_lo[b] <= j < key_hi[b]]
            for h in range(Hq):
                if not keys:
                    continue
                g = h // G
                xs = [inp.softmax_scale * math.fsum(q[row + i, h] * K[j - start, g]) for j in keys]
                m = max(xs)
                e = [math.exp(x - m) for x in xs]
                den = math.fsum(e)
                for d in range(128):
                    out[row + i, h, d] = math.fsum(e[t] * V[keys[t] - start, g, d] for t in range(len(keys))) / den
                lse[row + i, h] = m + math.log(den)
        row += n
    return out, lse


CASES = [
    # seq_lens, q_lens, page, window, kv
    ([40, 9, 70], [3, 1, 5], 4, 0, "bf16"),
    ([33, 64], [2, 8], 16, 12, "fp8"),
    ([17], [17], 1, 0, "bf16"),
]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_partial_matches_brute_force(ci):
    L, n, P, W, kv = CASES[ci]
    inp = make_paged_inputs(600 + ci, seq_lens=L, q_lens=n, num_q_heads=4, num_kv_heads=2,
                            page_size=P, kv_dtype=kv, window=W, extra_pages=2)
    rng = np.random.default_rng(ci)
    lo = np.array([int(rng.integers(0, x)) for x in L])
    hi = np.array([int(rng.integers(l + 1, x + 1)) for l, x in zip(lo, L)])
    res = attention_partial(**partial_args(inp), key_lo=lo, key_hi=hi)
    out, lse = brute_partial(inp, lo, hi)
    np.testing.assert_allclose(res.out, out, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(np.isfinite(res.lse), np.isfinite(lse))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(res.lse[fin], lse[fin], rtol=1e-12, atol=1e-12)
    assert np.all(res.out[~fin] == 0.0)


@pytest.mark.parametrize("sinks,kv,P,W", [(True, "bf16", 16, 0), (False, "fp8", 1, 0),
                                          (True, "fp8", 8, 20), (True, "bf16", 128, 0)])
def test_partition_combines_to_the_unsplit_result(sinks, kv, P, W):
    """Cut every sequence's keys into parts (inside pages, on page edges, empty
    parts included); the combined partials equal the unsplit oracle."""
    L = [300, 129, 64, 1000]
    inp = make_paged_inputs(610, seq_lens=L, q_lens=[4, 1, 8, 3], num_q_heads=8, num_kv_heads=2,
                            page_size=P, kv_dtype=kv, window=W, sinks=sinks, extra_pages=3,
                            write_align=P if W > 0 else None)
    cuts = [[0, 100, 100, 128, 300], [0, 1, 64, 129, 129], [0, 0, 32, 33, 64], [0, 250, 600, 999, 1000]]
    outs, lses = [], []
    for s in range(4):
        lo = np.array([c[s] for c in cuts])
        hi = np.array([c[s + 1] for c in cuts])
        r = attention_partial(**partial_args(inp), key_lo=lo, key_hi=hi)
        outs.append(r.out)
        lses.append(r.lse)
    out, lse = combine_partials(outs, lses, inp.sinks)
    ref = paged_attention(**inp.oracle_kwargs())
    np.testing.assert_allclose(out, ref.out, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref.lse, rtol=1e-12, atol=1e-12)


def test_whole_range_is_attention_without_sink():
    inp = make_paged_inputs(620, seq_lens=[90, 200], q_lens=[6, 2], num_q_heads=4, num_kv_heads=1,
                            page_size=16, kv_dtype="bf16", sinks=True)
    r = attention_partial(**partial_args(inp), key_lo=[0, 0], key_hi=inp.seq_lens)
    a = inp.oracle_kwargs()
    a["sinks"] = None
    ref = paged_attention(**a)
    np.testing.assert_array_equal(r.out, ref.out)
    np.testing.assert_array_equal(r.lse, ref.lse)


def test_single_key_range_and_empty_rows():
    """A range holding one key gives that key's V row and score; rows whose
    causal limit lies before the range see nothing (0, -inf)."""
    inp = make_paged_inputs(630, seq_lens=[50], q_lens=[5], num_q_heads=2, num_kv_heads=1,
                            page_size=4, kv_dtype="bf16")
    r = attention_partial(**partial_args(inp), key_lo=[47], key_hi=[48])
    # tokens at positions 45..49: 45, 46 see no key in [47, 48); 47..49 see key 47 alone
    assert np.all(r.count[:2] == 0) and np.all(r.count[2:] == 1)
    assert np.all(r.out[:2] == 0.0) and np.all(np.isneginf(r.lse[:2]))
    V = lib_decode(inp.logical_v[0], "bf16")[47, 0]
    K = lib_decode(inp.logical_k[0], "bf16")[47, 0]
    q = lib_decode(inp.q, "bf16")
    for t in range(2, 5):
        for h in range(2):
            np.testing.assert_allclose(r.out[t, h], V, rtol=0, atol=1e-15)
            x = inp.softmax_scale * math.fsum(q[t, h] * K)
            assert abs(r.lse[t, h] - x) < 1e-12


def test_combine_closed_forms():
    rng = np.random.default_rng(3)
    o = rng.standard_normal((1, 5, 3, 128))
    l = rng.standard_normal((1, 5, 3))
    s = rng.standard_normal(3)
    # one part with a sink: out = o / (1 + e^(s - lse)), lse unchanged
    out, lse = combine_partials(o, l, s)
    np.testing.assert_allclose(out, o[0] / (1 + np.exp(s[None, :] - l[0]))[..., None], rtol=1e-13)
    np.testing.assert_allclose(lse, l[0], rtol=1e-13)
    # an empty part (-inf) changes nothing
    o2 = np.concatenate([o, np.zeros_like(o)])
    l2 = np.concatenate([l, np.full_like(l, -np.inf)])
    out2, lse2 = combine_partials(o2, l2, s)
    np.testing.assert_allclose(out2, out, rtol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13)
    # two equal parts: same output, lse + ln 2 (no sink)
    out3, lse3 = combine_partials(np.concatenate([o, o]), np.concatenate([l, l]))
    np.testing.assert_allclose(out3, o[0], rtol=1e-13)
    np.testing.assert_allclose(lse3, l[0] + math.log(2), rtol=1e-13)
