"""The debug build's device-side precondition checks (libdiffkv_attn_debug.so,
-DDIFFKV_DEBUG; diffkv_attn_debug_flags).

On valid inputs the debug library returns the release library's outputs bit
for bit and reports no violation.  Each broken precondition (a block-table
entry past the pool, a q_len above its seq_len, a seq_len above max_seq_len,
q_lens that do not add up to total_q) sets its bit, and packed rows outside
[0, total_q) are left unwritten.  Every violating case is laid out so that
even a missing check would stay inside memory the test allocated: spare pages
behind the pool, spare rows behind the block table, valid page ids in the
block table's unused entries, a violating q_len on a sequence other than the
first, and q / out tensors with rows beyond total_q.
"""

import numpy as np
import pytest
import torch

from paged_asymmetric_head_amd import binding as B
from paged_asymmetric_head_amd.device import DeviceInputs
from paged_asymmetric_head_amd.synth import make_paged_inputs

pytestmark = pytest.mark.gpu

Q_LEN, SEQ_LEN, PAGES, ROWS_TOTAL = 1, 2, 4, 8
SPARE_PAGES = 8


@pytest.fixture
def debug_library():
    B.select_library("debug")
    try:
        yield
    finally:
        B.select_library("release")


def take_flags():
    f = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    assert B.diffkv_attn_debug_flags(f) == B.OK
    torch.cuda.synchronize()
    return int(f.item())


class Case:
    """A small verify-shaped workload with room around it (spare pages,
    spare block-table rows, spare q / out rows) and valid page ids in every
    block-table entry."""

    def __init__(self, seed=5, kv_dtype="bf16", window=0):
        inp = make_paged_inputs(seed, seq_lens=[700, 1300, 520], q_lens=[8, 5, 8], num_q_heads=8,
                                num_kv_heads=1, page_size=16, kv_dtype=kv_dtype, sinks=True,
                                window=window, write_align=16 if window else None)
        self.inp = inp
        self.dev = DeviceInputs(inp)
        dev = self.dev
        pad = lambda t: torch.cat([t, torch.zeros((SPARE_PAGES,) + tuple(t.shape[1:]), dtype=t.dtype,
                                                   device=t.device)])
        self.k_cache, self.v_cache = pad(dev.k_cache), pad(dev.v_cache)
        bt = inp.block_table.astype(np.int32).copy()
        bt[bt < 0] = 0                                   # unused entries: a valid page
        bt = np.concatenate([bt, np.zeros((2, bt.shape[1]), np.int32)])   # spare rows
        self.bt = torch.from_numpy(bt).cuda()
        self.seq_lens = dev.seq_lens.clone()
        self.q_lens = dev.q_lens.clone()
        self.q = torch.cat([dev.q, torch.zeros_like(dev.q[:8])])           # spare rows
        self.total_q = inp.total_q

    def desc(self, splits):
        return self.dev.desc("verify", splits)

    def call(self, entry, d, out_rows=None):
        inp = self.inp
        rows = out_rows or self.q.shape[0]
        out = torch.full((rows, inp.num_q_heads, 128), 7.0, dtype=torch.bfloat16, device="cuda")
        nbytes = B.diffkv_attn_workspace_bytes(d, B.ENTRIES[entry])
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
        fn = {"verify": B.diffkv_attn_verify, "prefill": B.diffkv_attn_prefill,
              "mixed": B.diffkv_attn_mixed}[entry]
        fn(d, self.q, self.k_cache, self.v_cache, self.bt, self.seq_lens, self.q_lens, inp.window,
           self.dev.sinks, inp.k_scale, inp.v_scale, inp.softmax_scale, out, None, None,
           ws if nbytes else None, nbytes)
        torch.cuda.synchronize()
        return out


CALLS = [("verify", 3), ("verify", 1), ("prefill", 0), ("mixed", 0)]


@pytest.mark.parametrize("kv_dtype,window", [("bf16", 0), ("fp8", 0), ("fp8", 100)])
def test_valid_inputs_match_the_release_build_and_flag_nothing(kv_dtype, window):
    print(f"[gpu] debug build on valid inputs ({kv_dtype}, window {window})", flush=True)
    case = Case(kv_dtype=kv_dtype, window=window)
    release = [case.call(e, case.desc(s)) for e, s in CALLS]
    B.select_library("debug")
    try:
        take_flags()
        for (entry, splits), want in zip(CALLS, release):
            got = case.call(entry, case.desc(splits))
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (entry, splits)
            assert take_flags() == 0, (entry, splits)
    finally:
        B.select_library("release")


def run_flags(case, d, calls=CALLS):
    """Flags after each call, on the debug library."""
    take_flags()
    out = []
    for entry, splits in calls:
        d.force_num_splits = splits
        case.call(entry, d)
        out.append(take_flags())
    return out


def test_block_table_entry_past_the_pool_is_flagged(debug_library):
    print("[gpu] debug build: block-table entry past the pool", flush=True)
    case = Case()
    case.bt[1, 3] = case.inp.num_pages + 3                # a visible page; a spare page exists there
    for f in run_flags(case, case.desc(0)):
        assert f & PAGES, f


def test_block_table_entry_past_the_pool_is_flagged_in_a_short_window(debug_library):
    # A window of 100 keys spans at most three 64-key tiles: the one-chunk
    # launch's short-range pass reads the block table itself.
    print("[gpu] debug build: block-table entry past the pool, short window", flush=True)
    case = Case(window=100)
    case.bt[1, (1300 - 1) // 16] = case.inp.num_pages + 3    # the last page of sequence 1
    for f in run_flags(case, case.desc(0), calls=[("verify", 0)]):
        assert f & PAGES, f


def test_q_len_above_seq_len_is_flagged(debug_library):
    print("[gpu] debug build: q_len above seq_len", flush=True)
    case = Case()
    case.seq_lens[1] = 3                                  # q_lens[1] is 5
    for f in run_flags(case, case.desc(0)):
        assert f & Q_LEN, f


def test_seq_len_above_max_seq_len_is_flagged(debug_library):
    print("[gpu] debug build: seq_len above max_seq_len", flush=True)
    case = Case()
    d = case.desc(0)
    d.max_seq_len = 1000                                  # sequence 1 holds 1300 tokens
    for f in run_flags(case, d):
        assert f & SEQ_LEN, f


def test_rows_not_adding_up_are_flagged_and_rows_past_total_q_are_not_written(debug_library):
    print("[gpu] debug build: q_lens that do not add up to total_q", flush=True)
    case = Case()
    d = case.desc(0)
    d.total_q = case.total_q + 2                          # more rows than the q_lens give
    for f in run_flags(case, d):
        assert f & ROWS_TOTAL, f
    d = case.desc(0)
    d.total_q = case.total_q - 3                          # the last sequence's rows spill past it
    take_flags()
    for entry, splits in CALLS:
        d.force_num_splits = splits
        out = case.call(entry, d)
        assert take_flags() & ROWS_TOTAL, (entry, splits)
        tail = out[d.total_q:case.total_q].float()
        assert bool((tail == 7.0).all()), (entry, splits)     # never written


def test_release_build_reports_unsupported():
    f = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert B.diffkv_attn_debug_flags(f) == B.UNSUPPORTED
