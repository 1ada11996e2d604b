"""GPU parity of the balanced split plan: batches whose sequences differ
widely in length, so some (sequence, query tile) pairs get one chunk (written
directly, skipped by the merge) and others many, and batches of more than 64
sequences (the plan walks the batch 64 sequences per pass), and batches whose
chunks are lengthened to fit one resident round.  count_out checks that every
visible key is combined exactly once.
"""

import numpy as np
import pytest

from paged_asymmetric_head_amd.device import DeviceInputs
from paged_asymmetric_head_amd.synth import make_paged_inputs
from test_gpu_parity import check_call

pytestmark = pytest.mark.gpu


def test_heterogeneous_decode_lengths():
    lens = [20000, 100, 64, 5000, 1, 700, 12000, 65]
    inp = make_paged_inputs(401, seq_lens=lens, q_lens=1, num_q_heads=8, num_kv_heads=1,
                            page_size=16, kv_dtype="bf16", sinks=True)
    check_call(DeviceInputs(inp), "decode", "heterogeneous decode")


@pytest.mark.parametrize("batch,entry", [(100, "verify"), (130, "decode")])
def test_batches_over_64_sequences(batch, entry):
    rng = np.random.default_rng(402 + batch)
    lens = [int(x) for x in rng.integers(20, 3000, batch)]
    q = 1 if entry == "decode" else [int(x) for x in rng.integers(1, 17, batch)]
    if entry == "verify":
        lens = [max(l, n) for l, n in zip(lens, q)]
    inp = make_paged_inputs(403 + batch, seq_lens=lens, q_lens=q, num_q_heads=4, num_kv_heads=2,
                            page_size=16, kv_dtype="fp8", window=0, sinks=False)
    check_call(DeviceInputs(inp), entry, f"{batch} sequences")


def test_mixed_with_long_sequences_between_short_ones():
    lens = [5000, 900, 30, 7000, 300, 64]
    q = [1, 200, 16, 8, 40, 1]
    inp = make_paged_inputs(404, seq_lens=lens, q_lens=q, num_q_heads=16, num_kv_heads=2,
                            page_size=128, kv_dtype="bf16", window=512, sinks=True,
                            write_align=128)
    check_call(DeviceInputs(inp), "mixed", "mixed heterogeneous")


@pytest.mark.parametrize("batch,seed,lo,hi,hq,hkv,page", [(48, 39, 2000, 6000, 8, 1, 128),
                                                         (100, 1, 500, 3000, 4, 2, 16)],
                         ids=["one_pass", "two_passes"])
def test_chunks_lengthened_to_fit_one_round(batch, seed, lo, hi, hq, hkv, page):
    """Lengths whose per-pair rounding gives more chunks than the slots of one
    resident round (534 for 512 with 48 sequences; 300 for 256 per KV head
    with 100 sequences, whose check runs in the plan's multi-pass count): the
    plan lengthens the chunks until they fit, and every workgroup and the
    merge must agree on the lengthened plan."""
    lens = [int(x) for x in np.random.default_rng(seed).integers(lo, hi, size=batch)]
    inp = make_paged_inputs(405 + batch, seq_lens=lens, q_lens=1, num_q_heads=hq, num_kv_heads=hkv,
                            page_size=page, kv_dtype="bf16", sinks=True)
    check_call(DeviceInputs(inp), "decode", f"{batch} sequences, chunks fitted to one round")


def test_verify_over_the_one_slot_bound():
    """A bf16 verify batch (64-row tiles) whose host bound exceeds 16 tiles per
    one-per-CU chunk, so the plan takes two workgroups per CU."""
    lens = [int(x) for x in np.random.default_rng(406).integers(20000, 24000, size=12)]
    inp = make_paged_inputs(407, seq_lens=lens, q_lens=8, num_q_heads=8, num_kv_heads=1,
                            page_size=128, kv_dtype="bf16", sinks=False)
    check_call(DeviceInputs(inp), "verify", "verify over the one-slot bound")
