"""GPU parity of the short-range pass (one-chunk launches whose pairs span at
most four 64-key tiles: every tile's loads at once, K straight into the MFMA
operands, one softmax update) against the FP64 oracle, at the edges of its
tile arithmetic: windows whose first key sits at offsets 0, 1, 62 and 63 of a
tile (three and four tiles), a window of one key, the widest span that still
fits four tiles, 16-token blocks at GQA 16 (sixteen 16-row query tiles per
pair), symmetric 128-wide heads, bf16 and FP8, pages of 1, 16 and 128.  The
pass is compiled for two, three and four tile slots (a pair of one tile takes
two, the second reading the zero row; three slots multiply the last tile's
keys alone); each count is covered in both formats.
Every row, its log-sum-exp and its visible-key count are compared."""

import pytest

from paged_asymmetric_head_amd.device import DeviceInputs
from paged_asymmetric_head_amd.synth import make_paged_inputs
from test_gpu_parity import check_call

pytestmark = pytest.mark.gpu


def window_case(off, W, n):
    """Sequence lengths whose window union starts at offset `off` of a tile."""
    return [64 * t + off + W + n - 1 for t in (10, 21, 3)]


CASES = [
    # (page, seq_lens, q_len, Hq, Hkv, window, sinks, kv, dqk)
    (1, window_case(0, 128, 4), 4, 8, 1, 128, True, "fp8", 192),
    (1, window_case(1, 128, 4), 4, 8, 1, 128, True, "fp8", 192),
    (16, window_case(62, 128, 4), 4, 8, 1, 128, True, "bf16", 192),
    (128, window_case(63, 128, 4), 4, 8, 1, 128, True, "fp8", 192),
    (16, window_case(5, 1, 1), 1, 4, 2, 1, False, "bf16", 192),
    (128, window_case(0, 256, 1), 1, 8, 1, 256, True, "bf16", 192),
    (16, window_case(40, 100, 16), 16, 16, 1, 100, True, "fp8", 192),
    (1, window_case(63, 128, 4), 4, 8, 2, 128, True, "fp8", 128),
    (16, [37, 200, 3, 256], 3, 8, 1, 0, False, "bf16", 128),
    # two tiles (sequences of 65-128 keys, no window), then three tiles in
    # bf16 and with 128-wide heads
    (128, [100, 90, 128, 65], 1, 8, 1, 0, True, "bf16", 192),
    (16, [70, 127, 66], 2, 8, 2, 0, False, "fp8", 192),
    (16, window_case(10, 128, 4), 4, 8, 1, 128, True, "bf16", 192),
    (1, window_case(20, 128, 4), 4, 8, 2, 128, False, "bf16", 128),
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{i}" for i in range(len(CASES))])
def test_short_range_pass_parity(case):
    P, L, n, Hq, Hkv, W, sinks, kv, dqk = case
    i = CASES.index(case)
    inp = make_paged_inputs(300 + i, seq_lens=L, q_lens=n, num_q_heads=Hq, num_kv_heads=Hkv,
                            page_size=P, kv_dtype=kv, window=W, sinks=sinks, extra_pages=3,
                            write_align=P if W > 0 else None, head_dim_qk=dqk)
    dev = DeviceInputs(inp)
    entries = (["decode"] if n == 1 else []) + ["verify"]
    for e in entries:
        check_call(dev, e, f"s{i}/{e}")
