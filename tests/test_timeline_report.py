"""The timeline module's tables (paged_asymmetric_head_amd/timeline.py) on
synthetic stamps: percentiles per point, the span of each call and the
per-XCD means come out of known inputs.  CPU only."""

import numpy as np

from paged_asymmetric_head_amd.timeline import PHASES, report


def test_report_on_known_stamps():
    # Two calls, 16 workgroups each; workgroup w starts at w * 0.1 us and
    # passes point k at start + k us, except point 5, which none passes.
    runs = []
    for call in range(2):
        wg = np.arange(16)
        rel = np.array([[w * 0.1 + k if k != 5 else np.nan for k in range(8)] for w in wg])
        runs.append((rel, wg))
    text = report("synthetic", runs)
    lines = text.splitlines()
    assert lines[0] == "### synthetic: 2 calls, 32 workgroup records"
    row = {ln.split("|")[1].strip(): [c.strip() for c in ln.split("|")[2:-1]] for ln in lines if ln.startswith("| ")}
    # 32 starts (0.0, 0.0, 0.1, 0.1, ..., 1.5, 1.5), linear interpolation
    # between order statistics: p10 at rank 3.1 -> 0.11, p50 at 15.5 -> 0.75,
    # p90 at 27.9 -> 1.39.
    assert row["0 start"] == ["0.00", "0.11", "0.75", "1.39", "1.50"]
    assert row["7 output stores issued"][0] == "7.00" and row["7 output stores issued"][-1] == "8.50"
    assert row["5 last round of the tile loop"] == ["-"] * 5
    assert row["span of the call (last store issued)"] == ["8.50"] * 5
    # XCD x holds workgroups x and x + 8: mean start (x + x + 8) * 0.1 / 2.
    assert row["mean start"] == [f"{(2 * x + 8) * 0.05:.2f}" for x in range(8)]
    assert row["mean from first data to stores"] == ["4.00"] * 8
    assert [k for k, _ in PHASES] == list(range(8))
