"""Shared checks for the GPU parity tests: the tolerance and the comparisons.

Tolerance (over the whole output of one call): max |gpu - oracle| <= 1e-2 and
||gpu - oracle||_2 / ||oracle||_2 <= 5e-3; any non-finite value fails.  FP8
caches are compared on the same dequantised values (the oracle decodes the
same codes with the same per-tensor scales).
"""

import numpy as np

MAX_ABS = 1e-2
REL_L2 = 5e-3


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def compare(gpu, ref, tag=""):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{tag}: non-finite GPU output"
    err = np.abs(g - r)
    max_abs = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
    print(f"[parity] {tag}: max_abs={max_abs:.3e} rel_l2={rel:.3e}", flush=True)
    assert max_abs <= MAX_ABS, f"{tag}: max_abs {max_abs}"
    assert rel <= REL_L2, f"{tag}: rel_l2 {rel}"
    return max_abs, rel


def expected_counts(inp):
    """Visible keys per (token, head), from the definition of the mask."""
    rows = []
    for b in range(inp.batch):
        L, n = int(inp.seq_lens[b]), int(inp.q_lens[b])
        p = L - n + np.arange(n)
        c = p + 1 if inp.window <= 0 else np.minimum(p + 1, inp.window)
        rows.append(c)
    c = np.concatenate(rows)
    return np.repeat(c[:, None], inp.num_q_heads, axis=1)
