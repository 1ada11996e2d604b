"""Paged KV write: the new tokens' K and V rows stored into their cache slots.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The FP8 KV cache of the "diffbot/MiMo-V2.6-Flash-RL-FP8KV-W4A8-2x-RTX-PRO-6000"
page (intro: the E4M3 KV cache that doubles the pool) is filled one step
before attention reads it: each new token's K (192 wide) and V (128 wide)
rows go to the slot its position maps to through the block table ("sglang PR
41886, Default MiMo attention to FA4 on SM100", paged caches with ragged page
boundaries; "sglang PR 32818", separate K and V caches of different widths).

For sequence b (L = seq_lens[b] tokens including its n = q_lens[b] new ones,
packed rows starting at r0 = q_lens[0] + ... + q_lens[b-1]) and new token i,
the position is p = L - n + i and, for KV head g,

    k_cache[block_table[b][p // P], p % P, g, :] = enc(k_new[r0 + i, g, :] / k_scale)
    v_cache[block_table[b][p // P], p % P, g, :] = enc(v_new[r0 + i, g, :] / v_scale)

with enc the identity for bf16 caches (no scale) and, for FP8 caches, E4M3FN
round-to-nearest-even after clamping to +-448 (codecs.encode_e4m3fn).  The
division is taken in float32: it decides an integer code, so the oracle and
the kernel take it in the same precision (the kernel's; the pages give none).
Nothing else in the caches changes.
"""

import numpy as np

from .codecs import decode_bf16, encode_e4m3fn


def paged_kv_write(k_new, v_new, k_cache, v_cache, block_table, seq_lens, q_lens, *, kv_dtype,
                   k_scale=1.0, v_scale=1.0):
    """Copies of (k_cache, v_cache) with every new token's rows stored.

    k_new, v_new: bf16 codes (uint16) [total_q, Hkv, 192] and [total_q, Hkv, 128].
    Caches: uint16 (bf16) or uint8 (E4M3FN codes) [pages, P, Hkv, width].
    Raises if a position maps to a block-table entry outside the pool.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    P = kc.shape[1]
    n_pages = kc.shape[0]
    ks = np.float32(k_scale)
    vs = np.float32(v_scale)
    r0 = 0
    for b in range(len(seq_lens)):
        L, n = int(seq_lens[b]), int(q_lens[b])
        for i in range(n):
            p = L - n + i
            page = int(block_table[b][p // P])
            if not 0 <= page < n_pages:
                raise ValueError(f"sequence {b} position {p}: block-table entry {page} out of range")
            slot = p % P
            if kv_dtype == "bf16":
                kc[page, slot] = k_new[r0 + i]
                vc[page, slot] = v_new[r0 + i]
            else:
                # A quotient may overflow to +-inf (a large value over a small
                # scale); the encoder clamps it to +-448.
                with np.errstate(over="ignore"):
                    k = decode_bf16(k_new[r0 + i]).astype(np.float32) / ks
                    v = decode_bf16(v_new[r0 + i]).astype(np.float32) / vs
                kc[page, slot] = encode_e4m3fn(k)
                vc[page, slot] = encode_e4m3fn(v)
        r0 += n
    return kc, vc
