"""Brute-force dense attention on tiny inputs, for pinning the oracle.

It works on the generator's logical (pre-paging) per-sequence arrays and never
sees the page pool or the block table.  Codes are decoded with torch's own
bfloat16 / float8_e4m3fn types (a library decoder, not the oracle's), the mask
is an explicit boolean matrix and every sum is math.fsum over Python floats.
"""

import math

import numpy as np
import torch


def lib_decode(codes, kv_dtype):
    t = torch.from_numpy(np.ascontiguousarray(codes))
    if kv_dtype == "bf16":
        return t.view(torch.bfloat16).double().numpy()
    return t.view(torch.float8_e4m3fn).double().numpy()


def visible_matrix(L, n, window):
    """mask[i][j] for new token i of n and key position j < L."""
    m = np.zeros((n, L), dtype=bool)
    for i in range(n):
        p = L - n + i
        for j in range(L):
            m[i, j] = j <= p and (window <= 0 or p - j < window)
    return m


def brute_force(inp):
    """Returns out [total_q, Hq, Dv], lse [total_q, Hq], count [total_q, Hq]."""
    Hq, Hkv = inp.num_q_heads, inp.num_kv_heads
    G = Hq // Hkv
    total_q = inp.total_q
    Dv = inp.logical_v[0].shape[-1]
    out = np.zeros((total_q, Hq, Dv))
    lse = np.zeros((total_q, Hq))
    cnt = np.zeros((total_q, Hq), dtype=np.int64)
    q = torch.from_numpy(np.ascontiguousarray(inp.q)).view(torch.bfloat16).double().numpy()
    ks = inp.k_scale if inp.kv_dtype == "fp8" else 1.0
    vs = inp.v_scale if inp.kv_dtype == "fp8" else 1.0
    row = 0
    for b in range(inp.batch):
        L, n, start = int(inp.seq_lens[b]), int(inp.q_lens[b]), int(inp.written_start[b])
        K = lib_decode(inp.logical_k[b], inp.kv_dtype) * ks      # [L - start, Hkv, Dqk]
        V = lib_decode(inp.logical_v[b], inp.kv_dtype) * vs
        vis = visible_matrix(L, n, inp.window)
        for i in range(n):
            for h in range(Hq):
                g = h // G
                keys = [j for j in range(L) if vis[i, j]]
                assert keys and min(keys) >= start, "a visible key has no data"
                # Products of decoded codes are exact in float64; fsum rounds once.
                xs = [inp.softmax_scale * math.fsum(q[row + i, h] * K[j - start, g])
                      for j in keys]
                m = max(xs)
                if inp.sinks is not None:
                    m = max(m, float(inp.sinks[h]))
                es = [math.exp(x - m) for x in xs]
                ksum = math.fsum(es)
                den = ksum + (math.exp(float(inp.sinks[h]) - m) if inp.sinks is not None else 0.0)
                Vk = np.stack([V[j - start, g] for j in keys])          # [nk, Dv]
                ev = np.asarray(es)
                for d in range(Dv):
                    out[row + i, h, d] = math.fsum(ev * Vk[:, d]) / den
                lse[row + i, h] = m + math.log(ksum)
                cnt[row + i, h] = len(keys)
        row += n
    return out, lse, cnt
