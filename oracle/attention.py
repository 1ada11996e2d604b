"""Paged attention with asymmetric head dims, computed from its definition in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition (one query head h, one new query token; the readings of points the
pages leave open are listed after it):

  For sequence b with L = seq_lens[b] cached tokens (the new tokens included)
  and n = q_lens[b] new tokens starting at packed row r0 = sum(q_lens[:b]),
  new token i in [0, n) sits at position p = L - n + i.
  Query head h reads KV head g = h // G with G = Hq / Hkv (contiguous GQA
  groups; "diffbot/MiMo-V2.6-Flash-RL-FP8KV-W4A8-2x-RTX-PRO-6000", What the
  kernels do, groups 16 query heads per KV head).
  Visible keys: lo <= j <= p, with lo = 0 for full attention and
  lo = max(0, p - W + 1) for a sliding window of W tokens (the token itself
  included); causal within the verify block ("sglang PR 41886", Accuracy
  Tests: full attention and SWA with sinks, decode, 8-token verify).
  Key j lives in physical page block_table[b][j // P] at slot j % P; K and V
  sit in two separate caches because their row widths differ (192 vs 128,
  "sglang PR 32818", the trtllm_mha failure it fixes).
      K_j = dec(k_cache[page, slot, g, :]) * k_scale     (192 values)
      V_j = dec(v_cache[page, slot, g, :]) * v_scale     (128 values)
  The scales multiply only FP8 caches (per-tensor dequantisation); bf16
  caches are used as stored.
      x_j = softmax_scale * sum_d q[r0 + i, h, d] * K_j[d]
      m   = max(max_j x_j, s_h)         (s_h only when sinks are given)
      den = sum_j exp(x_j - m) + exp(s_h - m)
      out = sum_j exp(x_j - m) V_j / den
      lse = m + ln sum_j exp(x_j - m)     (keys only; the sink is excluded)
      count = number of visible keys

Readings where the pages are silent (each the plainest one the text allows):
  * seq_lens counts the new tokens, whose K/V are already in the cache.
  * the verify mask is plain causal (linear draft chains, no trees).
  * a window of W keeps the W newest keys including the token itself;
    W <= 0 means full attention.
  * a sink s_h is one fp32 logit per query head in the already-scaled logit
    domain; it adds exp(s_h) to the denominator only and carries no value.
  * lse uses the natural log and excludes the sink.
Parity unpinned: the bf16 rounding pattern of a GPU output (compared within
the tolerance only); the window and sink conventions above are readings, not
statements of the pages.

Context split ("diffbot/...", What the kernels do: split-KV; cut across
GPUs, each GPU holding a range of a sequence's keys): `key_range` keeps only
the keys key_lo[b] <= j < key_hi[b] of sequence b visible; `attention_partial`
evaluates that restriction without the sink and returns each row's
normalised output (0 where no key is visible) and its log-sum-exp (-inf
there); `combine_partials` merges partials of disjoint key ranges by
log-sum-exp, the sink joining the merged denominator once, which gives the
unsplit result.

Split mode (`split=k` or `split="page"`) evaluates the same rows by cutting
each (sequence, KV head) key range into pieces, computing (max, sum, output)
per piece and merging by log-sum-exp, as split-KV does ("diffbot/...", What
the kernels do: split-KV for the verify step).  It exists to pin the merge
arithmetic; the result must equal the unsplit one to rounding.
"""

from dataclasses import dataclass

import numpy as np

from .codecs import decode_bf16, decode_e4m3fn


@dataclass
class OracleResult:
    out: np.ndarray     # float64 [T, Hq, Dv]
    lse: np.ndarray     # float64 [T, Hq]
    count: np.ndarray   # int64   [T, Hq]
    tokens: np.ndarray  # int64   [T], the packed query-token rows computed


def _decode_cache(raw, kv_dtype, scale):
    if kv_dtype == "bf16":
        return decode_bf16(raw)
    if kv_dtype == "fp8":
        return decode_e4m3fn(raw) * float(scale)
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")


def _piece_edges(j0, j1, split, page_size):
    """Edges of the key pieces over the inclusive range [j0, j1]."""
    if split is None:
        return np.array([j0, j1 + 1], dtype=np.int64)
    if split == "page":
        inner = np.arange((j0 // page_size + 1) * page_size, j1 + 1, page_size, dtype=np.int64)
        return np.concatenate([[j0], inner, [j1 + 1]]).astype(np.int64)
    k = int(split)
    if k < 1:
        raise ValueError("split must be >= 1")
    return np.round(np.linspace(j0, j1 + 1, k + 1)).astype(np.int64)


def _sum_visible(e, vis, V):
    """sum_j e[a, g, j] * V[j, :] over the keys j that row a sees (vis[a, j]).

    A key a row does not see adds nothing, not even 0 * NaN: value entries
    that are not finite are summed over the visible keys alone.
    """
    finite = np.isfinite(V)
    o = np.matmul(e, np.where(finite, V, 0.0))
    for d in np.flatnonzero(~finite.all(axis=0)):
        with np.errstate(invalid="ignore"):
            o[..., d] = np.where(vis[:, None, :], e * V[None, None, :, d], 0.0).sum(axis=2)
    return o


def _direct(x, vis, V, s_h):
    """The definition itself: one max, one denominator, one weighted sum.

    x [ni, G, nj] scaled scores with invisible keys at -inf; vis [ni, nj] the
    visible keys; V [nj, Dv]; s_h [G] sink logits or None.  A NaN score of a
    visible key stays NaN and reaches the output, as in the definition.
    """
    m = x.max(axis=2)                                                # [ni, G]; NaN propagates
    if s_h is not None:
        m = np.maximum(m, s_h[None, :])
    with np.errstate(invalid="ignore"):
        e = np.where(vis[:, None, :], np.exp(x - m[:, :, None]), 0.0)
    key_sum = e.sum(axis=2)
    den = key_sum + (0.0 if s_h is None else np.exp(s_h[None, :] - m))
    o = _sum_visible(e, vis, V) / den[:, :, None]
    with np.errstate(divide="ignore"):
        return o, m + np.log(key_sum)


def _pieces_merged(x, vis, V, s_h, edges):
    """Split-KV evaluation: per piece (max, sum, normalised output), merged by
    log-sum-exp with the sink joining the merged denominator."""
    piece_lse, piece_out = [], []
    for e0, e1 in zip(edges[:-1], edges[1:]):
        if e1 <= e0:
            continue
        xs = x[:, :, e0:e1]
        vs = vis[:, e0:e1]
        m = xs.max(axis=2)                                            # -inf if none visible
        m_safe = np.where(m == -np.inf, 0.0, m)
        with np.errstate(invalid="ignore"):
            w = np.where(vs[:, None, :], np.exp(xs - m_safe[:, :, None]), 0.0)
        l = w.sum(axis=2)
        o = _sum_visible(w, vs, V[e0:e1])
        with np.errstate(invalid="ignore", divide="ignore"):
            piece_out.append(np.where(l[:, :, None] == 0, 0.0, o / l[:, :, None]))
            piece_lse.append(np.where(l == 0, -np.inf, m_safe + np.log(l)))
    pl = np.stack(piece_lse)                                          # [S, ni, G]
    po = np.stack(piece_out)                                          # [S, ni, G, Dv]
    M = pl.max(axis=0)
    if s_h is not None:
        M = np.maximum(M, s_h[None, :])
    with np.errstate(invalid="ignore"):
        wts = np.where(pl == -np.inf, 0.0, np.exp(pl - M[None]))      # empty pieces only
    key_sum = wts.sum(axis=0)
    den = key_sum + (0.0 if s_h is None else np.exp(s_h[None, :] - M))
    o = (wts[..., None] * po).sum(axis=0) / den[..., None]
    with np.errstate(divide="ignore"):
        return o, M + np.log(key_sum)


def paged_attention(q, k_cache, v_cache, block_table, seq_lens, q_lens=None, *,
                    num_q_heads, num_kv_heads, kv_dtype, softmax_scale,
                    window=0, sinks=None, k_scale=1.0, v_scale=1.0,
                    tokens=None, split=None, key_range=None, max_chunk_elems=1 << 22):
    """Evaluate the definition above.

    q            uint16 [total_q, Hq, Dqk]         bf16 codes
    k_cache      uint16|uint8 [pages, P, Hkv, Dqk] bf16 codes or E4M3FN codes
    v_cache      uint16|uint8 [pages, P, Hkv, Dv]
    block_table  int   [B, stride]
    seq_lens     int   [B]
    q_lens       int   [B] or None (all 1)
    sinks        float [Hq] or None
    tokens       optional iterable of packed query rows to compute (default all)
    key_range    optional (key_lo [B], key_hi [B]): only keys key_lo[b] <= j <
                 key_hi[b] stay visible (a row may then see none)
    """
    q = np.asarray(q)
    k_cache = np.asarray(k_cache)
    v_cache = np.asarray(v_cache)
    block_table = np.asarray(block_table)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    B = seq_lens.shape[0]
    q_lens = np.ones(B, dtype=np.int64) if q_lens is None else np.asarray(q_lens, dtype=np.int64)
    Hq, Hkv = int(num_q_heads), int(num_kv_heads)
    if Hq % Hkv != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    num_pages, P = k_cache.shape[0], k_cache.shape[1]
    Dqk, Dv = k_cache.shape[3], v_cache.shape[3]
    total_q = int(q_lens.sum())
    if q.shape != (total_q, Hq, Dqk):
        raise ValueError(f"q shape {q.shape} != {(total_q, Hq, Dqk)}")
    W = int(window)
    sink = None if sinks is None else np.asarray(sinks, dtype=np.float64)

    starts = np.concatenate([[0], np.cumsum(q_lens)[:-1]]).astype(np.int64)
    if tokens is None:
        want = np.arange(total_q, dtype=np.int64)
    else:
        want = np.unique(np.asarray(tokens, dtype=np.int64))
    T = want.shape[0]
    out = np.full((T, Hq, Dv), np.nan)
    lse = np.full((T, Hq), np.nan)
    count = np.zeros((T, Hq), dtype=np.int64)
    row_of = {int(t): r for r, t in enumerate(want)}

    for b in range(B):
        L, n, r0 = int(seq_lens[b]), int(q_lens[b]), int(starts[b])
        if not (1 <= n <= L):
            raise ValueError(f"sequence {b}: need 1 <= q_len ({n}) <= seq_len ({L})")
        local = np.array([t - r0 for t in want if r0 <= t < r0 + n], dtype=np.int64)
        if local.size == 0:
            continue
        p_all = L - n + local
        lo_all = np.maximum(0, p_all - W + 1) if W > 0 else np.zeros_like(p_all)
        if key_range is not None:
            klo, khi = int(key_range[0][b]), int(key_range[1][b])
            lo_all = np.maximum(lo_all, klo)
            p_all = np.minimum(p_all, khi - 1)
            if int((p_all - lo_all).max()) < 0:      # no token of this sequence sees a key
                for t in local:
                    r = row_of[int(r0 + t)]
                    count[r, :] = 0
                continue

        # Union key range of the requested tokens; only its pages are read.
        j0, j1 = int(lo_all.min()), int(p_all.max())
        j = np.arange(j0, j1 + 1, dtype=np.int64)
        page_index = j // P
        phys = block_table[b, page_index].astype(np.int64)
        if phys.min() < 0 or phys.max() >= num_pages:
            raise ValueError(f"sequence {b}: block-table entry out of range for a visible page")
        slot = j % P

        # Rows per chunk so one score block stays near max_chunk_elems values.
        per_tok = max(1, G * j.size)
        step = max(1, max_chunk_elems // per_tok)
        edges = _piece_edges(j0, j1, split, P) - j0

        for g in range(Hkv):
            K = _decode_cache(k_cache[phys, slot, g, :], kv_dtype, k_scale)   # [nj, Dqk]
            V = _decode_cache(v_cache[phys, slot, g, :], kv_dtype, v_scale)   # [nj, Dv]
            heads = np.arange(g * G, (g + 1) * G)
            s_h = None if sink is None else sink[heads]                     # [G]
            for c0 in range(0, local.size, step):
                li = local[c0:c0 + step]
                p = p_all[c0:c0 + step]
                lo = lo_all[c0:c0 + step]
                Q = decode_bf16(q[r0 + li][:, heads, :])                      # [ni, G, Dqk]
                vis = (j[None, :] >= lo[:, None]) & (j[None, :] <= p[:, None])  # [ni, nj]
                x = softmax_scale * np.matmul(Q, K.T)                        # [ni, G, nj]
                x = np.where(vis[:, None, :], x, -np.inf)

                if split is None:
                    o, row_lse = _direct(x, vis, V, s_h)
                else:
                    o, row_lse = _pieces_merged(x, vis, V, s_h, edges)

                cnt = vis.sum(axis=1)
                for a, t in enumerate(li):
                    r = row_of[int(r0 + t)]
                    out[r, heads, :] = o[a]
                    lse[r, heads] = row_lse[a]
                    count[r, heads] = cnt[a]
    return OracleResult(out=out, lse=lse, count=count, tokens=want)


def attention_partial(q, k_cache, v_cache, block_table, seq_lens, q_lens=None, *, key_lo, key_hi,
                      num_q_heads, num_kv_heads, kv_dtype, softmax_scale, window=0, k_scale=1.0,
                      v_scale=1.0, tokens=None):
    """One key range's share of every row: the definition restricted to the keys
    key_lo[b] <= j < key_hi[b], without the sink.  Returns an OracleResult whose
    out is the normalised partial output (0 for a row that sees no key in the
    range) and lse its natural log-sum-exp (-inf there)."""
    with np.errstate(invalid="ignore", divide="ignore"):
        res = paged_attention(q, k_cache, v_cache, block_table, seq_lens, q_lens,
                              num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                              kv_dtype=kv_dtype, softmax_scale=softmax_scale, window=window,
                              sinks=None, k_scale=k_scale, v_scale=v_scale, tokens=tokens,
                              key_range=(np.asarray(key_lo), np.asarray(key_hi)))
    empty = res.count == 0
    res.out[empty] = 0.0
    res.lse[empty] = -np.inf
    return res


def combine_partials(outs, lses, sinks=None):
    """Merge partials of disjoint key ranges of the same rows.

    outs [S, T, Hq, Dv] normalised partial outputs, lses [S, T, Hq] their
    log-sum-exp (-inf for a part with no key), sinks [Hq] or None.  With
    M = max(max_s lse_s, s_h) and w_s = exp(lse_s - M):
        out = sum_s w_s out_s / (sum_s w_s + exp(s_h - M))
        lse = M + ln sum_s w_s          (keys only)
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    M = lses.max(axis=0)
    if sinks is not None:
        M = np.maximum(M, np.asarray(sinks, dtype=np.float64)[None, :])
    with np.errstate(invalid="ignore"):
        w = np.where(lses == -np.inf, 0.0, np.exp(lses - M[None]))   # empty parts only
    key_sum = w.sum(axis=0)
    den = key_sum + (0.0 if sinks is None else np.exp(np.asarray(sinks, dtype=np.float64)[None, :] - M))
    out = (w[..., None] * outs).sum(axis=0) / den[..., None]
    with np.errstate(divide="ignore"):
        return out, M + np.log(key_sum)
