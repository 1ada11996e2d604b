"""Seeded synthetic inputs for paged asymmetric-head attention.

This module only builds inputs: random draws, rounding to the storage formats
(bf16, FP8 E4M3FN with a per-tensor scale), the physical page permutation and
the block table.  It holds none of the attention arithmetic, so the HIP path
and the CPU oracle can both be fed from it without sharing any of the method.

Recipe (every workload):
  * independent child streams of numpy.random.SeedSequence(seed) for, in
    order, sequence lengths, the page permutation, Q, K, V and sinks, so the
    logical data does not depend on the page size;
  * normals from standard_normal(dtype=float32), rounded to bf16 by
    round-to-nearest-even, or quantised to FP8 E4M3FN with
    scale = max|x| / 448 over the tensor's written slots and
    code = RNE(clamp(x / scale, +-448));
  * both caches start filled with 0xFF bytes, which is NaN in bf16 and in
    E4M3FN, and only logical token slots are written, so every unused tail
    slot and unused page holds NaN;
  * physical pages are a seeded permutation of the pool; block-table entries
    past a sequence's last page are -1.
"""

from dataclasses import dataclass, field
import math

import numpy as np
import torch

HEAD_DIM_QK = 192
HEAD_DIM_V = 128
FP8_MAX = 448.0


@dataclass
class PagedInputs:
    name: str
    num_q_heads: int
    num_kv_heads: int
    page_size: int
    kv_dtype: str                 # "bf16" or "fp8"
    q: np.ndarray                 # uint16 [total_q, Hq, Dqk] (bf16 codes), Dqk 192 or 128
    k_cache: np.ndarray           # uint16|uint8 [pages, P, Hkv, Dqk]
    v_cache: np.ndarray           # uint16|uint8 [pages, P, Hkv, 128]
    block_table: np.ndarray       # int32 [B, stride]
    seq_lens: np.ndarray          # int32 [B]
    q_lens: np.ndarray            # int32 [B]
    window: int
    sinks: object                 # float32 [Hq] or None
    k_scale: float
    v_scale: float
    softmax_scale: float
    max_seq_len: int              # host-side bound used to size the launch
    max_q_len: int
    written_start: np.ndarray     # int64 [B]: first position holding data
    logical_k: list = field(default_factory=list)   # per seq: codes [L - start, Hkv, Dqk]
    logical_v: list = field(default_factory=list)   # per seq: codes [L - start, Hkv, 128]

    @property
    def batch(self):
        return int(self.seq_lens.shape[0])

    @property
    def total_q(self):
        return int(self.q_lens.sum())

    @property
    def num_pages(self):
        return int(self.k_cache.shape[0])

    @property
    def block_table_stride(self):
        return int(self.block_table.shape[1])

    def oracle_kwargs(self):
        """Keyword arguments in the oracle's vocabulary (plain arrays only)."""
        return dict(q=self.q, k_cache=self.k_cache, v_cache=self.v_cache,
                    block_table=self.block_table, seq_lens=self.seq_lens,
                    q_lens=self.q_lens, num_q_heads=self.num_q_heads,
                    num_kv_heads=self.num_kv_heads, kv_dtype=self.kv_dtype,
                    softmax_scale=self.softmax_scale, window=self.window,
                    sinks=self.sinks, k_scale=self.k_scale, v_scale=self.v_scale)


def to_bf16_bits(x):
    """float32 array -> bf16 codes (uint16), round to nearest even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def fp8_scale(arrays):
    """Per-tensor scale max|x| / 448 over the written slots (float32)."""
    amax = max((float(np.abs(a).max()) for a in arrays if a.size), default=0.0)
    return np.float32(amax / FP8_MAX) if amax > 0 else np.float32(1.0)


def to_e4m3fn_codes(x, scale):
    """float32 array -> E4M3FN codes (uint8): RNE(clamp(x / scale, +-448))."""
    y = np.clip(np.asarray(x, dtype=np.float32) / np.float32(scale), -FP8_MAX, FP8_MAX)
    return torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def make_paged_inputs(seed, *, seq_lens, q_lens, num_q_heads, num_kv_heads, page_size,
                      kv_dtype="bf16", window=0, sinks=False, softmax_scale=None,
                      extra_pages=0, block_table_stride=None, write_align=None,
                      max_seq_len=None, head_dim_qk=HEAD_DIM_QK, name="custom"):
    """Build one workload.

    seq_lens   list of ints, or (lo, hi) for integers uniform in [lo, hi]
               together with batch taken from q_lens when that is a list, or
               a list mixing ints and (lo, hi) pairs (one draw per pair).
    q_lens     int (same for every sequence) or list.
    head_dim_qk  key/query head dim (192, or 128 for symmetric heads); V is 128.
    write_align  with a window, positions before the start of the aligned
               block (of this many tokens) holding the window union's first
               key stay unwritten (NaN); otherwise every position is written.
    """
    ss = np.random.SeedSequence(seed)
    r_len, r_perm, r_q, r_k, r_v, r_sink = [np.random.default_rng(s) for s in ss.spawn(6)]

    if isinstance(seq_lens, tuple):
        if isinstance(q_lens, (list, np.ndarray)):
            batch = len(q_lens)
        else:
            raise ValueError("a (lo, hi) range needs q_lens as a list to fix the batch")
        lo, hi = seq_lens
        L = r_len.integers(lo, hi, size=batch, endpoint=True).astype(np.int64)
        bound = hi
    elif any(isinstance(x, tuple) for x in seq_lens):
        L = np.array([int(r_len.integers(x[0], x[1], endpoint=True)) if isinstance(x, tuple)
                      else int(x) for x in seq_lens], dtype=np.int64)
        batch = L.shape[0]
        bound = max(x[1] if isinstance(x, tuple) else int(x) for x in seq_lens)
    else:
        L = np.asarray(seq_lens, dtype=np.int64)
        batch = L.shape[0]
        bound = int(L.max())
    n = (np.full(batch, int(q_lens), dtype=np.int64) if np.isscalar(q_lens)
         else np.asarray(q_lens, dtype=np.int64))
    if np.any(n < 1) or np.any(n > L):
        raise ValueError("need 1 <= q_len <= seq_len for every sequence")
    if max_seq_len is None:
        max_seq_len = bound
    Hq, Hkv, P = int(num_q_heads), int(num_kv_heads), int(page_size)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(head_dim_qk)

    pages_per_seq = -(-L // P)
    num_pages = int(pages_per_seq.sum()) + int(extra_pages)
    perm = r_perm.permutation(num_pages).astype(np.int64)
    if block_table_stride is None:
        block_table_stride = -(-int(max_seq_len) // P)
    bt = np.full((batch, block_table_stride), -1, dtype=np.int32)
    off = 0
    for b in range(batch):
        k = int(pages_per_seq[b])
        bt[b, :k] = perm[off:off + k]
        off += k

    total_q = int(n.sum())
    q = to_bf16_bits(r_q.standard_normal((total_q, Hq, head_dim_qk), dtype=np.float32))

    W = int(window)
    start = np.zeros(batch, dtype=np.int64)
    if W > 0 and write_align:
        first_key = np.maximum(0, L - n - W + 1)
        start = (first_key // int(write_align)) * int(write_align)
    k_f = [r_k.standard_normal((int(L[b] - start[b]), Hkv, head_dim_qk), dtype=np.float32)
           for b in range(batch)]
    v_f = [r_v.standard_normal((int(L[b] - start[b]), Hkv, HEAD_DIM_V), dtype=np.float32)
           for b in range(batch)]
    if kv_dtype == "bf16":
        k_scale = v_scale = 1.0
        lk = [to_bf16_bits(a) for a in k_f]
        lv = [to_bf16_bits(a) for a in v_f]
        code_t = np.uint16
    elif kv_dtype == "fp8":
        k_scale = float(fp8_scale(k_f))
        v_scale = float(fp8_scale(v_f))
        lk = [to_e4m3fn_codes(a, k_scale) for a in k_f]
        lv = [to_e4m3fn_codes(a, v_scale) for a in v_f]
        code_t = np.uint8
    else:
        raise ValueError(f"unknown kv dtype {kv_dtype!r}")
    del k_f, v_f

    nan_code = np.iinfo(code_t).max          # 0xFFFF bf16 NaN, 0xFF E4M3FN NaN
    k_cache = np.full((num_pages, P, Hkv, head_dim_qk), nan_code, dtype=code_t)
    v_cache = np.full((num_pages, P, Hkv, HEAD_DIM_V), nan_code, dtype=code_t)
    for b in range(batch):
        pos = np.arange(start[b], L[b], dtype=np.int64)
        pages = bt[b, pos // P].astype(np.int64)
        slots = pos % P
        k_cache[pages, slots] = lk[b]
        v_cache[pages, slots] = lv[b]

    sink_vals = r_sink.standard_normal(Hq, dtype=np.float32) if sinks else None

    return PagedInputs(name=name, num_q_heads=Hq, num_kv_heads=Hkv, page_size=P,
                       kv_dtype=kv_dtype, q=q, k_cache=k_cache, v_cache=v_cache,
                       block_table=bt, seq_lens=L.astype(np.int32), q_lens=n.astype(np.int32),
                       window=W, sinks=sink_vals, k_scale=k_scale, v_scale=v_scale,
                       softmax_scale=float(softmax_scale), max_seq_len=int(max_seq_len),
                       max_q_len=int(n.max()), written_start=start, logical_k=lk, logical_v=lv)


# The workloads the path is measured and checked on.  Head counts are one
# GPU's share of a layer; the page size, K/V format, window and sinks follow the
# serving setups on the pages (page 128 and page 1 caches, FP8 E4M3 K/V,
# sliding-window layers with sinks, 8-token verify, 4096-token prefill chunks
# at 26K context).
WORKLOADS = {
    # 2 sequences (37 and 300 tokens), 32 pages of 16 under a permutation.
    "tiny_decode": dict(seed=1, seq_lens=[37, 300], q_lens=1, num_q_heads=4, num_kv_heads=1,
                        page_size=16, kv_dtype="bf16", extra_pages=10),
    # 32 sequences of 8192..9216 tokens, one KV head with 8 query heads.
    "batched_decode": dict(seed=2, seq_lens=(8192, 9216), q_lens=[1] * 32, num_q_heads=8,
                           num_kv_heads=1, page_size=128, kv_dtype="bf16"),
    # 4 sequences of 40000..50000 tokens, 8-token causal verify block.
    "verify_long": dict(seed=3, seq_lens=(40000, 50000), q_lens=[8] * 4, num_q_heads=8,
                        num_kv_heads=1, page_size=128, kv_dtype="bf16"),
    # 64 sequences of 8192..102400 tokens, 4-token verify, window 128, sinks,
    # FP8 K/V; page size 1 and 128 see the same logical data.
    "swa_sinks_fp8_p1": dict(seed=4, seq_lens=(8192, 102400), q_lens=[4] * 64, num_q_heads=8,
                             num_kv_heads=1, page_size=1, kv_dtype="fp8", window=128,
                             sinks=True, block_table_stride=102400, write_align=128),
    "swa_sinks_fp8_p128": dict(seed=4, seq_lens=(8192, 102400), q_lens=[4] * 64, num_q_heads=8,
                               num_kv_heads=1, page_size=128, kv_dtype="fp8", window=128,
                               sinks=True, block_table_stride=800, write_align=128),
    # One sequence: 4096 new tokens after 26624 cached, GQA 32/2, FP8 K/V.
    "chunked_prefill": dict(seed=5, seq_lens=[30720], q_lens=4096, num_q_heads=32,
                            num_kv_heads=2, page_size=128, kv_dtype="fp8"),
    # Symmetric 128/128 heads at the batched-decode shape.
    "batched_decode_sym": dict(seed=7, seq_lens=(8192, 9216), q_lens=[1] * 32, num_q_heads=8,
                               num_kv_heads=1, page_size=128, kv_dtype="bf16", head_dim_qk=128),
    # One serving step mixing the three kinds of sequence at the prefill
    # chunk's head shape (GQA 32/2, page 128, FP8 K/V): the 4096-token chunk
    # at 26K context, 4 verify blocks of 8 at 40000..50000 tokens and 32
    # decodes at 8192..9216 tokens.
    "mixed_batch": dict(seed=6, seq_lens=[30720] + [(40000, 50000)] * 4 + [(8192, 9216)] * 32,
                        q_lens=[4096] + [8] * 4 + [1] * 32, num_q_heads=32, num_kv_heads=2,
                        page_size=128, kv_dtype="fp8"),
}


def workload(name):
    return make_paged_inputs(name=name, **WORKLOADS[name])
