"""FP64 CPU oracle for paged attention with asymmetric key/value head dims.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only the test-suite, the smoke check and the CPU-baseline
leg of the benchmark use it, to check and to time against.  It shares no code
with the HIP path; its only inputs are the arrays the seeded generator writes.

What it follows (the web pages this project is built from):
  * "sglang PR 41886, Default MiMo attention to FA4 on SM100", Accuracy Tests:
    QK head dim 192 / V head dim 128, full attention and sliding-window
    attention with sinks, decode and 8-token verify, ragged page boundaries.
  * "diffbot/MiMo-V2.6-Flash-RL-FP8KV-W4A8-2x-RTX-PRO-6000", What the kernels
    do: split-KV for verify, GQA groups of 16 query heads per KV head, FP8
    (E4M3) K/V converted when loaded.
  * "sglang PR 32818, Route asymmetric-KV models to fa4 on SM100": K and V
    live in separate paged caches because their row widths differ.

It also holds the paged KV write (kv_write.py): the new tokens' rows stored
into their slots, FP8 encoding from the format's definition.

Every function computes a plain definition in float64; no blocking or fusion
beyond what the definition states.  Pinned by the CPU tests against brute
force, a library attention routine, closed forms and invariants; the only
unpinned part is noted in `attention.py`.
"""

from .codecs import decode_bf16, decode_e4m3fn, encode_e4m3fn
from .attention import paged_attention, attention_partial, combine_partials, OracleResult
from .kv_write import paged_kv_write

__all__ = ["decode_bf16", "decode_e4m3fn", "encode_e4m3fn", "paged_attention", "attention_partial",
           "combine_partials", "OracleResult",
           "paged_kv_write"]
