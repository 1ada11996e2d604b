"""The oracle evaluated over many query tokens at once, on every host core.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Every output row of `paged_attention` depends only on its own query token
(the definition has no term that couples two tokens), so the rows of a call
can be computed in independent groups and put back in place.  This module
cuts the requested packed query rows into groups of consecutive tokens and
runs the plain `paged_attention` on each group in a pool of threads, one per
core in this process's CPU affinity set, with the BLAS library held to one
thread per call so the pool, not BLAS, spreads the work.  NumPy releases the
interpreter lock inside its array operations (matrix products, exp, the
reductions), so the threads run in parallel; no process is forked.  Nothing
here changes the arithmetic: each row is the one `paged_attention` gives for
it.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .attention import OracleResult, paged_attention


def host_cores():
    """Cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:                      # platforms without affinity sets
        return os.cpu_count() or 1


def paged_attention_parallel(*, tokens=None, workers=None, tokens_per_item=8, **kwargs):
    """paged_attention(**kwargs, tokens=...) computed in groups of
    `tokens_per_item` consecutive requested rows on `workers` threads (default:
    every core of the affinity set).  Returns the same OracleResult as one
    call over all the rows."""
    from threadpoolctl import threadpool_limits

    q_lens = kwargs.get("q_lens")
    total_q = int(np.asarray(q_lens).sum()) if q_lens is not None else len(kwargs["seq_lens"])
    want = (np.arange(total_q, dtype=np.int64) if tokens is None
            else np.unique(np.asarray(tokens, dtype=np.int64)))
    items = [want[i:i + tokens_per_item] for i in range(0, want.size, tokens_per_item)]
    workers = host_cores() if workers is None else int(workers)

    with threadpool_limits(limits=1, user_api="blas"):
        with ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
            parts = list(ex.map(lambda t: paged_attention(**kwargs, tokens=t), items))

    Hq = parts[0].out.shape[1] if parts else int(kwargs["num_q_heads"])
    Dv = parts[0].out.shape[2] if parts else np.asarray(kwargs["v_cache"]).shape[3]
    out = np.empty((want.size, Hq, Dv))
    lse = np.empty((want.size, Hq))
    count = np.empty((want.size, Hq), dtype=np.int64)
    row = 0
    for part in parts:                          # items are consecutive slices of `want`
        n = part.tokens.size
        out[row:row + n] = part.out
        lse[row:row + n] = part.lse
        count[row:row + n] = part.count
        row += n
    return OracleResult(out=out, lse=lse, count=count, tokens=want)
