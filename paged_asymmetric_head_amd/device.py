"""Device-resident inputs and one-call helpers over the C ABI.

torch provides device memory and the stream; every step of the attention runs
in libdiffkv_attn.so.  `run` allocates the outputs and the workspace the
library asks for, then makes exactly one C-ABI call.
"""

import numpy as np
import torch

from . import binding as B


def _to_device(arr, device):
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)        # bf16 codes travel as int16 storage
    return torch.from_numpy(a).to(device)


class DeviceInputs:
    """A PagedInputs workload copied to one GPU (caches, tables, queries)."""

    def __init__(self, inp, device="cuda"):
        self.inp = inp
        self.device = torch.device(device)
        self.q = _to_device(inp.q, self.device)
        self.k_cache = _to_device(inp.k_cache, self.device)
        self.v_cache = _to_device(inp.v_cache, self.device)
        self.block_table = _to_device(inp.block_table.astype(np.int32), self.device)
        self.seq_lens = _to_device(inp.seq_lens.astype(np.int32), self.device)
        self.q_lens = _to_device(inp.q_lens.astype(np.int32), self.device)
        self.sinks = None if inp.sinks is None else _to_device(inp.sinks.astype(np.float32), self.device)

    def desc(self, entry, force_num_splits=0):
        inp = self.inp
        return B.AttnDesc(batch=inp.batch, num_q_heads=inp.num_q_heads,
                          num_kv_heads=inp.num_kv_heads, head_dim_qk=inp.q.shape[2],
                          head_dim_v=inp.v_cache.shape[3], page_size=inp.page_size,
                          num_pages=inp.num_pages, block_table_stride=inp.block_table_stride,
                          max_seq_len=inp.max_seq_len,
                          max_q_len=1 if entry == "decode" else inp.max_q_len,
                          total_q=inp.total_q,
                          kv_dtype=B.KV_FP8_E4M3 if inp.kv_dtype == "fp8" else B.KV_BF16,
                          force_num_splits=force_num_splits)

    def workspace_for(self, entry, force_num_splits=0):
        d = self.desc(entry, force_num_splits)
        nbytes = B.diffkv_attn_workspace_bytes(d, B.ENTRIES[entry])
        if nbytes == 0:
            return None, 0
        return torch.empty(nbytes, dtype=torch.uint8, device=self.device), nbytes

    def run(self, entry, *, lse=False, count=False, force_num_splits=0, out=None, workspace=None,
            stream=None, block_table=None, sinks="default", window=None):
        """One call of diffkv_attn_<entry>; returns (out bf16, lse fp32|None, count int32|None)."""
        inp = self.inp
        d = self.desc(entry, force_num_splits)
        if out is None:
            out = torch.empty((inp.total_q, inp.num_q_heads, inp.v_cache.shape[3]),
                              dtype=torch.bfloat16, device=self.device)
        lse_t = torch.empty((inp.total_q, inp.num_q_heads), dtype=torch.float32,
                            device=self.device) if lse else None
        cnt_t = torch.empty((inp.total_q, inp.num_q_heads), dtype=torch.int32,
                            device=self.device) if count else None
        if workspace is None:
            ws, nbytes = self.workspace_for(entry, force_num_splits)
        else:
            ws, nbytes = workspace, workspace.numel() * workspace.element_size()
        fn = {"decode": B.diffkv_attn_decode, "verify": B.diffkv_attn_verify,
              "prefill": B.diffkv_attn_prefill, "mixed": B.diffkv_attn_mixed}[entry]
        fn(d, self.q, self.k_cache, self.v_cache,
           self.block_table if block_table is None else block_table,
           self.seq_lens, self.q_lens, inp.window if window is None else window,
           self.sinks if isinstance(sinks, str) else sinks, inp.k_scale, inp.v_scale,
           inp.softmax_scale, out, lse_t, cnt_t, ws, nbytes, stream)
        return out, lse_t, cnt_t

    def prepare(self, entry, *, k_cache=None, v_cache=None, force_num_splits=0, stream=None,
                lse=False, count=False):
        """Allocate outputs and workspace once and return a no-argument callable
        making one C-ABI call (its `.out` is the output tensor)."""
        inp = self.inp
        d = self.desc(entry, force_num_splits)
        out = torch.empty((inp.total_q, inp.num_q_heads, inp.v_cache.shape[3]),
                          dtype=torch.bfloat16, device=self.device)
        lse_t = torch.empty((inp.total_q, inp.num_q_heads), dtype=torch.float32,
                            device=self.device) if lse else None
        cnt_t = torch.empty((inp.total_q, inp.num_q_heads), dtype=torch.int32,
                            device=self.device) if count else None
        ws, nbytes = self.workspace_for(entry, force_num_splits)
        call = B.prepared_call(f"diffkv_attn_{entry}", d, self.q,
                               self.k_cache if k_cache is None else k_cache,
                               self.v_cache if v_cache is None else v_cache,
                               self.block_table, self.seq_lens, self.q_lens, inp.window,
                               self.sinks, inp.k_scale, inp.v_scale, inp.softmax_scale, out,
                               lse_t, cnt_t, ws, nbytes, stream)
        call.out, call.lse, call.count = out, lse_t, cnt_t
        return call
