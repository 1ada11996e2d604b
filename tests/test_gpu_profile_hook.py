"""The measurement events of the call descriptor (profile_start /
profile_stop): a call made with them stamps its main kernel (a positive
duration no longer than the host's wall time around the call); a call that
fails its argument checks leaves them untouched, and a call made with the
fields cleared again records nothing in them."""

import ctypes
import time

import pytest
import torch

from paged_asymmetric_head_amd import binding as B
from paged_asymmetric_head_amd.device import DeviceInputs
from paged_asymmetric_head_amd.synth import make_paged_inputs

pytestmark = pytest.mark.gpu


class Events:
    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        for fn in ("hipEventCreate", "hipEventRecord", "hipEventElapsedTime", "hipEventDestroy"):
            getattr(self.hip, fn).restype = ctypes.c_int
        self.made = []

    def create(self):
        ev = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(ev)) == 0
        self.made.append(ev.value)
        return ev.value

    def record(self, ev, stream):
        assert self.hip.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) == 0

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return float(ms.value)

    def close(self):
        for ev in self.made:
            self.hip.hipEventDestroy(ctypes.c_void_p(ev))


def test_descriptor_events_time_the_main_kernel():
    lens = [9000, 7000, 8000, 6500]
    inp = make_paged_inputs(71, seq_lens=lens, q_lens=8, num_q_heads=8, num_kv_heads=1,
                            page_size=128, kv_dtype="bf16", sinks=True)
    dev = DeviceInputs(inp)
    call = dev.prepare("verify")
    stream = torch.cuda.current_stream().cuda_stream
    ev = Events()
    try:
        print("[gpu] measurement events: verify call with events", flush=True)
        s1, e1 = ev.create(), ev.create()
        torch.cuda.synchronize()
        B.set_profile_events(call.desc, s1, e1)
        t0 = time.perf_counter()
        call()
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3
        ms = ev.elapsed_ms(s1, e1)
        assert 0.0 < ms <= wall_ms

        print("[gpu] measurement events: failed call, then a call without events", flush=True)
        s2, e2 = ev.create(), ev.create()
        ev.record(s2, stream)
        ev.record(e2, stream)
        torch.cuda.synchronize()
        before = ev.elapsed_ms(s2, e2)
        bad = dev.desc("verify")
        B.set_profile_events(bad, s2, e2)
        bad.max_q_len = 17                         # over the verify limit: rejected before any launch
        lib = B.load_library()
        st = lib.diffkv_attn_verify(ctypes.byref(bad), None, None, None, None, None, None, 0, None,
                                    1.0, 1.0, 1.0, None, None, None, None, 0, None)
        assert st == B.INVALID_ARGUMENT
        B.set_profile_events(call.desc, None, None)
        call()                                     # records nothing in s2 / e2 (or s1 / e1)
        torch.cuda.synchronize()
        assert ev.elapsed_ms(s2, e2) == before
        assert ev.elapsed_ms(s1, e1) == ms
    finally:
        B.set_profile_events(call.desc, None, None)
        torch.cuda.synchronize()
        ev.close()
