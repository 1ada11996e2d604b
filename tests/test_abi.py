"""Host-side checks of the C-ABI library (no GPU needed, no compute call).

The library must load, export every function include/diffkv_attn.h declares,
and reject bad descriptors synchronously through diffkv_attn_validate.
"""

import ctypes
import os
import re

import pytest

from paged_asymmetric_head_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "diffkv_attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(diffkv_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.library_path()):
        pytest.fail("libdiffkv_attn.so is not built (run __graft_entry__.build())")
    return B.load_library()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("diffkv_attn_decode", "diffkv_attn_verify", "diffkv_attn_prefill",
              "diffkv_attn_workspace_bytes", "diffkv_attn_validate", "diffkv_attn_strerror",
              "diffkv_attn_num_splits", "diffkv_kv_write", "diffkv_attn_mixed",
              "diffkv_attn_partial", "diffkv_attn_combine"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_debug_library_exports_every_declared_symbol():
    """The debug build (device-side precondition checks) has the same ABI;
    its flag call rejects a NULL destination before touching the GPU."""
    path = os.path.join(ROOT, "paged_asymmetric_head_amd", "libdiffkv_attn_debug.so")
    if not os.path.exists(path):
        pytest.fail("libdiffkv_attn_debug.so is not built (run __graft_entry__.build())")
    dlib = ctypes.CDLL(path)
    for name in declared_functions():
        assert hasattr(dlib, name), name
    dlib.diffkv_attn_debug_flags.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    assert dlib.diffkv_attn_debug_flags(None, None) == B.INVALID_ARGUMENT


def test_release_library_has_no_debug_checks(lib):
    assert lib.diffkv_attn_debug_flags(None, None) == B.UNSUPPORTED


def test_timeline_library_exports_every_declared_symbol():
    """The timeline build (per-workgroup real-time stamps) has the same ABI;
    its buffer call rejects a pointer / size mismatch before touching the
    GPU, and the release build has no stamps."""
    path = os.path.join(ROOT, "paged_asymmetric_head_amd", "libdiffkv_attn_timeline.so")
    if not os.path.exists(path):
        pytest.fail("libdiffkv_attn_timeline.so is not built (run __graft_entry__.build())")
    tlib = ctypes.CDLL(path)
    for name in declared_functions():
        assert hasattr(tlib, name), name
    tlib.diffkv_attn_timeline_buffer.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    assert tlib.diffkv_attn_timeline_buffer(None, 8) == B.INVALID_ARGUMENT


def test_release_library_has_no_timeline(lib):
    assert lib.diffkv_attn_timeline_buffer(None, 0) == B.UNSUPPORTED


def good_desc(**kw):
    d = dict(batch=4, num_q_heads=8, num_kv_heads=1, head_dim_qk=192, head_dim_v=128,
             page_size=128, num_pages=2000, block_table_stride=400, max_seq_len=50000,
             max_q_len=8, total_q=32, kv_dtype=B.KV_BF16, force_num_splits=0)
    d.update(kw)
    return B.AttnDesc(**d)


def test_validate_accepts_good_descriptors(lib):
    assert B.diffkv_attn_validate(good_desc(), B.ENTRY_VERIFY) == B.OK
    assert B.diffkv_attn_validate(good_desc(), B.ENTRY_PREFILL) == B.OK
    assert B.diffkv_attn_validate(good_desc(max_q_len=1, total_q=4), B.ENTRY_DECODE) == B.OK
    assert B.diffkv_attn_validate(good_desc(kv_dtype=B.KV_FP8_E4M3, page_size=1,
                                            block_table_stride=50000), B.ENTRY_VERIFY) == B.OK
    assert B.diffkv_attn_validate(good_desc(max_q_len=4096, total_q=4200), B.ENTRY_MIXED) == B.OK
    for entry in (B.ENTRY_VERIFY, B.ENTRY_PREFILL, B.ENTRY_MIXED):     # symmetric 128/128 heads
        assert B.diffkv_attn_validate(good_desc(head_dim_qk=128), entry) == B.OK


@pytest.mark.parametrize("field,value,entry,status", [
    ("num_q_heads", 7, B.ENTRY_VERIFY, B.INVALID_ARGUMENT),       # Hq % Hkv with Hkv=2 below
    ("head_dim_qk", 64, B.ENTRY_VERIFY, B.UNSUPPORTED),
    ("head_dim_qk", 256, B.ENTRY_VERIFY, B.UNSUPPORTED),
    ("head_dim_v", 192, B.ENTRY_VERIFY, B.UNSUPPORTED),
    ("page_size", 96, B.ENTRY_VERIFY, B.UNSUPPORTED),
    ("page_size", 512, B.ENTRY_VERIFY, B.UNSUPPORTED),
    ("kv_dtype", 7, B.ENTRY_VERIFY, B.UNSUPPORTED),
    ("batch", 0, B.ENTRY_VERIFY, B.INVALID_ARGUMENT),
    ("max_q_len", 17, B.ENTRY_VERIFY, B.INVALID_ARGUMENT),
    ("max_q_len", 8, B.ENTRY_DECODE, B.INVALID_ARGUMENT),
    ("block_table_stride", 390, B.ENTRY_VERIFY, B.INVALID_ARGUMENT),
    ("total_q", 33, B.ENTRY_VERIFY, B.INVALID_ARGUMENT),
    ("total_q", 3, B.ENTRY_VERIFY, B.INVALID_ARGUMENT),
    ("force_num_splits", -1, B.ENTRY_VERIFY, B.INVALID_ARGUMENT),
    ("num_pages", 0, B.ENTRY_VERIFY, B.INVALID_ARGUMENT),
])
def test_validate_rejects(lib, field, value, entry, status):
    kw = {field: value}
    if field == "num_q_heads":
        kw["num_kv_heads"] = 2
    assert B.diffkv_attn_validate(good_desc(**kw), entry) == status


def test_validate_rejects_null_and_bad_entry(lib):
    assert lib.diffkv_attn_validate(None, 0) == B.INVALID_ARGUMENT
    assert B.diffkv_attn_validate(good_desc(), 4) == B.INVALID_ARGUMENT
    assert B.diffkv_attn_validate(good_desc(), -1) == B.INVALID_ARGUMENT


def test_workspace_and_splits(lib):
    d = good_desc()
    ns = B.diffkv_attn_num_splits(d, B.ENTRY_VERIFY)
    assert ns > 1
    ws = B.diffkv_attn_workspace_bytes(d, B.ENTRY_VERIFY)
    # partial rows (bf16 x 128) + one fp32 lse per row, per split, per 64-row query tile
    assert ws >= 4 * 1 * ns * 64 * (128 * 2 + 4)
    assert B.diffkv_attn_workspace_bytes(d, B.ENTRY_PREFILL) == 0
    assert B.diffkv_attn_num_splits(d, B.ENTRY_PREFILL) == 1
    # A window only shrinks the split count, so the full-attention workspace covers it.
    assert B.diffkv_attn_num_splits(d, B.ENTRY_VERIFY, 128) <= ns
    # Forced split count.
    assert B.diffkv_attn_num_splits(good_desc(force_num_splits=7), B.ENTRY_VERIFY) == 7
    # Mixed: the split part is planned as a verify call with q_len clipped to
    # 16, so its splits and workspace match that verify call.
    mixed = good_desc(max_q_len=4096, total_q=4200)
    clipped = good_desc(max_q_len=16, total_q=32)
    assert (B.diffkv_attn_num_splits(mixed, B.ENTRY_MIXED)
            == B.diffkv_attn_num_splits(clipped, B.ENTRY_VERIFY))
    assert (B.diffkv_attn_workspace_bytes(mixed, B.ENTRY_MIXED)
            == B.diffkv_attn_workspace_bytes(clipped, B.ENTRY_VERIFY))
    assert (B.diffkv_attn_num_splits(d, B.ENTRY_MIXED) == ns)
    # Invalid descriptor -> 0 bytes.
    assert B.diffkv_attn_workspace_bytes(good_desc(batch=0), B.ENTRY_VERIFY) == 0


def test_strerror(lib):
    assert B.diffkv_attn_strerror(B.OK) == "success"
    assert "workspace" in B.diffkv_attn_strerror(B.WORKSPACE_TOO_SMALL)
    assert B.diffkv_attn_strerror(99) == "unknown status"


def test_entry_rejects_before_touching_the_gpu(lib):
    """Argument errors return synchronously, before any HIP call."""
    d = good_desc(head_dim_qk=64)
    fn = lib.diffkv_attn_verify
    st = fn(ctypes.byref(d), None, None, None, None, None, None, 0, None, 1.0, 1.0, 1.0,
            None, None, None, None, 0, None)
    assert st == B.UNSUPPORTED
    d = good_desc()
    st = fn(ctypes.byref(d), None, None, None, None, None, None, 0, None, 1.0, 1.0, 1.0,
            None, None, None, None, 0, None)
    assert st == B.INVALID_ARGUMENT


def test_kv_write_rejects_before_touching_the_gpu(lib):
    """Descriptor, pointer and scale errors of the KV write return synchronously."""
    fn = lib.diffkv_kv_write
    fake = 256                      # never dereferenced: every case fails its checks first
    ptrs = [fake] * 7

    def call(d, ptrs=ptrs, ks=1.0, vs=1.0):
        return fn(ctypes.byref(d), *ptrs, ks, vs, None)

    assert call(good_desc(head_dim_v=64)) == B.UNSUPPORTED
    assert call(good_desc(page_size=96)) == B.UNSUPPORTED
    assert call(good_desc(total_q=0)) == B.INVALID_ARGUMENT
    for i in range(6):              # k_new, v_new, caches, block table, seq_lens
        p = list(ptrs)
        p[i] = None
        assert call(good_desc(), p) == B.INVALID_ARGUMENT, i
    p = list(ptrs)
    p[6] = None                     # q_lens NULL needs max_q_len == 1
    assert call(good_desc(), p) == B.INVALID_ARGUMENT
    fp8 = good_desc(kv_dtype=B.KV_FP8_E4M3)
    for ks, vs in ((0.0, 1.0), (1.0, -2.0), (float("nan"), 1.0), (1.0, float("inf"))):
        assert call(fp8, ks=ks, vs=vs) == B.INVALID_ARGUMENT, (ks, vs)


def test_partial_and_combine_reject_before_touching_the_gpu(lib):
    fake = 256                      # never dereferenced: every case fails its checks first
    d = good_desc()
    fn = lib.diffkv_attn_partial
    # out_part / lse_part missing
    assert fn(ctypes.byref(d), *[fake] * 8, 0, 1.0, 1.0, 1.0, None, fake, None, None, 0, None) \
        == B.INVALID_ARGUMENT
    assert fn(ctypes.byref(d), *[fake] * 8, 0, 1.0, 1.0, 1.0, fake, None, None, None, 0, None) \
        == B.INVALID_ARGUMENT
    # verify-shaped only
    d17 = good_desc(max_q_len=17)
    assert fn(ctypes.byref(d17), *[fake] * 8, 0, 1.0, 1.0, 1.0, fake, fake, None, None, 0, None) \
        == B.INVALID_ARGUMENT
    c = lib.diffkv_attn_combine
    assert c(0, 8, 4, fake, fake, None, fake, None, None) == B.INVALID_ARGUMENT
    assert c(2, 10, 4, fake, fake, None, fake, None, None) == B.INVALID_ARGUMENT   # rows % Hq
    assert c(65, 8, 4, fake, fake, None, fake, None, None) == B.UNSUPPORTED
    assert c(2, 8, 4, None, fake, None, fake, None, None) == B.INVALID_ARGUMENT


def test_stream_reference_library_loads_and_rejects_bad_arguments():
    """The streaming-read reference the benchmark quotes (its own library,
    outside the attention ABI) loads, exports its one call, and rejects bad
    arguments on the host without launching anything."""
    import ctypes
    path = os.path.join(ROOT, "paged_asymmetric_head_amd", "libdiffkv_stream.so")
    lib = ctypes.CDLL(path)
    fn = lib.diffkv_stream_read
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                   ctypes.c_void_p]
    fn.restype = ctypes.c_int
    assert fn(None, 16, 16, 1, 4, None) == 1            # null source
    assert fn(16, 16, None, 1, 4, None) == 1            # null sink
    assert fn(16, 16, 16, 0, 4, None) == 1              # no workgroups
    assert fn(16, 17, 16, 1, 4, None) == 1              # not a multiple of 16 bytes
    assert fn(8, 16, 16, 1, 4, None) == 1               # misaligned source
    assert fn(16, 16, 16, 1, 5, None) == 1              # unsupported loads per thread


def test_measurement_events_come_in_pairs(lib):
    """The descriptor's measurement events are both set or both NULL (host
    only: the handles are checked, never used, by the validation)."""
    d = good_desc()
    assert B.diffkv_attn_validate(d, B.ENTRY_VERIFY) == B.OK
    fake = 256
    for start, stop, want in ((fake, None, B.INVALID_ARGUMENT), (None, fake, B.INVALID_ARGUMENT),
                              (fake, fake + 8, B.OK), (None, None, B.OK)):
        B.set_profile_events(d, start, stop)
        assert B.diffkv_attn_validate(d, B.ENTRY_VERIFY) == want, (start, stop)
