"""ctypes binding of libdiffkv_attn.so: the C-ABI entry points under the same names.

Argument marshalling only.  Tensors are passed as raw device pointers and the
stream as torch's current HIP stream; every step of the computation runs in
the library's kernels.  There is no fallback: if the library is missing,
every call raises.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

OK, INVALID_ARGUMENT, UNSUPPORTED, WORKSPACE_TOO_SMALL, HIP_ERROR = range(5)
ENTRY_DECODE, ENTRY_VERIFY, ENTRY_PREFILL, ENTRY_MIXED = 0, 1, 2, 3
KV_BF16, KV_FP8_E4M3 = 0, 1
ENTRIES = {"decode": ENTRY_DECODE, "verify": ENTRY_VERIFY, "prefill": ENTRY_PREFILL,
           "mixed": ENTRY_MIXED}


class DiffKVError(RuntimeError):
    pass


class AttnDesc(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "batch", "num_q_heads", "num_kv_heads", "head_dim_qk", "head_dim_v", "page_size",
        "num_pages", "block_table_stride", "max_seq_len", "max_q_len", "total_q", "kv_dtype",
        "force_num_splits")] + [("profile_start", ctypes.c_void_p), ("profile_stop", ctypes.c_void_p)]


_LIBRARY_FILES = {"release": "libdiffkv_attn.so", "debug": "libdiffkv_attn_debug.so",
                  "timeline": "libdiffkv_attn_timeline.so"}
_VARIANT = "release"


def library_path():
    return os.path.join(_HERE, _LIBRARY_FILES[_VARIANT])


def select_library(variant):
    """Which build later calls open: "release" (the default), "debug" (the
    same library with the device-side precondition checks compiled in; see
    diffkv_attn_debug_flags) or "timeline" (with per-workgroup real-time
    stamps in the split-KV kernels; see diffkv_attn_timeline_buffer).  Calls
    prepared earlier keep their library."""
    global _VARIANT, _LIB
    if variant not in _LIBRARY_FILES:
        raise ValueError(f"unknown library variant {variant!r}")
    if variant != _VARIANT:
        _VARIANT, _LIB = variant, None


_ENTRY_ARGS = [ctypes.POINTER(AttnDesc)] + [ctypes.c_void_p] * 6 + [
    ctypes.c_int32, ctypes.c_void_p, ctypes.c_float, ctypes.c_float, ctypes.c_float,
    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
    ctypes.c_void_p]


def load_library():
    """Open the HIP library once; raise if it is not built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise DiffKVError(f"{path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    for name in ("diffkv_attn_decode", "diffkv_attn_verify", "diffkv_attn_prefill",
                 "diffkv_attn_mixed"):
        fn = getattr(lib, name)
        fn.argtypes = _ENTRY_ARGS
        fn.restype = ctypes.c_int
    lib.diffkv_attn_verify_noalloc.argtypes = _ENTRY_ARGS[:15] + [ctypes.c_void_p]
    lib.diffkv_attn_verify_noalloc.restype = ctypes.c_int
    lib.diffkv_kv_write.argtypes = [ctypes.POINTER(AttnDesc)] + [ctypes.c_void_p] * 7 + [
        ctypes.c_float, ctypes.c_float, ctypes.c_void_p]
    lib.diffkv_attn_partial.argtypes = [ctypes.POINTER(AttnDesc)] + [ctypes.c_void_p] * 8 + [
        ctypes.c_int32, ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.diffkv_attn_partial.restype = ctypes.c_int
    lib.diffkv_attn_combine.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32] + [
        ctypes.c_void_p] * 6
    lib.diffkv_attn_combine.restype = ctypes.c_int
    lib.diffkv_kv_write.restype = ctypes.c_int
    lib.diffkv_attn_workspace_bytes.argtypes = [ctypes.POINTER(AttnDesc), ctypes.c_int]
    lib.diffkv_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.diffkv_attn_validate.argtypes = [ctypes.POINTER(AttnDesc), ctypes.c_int]
    lib.diffkv_attn_validate.restype = ctypes.c_int
    lib.diffkv_attn_num_splits.argtypes = [ctypes.POINTER(AttnDesc), ctypes.c_int, ctypes.c_int32]
    lib.diffkv_attn_num_splits.restype = ctypes.c_int
    lib.diffkv_attn_debug_flags.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.diffkv_attn_debug_flags.restype = ctypes.c_int
    lib.diffkv_attn_timeline_buffer.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.diffkv_attn_timeline_buffer.restype = ctypes.c_int
    lib.diffkv_attn_strerror.argtypes = [ctypes.c_int]
    lib.diffkv_attn_strerror.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def _ptr(x):
    """Device address of a tensor (or an int address, or None -> NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def diffkv_attn_strerror(status):
    return load_library().diffkv_attn_strerror(int(status)).decode()


def diffkv_attn_validate(desc, entry):
    return int(load_library().diffkv_attn_validate(ctypes.byref(desc), int(entry)))


def diffkv_attn_workspace_bytes(desc, entry):
    return int(load_library().diffkv_attn_workspace_bytes(ctypes.byref(desc), int(entry)))


def diffkv_attn_num_splits(desc, entry, window=0):
    return int(load_library().diffkv_attn_num_splits(ctypes.byref(desc), int(entry), int(window)))


def diffkv_attn_debug_flags(flags, stream=None):
    """Enqueue the copy of the debug build's violation bits into `flags` (a
    one-element int32 device tensor) and clear them; returns the status
    (UNSUPPORTED from a release build, which enqueues nothing)."""
    return int(load_library().diffkv_attn_debug_flags(_ptr(flags), _stream(stream)))


def diffkv_attn_timeline_buffer(stamps):
    """Register a uint64/int64 device tensor for the timeline build's stamps
    (eight per workgroup), or None to turn them off; returns the status
    (UNSUPPORTED from other builds).  Synchronous; not for graph capture."""
    if stamps is None:
        return int(load_library().diffkv_attn_timeline_buffer(None, 0))
    return int(load_library().diffkv_attn_timeline_buffer(_ptr(stamps), stamps.numel()))


def set_profile_events(desc, start, stop):
    """Put two raw hipEvent_t handles (ints), or two Nones, in the descriptor's
    measurement fields: every call made with it then stamps its first main
    kernel with them."""
    desc.profile_start = start
    desc.profile_stop = stop


def prepared_call(name, desc, q, k_cache, v_cache, block_table, seq_lens, q_lens, window, sinks,
                  k_scale, v_scale, softmax_scale, out, lse_out=None, count_out=None,
                  workspace=None, workspace_bytes=0, stream=None):
    """Resolve every argument once and return a no-argument callable that
    makes the C-ABI call (for tight timing loops); it raises on a bad status."""
    fn = getattr(load_library(), name)
    args = (ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            _ptr(seq_lens), _ptr(q_lens), int(window), _ptr(sinks), float(k_scale),
            float(v_scale), float(softmax_scale), _ptr(out), _ptr(lse_out), _ptr(count_out),
            _ptr(workspace), int(workspace_bytes), _stream(stream))
    keep = (desc, q, k_cache, v_cache, block_table, seq_lens, q_lens, sinks, out, lse_out,
            count_out, workspace)

    def call():
        status = fn(*args)
        if status != OK:
            raise DiffKVError(f"{name}: {diffkv_attn_strerror(status)} (status {status})")
    call.keep_alive = keep
    call.desc = desc
    return call


def _call(name, desc, q, k_cache, v_cache, block_table, seq_lens, q_lens, window, sinks,
          k_scale, v_scale, softmax_scale, out, lse_out=None, count_out=None, workspace=None,
          workspace_bytes=0, stream=None):
    fn = getattr(load_library(), name)
    status = fn(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                _ptr(seq_lens), _ptr(q_lens), int(window), _ptr(sinks), float(k_scale),
                float(v_scale), float(softmax_scale), _ptr(out), _ptr(lse_out), _ptr(count_out),
                _ptr(workspace), int(workspace_bytes), _stream(stream))
    if status != OK:
        raise DiffKVError(f"{name}: {diffkv_attn_strerror(status)} (status {status})")


def diffkv_attn_decode(*args, **kwargs):
    _call("diffkv_attn_decode", *args, **kwargs)


def diffkv_attn_verify(*args, **kwargs):
    _call("diffkv_attn_verify", *args, **kwargs)


def diffkv_attn_prefill(*args, **kwargs):
    _call("diffkv_attn_prefill", *args, **kwargs)


def diffkv_attn_mixed(*args, **kwargs):
    _call("diffkv_attn_mixed", *args, **kwargs)


def diffkv_attn_verify_noalloc(desc, q, k_cache, v_cache, block_table, seq_lens, q_lens, window,
                               sinks, k_scale, v_scale, softmax_scale, out, lse_out=None,
                               count_out=None, stream=None):
    """diffkv_attn_verify on the library's static per-device workspace."""
    status = load_library().diffkv_attn_verify_noalloc(
        ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(seq_lens), _ptr(q_lens), int(window), _ptr(sinks), float(k_scale), float(v_scale),
        float(softmax_scale), _ptr(out), _ptr(lse_out), _ptr(count_out), _stream(stream))
    if status != OK:
        raise DiffKVError(f"diffkv_attn_verify_noalloc: {diffkv_attn_strerror(status)} "
                          f"(status {status})")


def prepared_kv_write(desc, k_new, v_new, k_cache, v_cache, block_table, seq_lens, q_lens,
                      k_scale=1.0, v_scale=1.0, stream=None):
    """Like prepared_call, for diffkv_kv_write."""
    fn = load_library().diffkv_kv_write
    args = (ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
            _ptr(block_table), _ptr(seq_lens), _ptr(q_lens), float(k_scale), float(v_scale),
            _stream(stream))
    keep = (desc, k_new, v_new, k_cache, v_cache, block_table, seq_lens, q_lens)

    def call():
        status = fn(*args)
        if status != OK:
            raise DiffKVError(f"diffkv_kv_write: {diffkv_attn_strerror(status)} (status {status})")
    call.keep_alive = keep
    call.desc = desc
    return call


def diffkv_kv_write(desc, k_new, v_new, k_cache, v_cache, block_table, seq_lens, q_lens,
                    k_scale=1.0, v_scale=1.0, stream=None):
    prepared_kv_write(desc, k_new, v_new, k_cache, v_cache, block_table, seq_lens, q_lens,
                      k_scale, v_scale, stream)()


def _prepared(name, args, keep):
    fn = getattr(load_library(), name)

    def call():
        status = fn(*args)
        if status != OK:
            raise DiffKVError(f"{name}: {diffkv_attn_strerror(status)} (status {status})")
    call.keep_alive = keep
    return call


def prepared_partial(desc, q, k_cache, v_cache, block_table, seq_lens, q_lens, key_lo, key_hi,
                     window, k_scale, v_scale, softmax_scale, out_part, lse_part, count_out=None,
                     workspace=None, workspace_bytes=0, stream=None):
    """Like prepared_call, for diffkv_attn_partial."""
    args = (ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            _ptr(seq_lens), _ptr(q_lens), _ptr(key_lo), _ptr(key_hi), int(window), float(k_scale),
            float(v_scale), float(softmax_scale), _ptr(out_part), _ptr(lse_part), _ptr(count_out),
            _ptr(workspace), int(workspace_bytes), _stream(stream))
    call = _prepared("diffkv_attn_partial", args,
                     (desc, q, k_cache, v_cache, block_table, seq_lens, q_lens, key_lo, key_hi,
                      out_part, lse_part, count_out, workspace))
    call.desc = desc
    return call


def prepared_combine(num_parts, rows, num_q_heads, out_parts, lse_parts, sinks, out,
                     lse_out=None, stream=None):
    """Like prepared_call, for diffkv_attn_combine."""
    args = (int(num_parts), int(rows), int(num_q_heads), _ptr(out_parts), _ptr(lse_parts),
            _ptr(sinks), _ptr(out), _ptr(lse_out), _stream(stream))
    return _prepared("diffkv_attn_combine", args, (out_parts, lse_parts, sinks, out, lse_out))


def diffkv_attn_partial(*args, **kwargs):
    prepared_partial(*args, **kwargs)()


def diffkv_attn_combine(*args, **kwargs):
    prepared_combine(*args, **kwargs)()
