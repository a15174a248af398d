"""ctypes binding of libpa.so (include/pa.h).  Argument marshalling only:
torch tensors become pa_tensor descriptors, torch's current stream becomes the
hipStream_t, status codes become exceptions.  Every step of the computation runs
in the library's HIP kernels; there is no fallback.

libpa.so must be loaded after ``import torch`` so that it binds to the HIP
runtime torch already loaded (both carry the soname libamdhip64.so.7).
"""

import ctypes
import os
import struct

import numpy as np

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")

PA_OK, PA_ERR_INVALID, PA_ERR_UNSUPPORTED, PA_ERR_HIP, PA_ERR_WORKSPACE, PA_ERR_CONTRACT = 0, -1, -2, -3, -4, -5
PA_BF16, PA_F32, PA_I32, PA_I64 = 1, 2, 3, 4
MAX_DIMS = 5

EXPORTED = ("pa_append_decode", "pa_cache_append", "pa_copy_blocks", "pa_decode", "pa_decode_contiguous",
            "pa_decode_ex", "pa_decode_noalloc",
            "pa_decode_multi", "pa_decode_multi_ex", "pa_decode_multi_workspace_bytes", "pa_decode_workspace_bytes",
            "pa_decode_schedule", "pa_last_error", "pa_last_launch", "pa_set_debug")

_DTYPES = {torch.bfloat16: PA_BF16, torch.float32: PA_F32, torch.int32: PA_I32, torch.int64: PA_I64}


class PaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * MAX_DIMS), ("stride", ctypes.c_int64 * MAX_DIMS)]


class PaDecodeOpts(ctypes.Structure):
    _fields_ = [("partition_tokens", ctypes.c_int32), ("path", ctypes.c_int32),
                ("max_context_len", ctypes.c_int64), ("workgroups_per_cu", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("kernel_start", ctypes.c_void_p),
                ("kernel_stop", ctypes.c_void_p), ("host_context_lens", ctypes.c_void_p)]


class PaError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"libpa error {code}: {message}")
        self.code = code


_lib = None


def load(path=None):
    """Load libpa.so (once).  Raises if it is missing: there is no fallback."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing; build it with `python -m paged_kv_cache_122_amd.build`")
    lib = ctypes.CDLL(p)
    P = ctypes.POINTER(PaTensor)
    lib.pa_cache_append.argtypes = [P, P, P, P, P, ctypes.c_void_p]
    lib.pa_cache_append.restype = ctypes.c_int
    lib.pa_copy_blocks.argtypes = [P, P, P, ctypes.c_void_p]
    lib.pa_decode_contiguous.argtypes = [P, P, P, P, P, ctypes.c_float, ctypes.c_void_p]
    lib.pa_decode_multi.argtypes = [P] * 10 + [ctypes.c_float, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    lib.pa_decode_multi_ex.argtypes = [P] * 10 + [ctypes.c_float, ctypes.c_int32, ctypes.c_int32,
                                                  ctypes.POINTER(PaDecodeOpts), ctypes.c_void_p, ctypes.c_size_t,
                                                  ctypes.c_void_p]
    lib.pa_decode_multi_ex.restype = ctypes.c_int
    lib.pa_decode_multi_workspace_bytes.argtypes = [ctypes.c_int64] * 5 + [ctypes.c_int32, ctypes.c_int64,
                                                                           ctypes.c_int32]
    lib.pa_decode_multi_workspace_bytes.restype = ctypes.c_size_t
    lib.pa_decode_contiguous.restype = ctypes.c_int
    lib.pa_copy_blocks.restype = ctypes.c_int
    lib.pa_decode.argtypes = [P, P, P, P, P, P, ctypes.c_float, ctypes.c_int32, ctypes.c_void_p]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode_noalloc.argtypes = [P, P, P, P, P, P, ctypes.c_float, ctypes.c_int32, ctypes.c_void_p]
    lib.pa_decode_noalloc.restype = ctypes.c_int
    lib.pa_decode_ex.argtypes = [P, P, P, P, P, P, ctypes.c_float, ctypes.c_int32,
                                 ctypes.POINTER(PaDecodeOpts), ctypes.c_void_p, ctypes.c_size_t,
                                 ctypes.c_void_p]
    lib.pa_decode_ex.restype = ctypes.c_int
    lib.pa_append_decode.argtypes = [P] * 9 + [ctypes.c_float, ctypes.c_int32, ctypes.POINTER(PaDecodeOpts),
                                               ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.pa_append_decode.restype = ctypes.c_int
    lib.pa_decode_workspace_bytes.argtypes = [ctypes.c_int64] * 5 + [ctypes.c_int32]
    lib.pa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.pa_decode_schedule.argtypes = [ctypes.c_int64] * 4 + [ctypes.POINTER(ctypes.c_int32)]
    lib.pa_decode_schedule.restype = ctypes.c_int
    lib.pa_last_error.argtypes = []
    lib.pa_last_error.restype = ctypes.c_char_p
    lib.pa_last_launch.argtypes = []
    lib.pa_last_launch.restype = ctypes.c_char_p
    lib.pa_set_debug.argtypes = [ctypes.c_int]
    lib.pa_set_debug.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


# pa_tensor's bytes: data pointer, dtype, ndim, shape[5], stride[5] (no padding)
_PA_TENSOR = struct.Struct("<Qii5q5q")
_ZEROS = (0,) * MAX_DIMS


def describe(t):
    """pa_tensor for a torch tensor (no copy; the tensor must outlive the call).
    Packed in one struct.pack: a step passes nine of these, and building them
    field by field cost more host time than the library's own call."""
    dtype = _DTYPES.get(t.dtype)
    if dtype is None:
        raise TypeError(f"unsupported dtype {t.dtype}")
    nd = t.dim()
    if nd > MAX_DIMS or nd < 1:
        raise ValueError("tensor rank must be 1..5")
    pad = _ZEROS[nd:]
    return PaTensor.from_buffer_copy(_PA_TENSOR.pack(t.data_ptr() if t.numel() > 0 else 0, dtype, nd, *t.shape,
                                                     *pad, *t.stride(), *pad))


def _device_tensor(t, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    return t


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(lib, rc):
    if rc != PA_OK:
        raise PaError(rc, lib.pa_last_error().decode())


def cache_append(k, v, slot_mapping, k_cache, v_cache, stream=None):
    """pa_cache_append: write k/v [T, Hkv, D] (bf16) at slot_mapping [T] (int64)."""
    lib = load()
    ts = [_device_tensor(x, n) for x, n in ((k, "k"), (v, "v"), (slot_mapping, "slot_mapping"),
                                           (k_cache, "k_cache"), (v_cache, "v_cache"))]
    ds = [describe(x) for x in ts]
    _check(lib, lib.pa_cache_append(*[ctypes.byref(d) for d in ds], _stream(stream)))


def decode_contiguous(out, q, k, v, context_lens, scale, stream=None):
    """pa_decode_contiguous: decode over per-(sequence, head) contiguous K/V (the paging control)."""
    lib = load()
    ts = [_device_tensor(x, n) for x, n in ((out, "out"), (q, "q"), (k, "k"), (v, "v"),
                                           (context_lens, "context_lens"))]
    ds = [describe(x) for x in ts]
    _check(lib, lib.pa_decode_contiguous(*[ctypes.byref(d) for d in ds], ctypes.c_float(scale),
                                         _stream(stream)))


def decode_multi(out, q, k_new, v_new, slot_mapping, query_start, k_cache, v_cache, block_tables,
                 context_lens, scale, block_size, max_query_len, stream=None):
    """pa_decode_multi: append the rows of k_new / v_new and attend every row of q
    [T, Hq, D] causally over its sequence (query_start int32 [S + 1])."""
    lib = load()
    ts = [_device_tensor(x, n) for x, n in (
        (out, "out"), (q, "q"), (k_new, "k_new"), (v_new, "v_new"), (slot_mapping, "slot_mapping"),
        (query_start, "query_start"), (k_cache, "k_cache"), (v_cache, "v_cache"),
        (block_tables, "block_tables"), (context_lens, "context_lens"))]
    ds = [describe(x) for x in ts]
    _check(lib, lib.pa_decode_multi(*[ctypes.byref(d) for d in ds], ctypes.c_float(scale),
                                    ctypes.c_int32(block_size), ctypes.c_int32(max_query_len),
                                    _stream(stream)))


def decode_multi_ex(out, q, k_new, v_new, slot_mapping, query_start, k_cache, v_cache, block_tables,
                    context_lens, scale, block_size, max_query_len, *, partition_tokens=0, path=0,
                    max_context_len=0, workspace=None, kernel_events=None, host_context_lens=None, stream=None):
    """pa_decode_multi_ex: pa_decode_multi with options and a caller-owned workspace (no allocation)."""
    lib = load()
    ts = [_device_tensor(x, n) for x, n in (
        (out, "out"), (q, "q"), (k_new, "k_new"), (v_new, "v_new"), (slot_mapping, "slot_mapping"),
        (query_start, "query_start"), (k_cache, "k_cache"), (v_cache, "v_cache"),
        (block_tables, "block_tables"), (context_lens, "context_lens"))]
    ds = [describe(x) for x in ts]
    hl = _host_lens(host_context_lens, context_lens)
    opts = _opts(partition_tokens, path, max_context_len, 0, kernel_events, hl)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(lib, lib.pa_decode_multi_ex(*[ctypes.byref(d) for d in ds], ctypes.c_float(scale),
                                       ctypes.c_int32(block_size), ctypes.c_int32(max_query_len), ctypes.byref(opts),
                                       ctypes.c_void_p(ws_ptr) if ws_ptr else None, ctypes.c_size_t(ws_bytes),
                                       _stream(stream)))


def multi_workspace_bytes(num_rows, num_seqs, num_q_heads, num_kv_heads, head_dim, max_query_len,
                          max_context_len, partition_tokens=0):
    """pa_decode_multi_workspace_bytes."""
    return int(load().pa_decode_multi_workspace_bytes(int(num_rows), int(num_seqs), int(num_q_heads),
                                                      int(num_kv_heads), int(head_dim), int(max_query_len),
                                                      int(max_context_len), int(partition_tokens)))


def copy_blocks(k_cache, v_cache, block_pairs, stream=None):
    """pa_copy_blocks: for each (src, dst) row of block_pairs (int64 [N, 2]), copy block src to dst."""
    lib = load()
    ts = [_device_tensor(x, n) for x, n in ((k_cache, "k_cache"), (v_cache, "v_cache"),
                                           (block_pairs, "block_pairs"))]
    ds = [describe(x) for x in ts]
    _check(lib, lib.pa_copy_blocks(*[ctypes.byref(d) for d in ds], _stream(stream)))


def decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size, stream=None):
    """pa_decode: out [S, Hq, D] (bf16 or f32) = paged attention of q [S, Hq, D]."""
    lib = load()
    ts = [_device_tensor(x, n) for x, n in ((out, "out"), (q, "q"), (k_cache, "k_cache"),
                                           (v_cache, "v_cache"), (block_tables, "block_tables"),
                                           (context_lens, "context_lens"))]
    ds = [describe(x) for x in ts]
    _check(lib, lib.pa_decode(*[ctypes.byref(d) for d in ds], ctypes.c_float(scale),
                              ctypes.c_int32(block_size), _stream(stream)))


def decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size, stream=None):
    """pa_decode_noalloc: pa_decode with its partial results in the library's fixed
    per-GPU scratch array (no allocation)."""
    lib = load()
    ts = [_device_tensor(x, n) for x, n in ((out, "out"), (q, "q"), (k_cache, "k_cache"),
                                           (v_cache, "v_cache"), (block_tables, "block_tables"),
                                           (context_lens, "context_lens"))]
    ds = [describe(x) for x in ts]
    _check(lib, lib.pa_decode_noalloc(*[ctypes.byref(d) for d in ds], ctypes.c_float(scale),
                                      ctypes.c_int32(block_size), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 64 << 20  # PA_NOALLOC_SCRATCH_BYTES in include/pa.h


def workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                    partition_tokens=0):
    return int(load().pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                max_context_len, partition_tokens))


def schedule(num_seqs, num_q_heads, num_kv_heads, max_context_len):
    """Partition choice of an automatic call: -1 no split, -2 stream-K, else tokens."""
    lib = load()
    part = ctypes.c_int32(0)
    _check(lib, lib.pa_decode_schedule(num_seqs, num_q_heads, num_kv_heads, max_context_len,
                                       ctypes.byref(part)))
    return int(part.value)


def alloc_workspace(nbytes, device):
    """Zero-filled device workspace for decode_ex (a uint8 tensor; 256-byte aligned)."""
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _event_handle(e):
    """Raw hipEvent_t of a torch.cuda.Event (created on first use by recording it),
    or an integer handle passed through."""
    if isinstance(e, int):
        return e
    if e.cuda_event == 0:
        e.record()  # torch creates the HIP event on its first record
    h = int(e.cuda_event)
    if h == 0:
        raise PaError(PA_ERR_INVALID, "could not create the timing event")
    return h


def _host_lens(host_context_lens, context_lens):
    """A host copy of context_lens as a contiguous int32 array (kept alive by the caller
    for the call), or None."""
    if host_context_lens is None:
        return None
    if isinstance(host_context_lens, torch.Tensor):
        if host_context_lens.device.type != "cpu":
            raise ValueError("host_context_lens must live in host memory")
        host_context_lens = host_context_lens.numpy()
    a = np.ascontiguousarray(host_context_lens, dtype=np.int32)
    if a.ndim != 1 or a.shape[0] != context_lens.shape[0]:
        raise ValueError(f"host_context_lens: {context_lens.shape[0]} entries expected, got shape {a.shape}")
    return a


def _opts(partition_tokens, path, max_context_len, workgroups_per_cu, kernel_events, host_lens):
    ev = (None, None)
    if kernel_events is not None:
        ev = tuple(_event_handle(e) for e in kernel_events)
    return PaDecodeOpts(int(partition_tokens), int(path), int(max_context_len), int(workgroups_per_cu), 0,
                        ev[0], ev[1], None if host_lens is None else host_lens.ctypes.data)


def decode_ex(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size, *,
              partition_tokens=0, path=0, max_context_len=0, workgroups_per_cu=0, workspace=None,
              kernel_events=None, host_context_lens=None, stream=None):
    """pa_decode_ex: decode with options and a caller-owned workspace.

    kernel_events: optional (start, stop) pair of timing events (torch.cuda.Event with
    enable_timing=True, or raw hipEvent_t handles) that then time the main decode
    kernel alone on the GPU.
    host_context_lens: optional host copy of context_lens (numpy / list / CPU tensor);
    unsplit schedules then rank the sequences on the host.
    """
    lib = load()
    ts = [_device_tensor(x, n) for x, n in ((out, "out"), (q, "q"), (k_cache, "k_cache"),
                                           (v_cache, "v_cache"), (block_tables, "block_tables"),
                                           (context_lens, "context_lens"))]
    ds = [describe(x) for x in ts]
    hl = _host_lens(host_context_lens, context_lens)
    opts = _opts(partition_tokens, path, max_context_len, workgroups_per_cu, kernel_events, hl)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(lib, lib.pa_decode_ex(*[ctypes.byref(d) for d in ds], ctypes.c_float(scale),
                                 ctypes.c_int32(block_size), ctypes.byref(opts),
                                 ctypes.c_void_p(ws_ptr) if ws_ptr else None,
                                 ctypes.c_size_t(ws_bytes), _stream(stream)))


def append_decode(out, q, k, v, slot_mapping, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                  *, partition_tokens=0, path=0, max_context_len=0, workgroups_per_cu=0, workspace=None,
                  kernel_events=None, host_context_lens=None, stream=None):
    """pa_append_decode: this step's k/v [S, Hkv, D] appended at slot_mapping [S], then the
    decode of q [S, Hq, D], as one call (one launch where the schedule is unsplit MFMA)."""
    lib = load()
    ts = [_device_tensor(x, n) for x, n in (
        (out, "out"), (q, "q"), (k, "k"), (v, "v"), (slot_mapping, "slot_mapping"), (k_cache, "k_cache"),
        (v_cache, "v_cache"), (block_tables, "block_tables"), (context_lens, "context_lens"))]
    ds = [describe(x) for x in ts]
    hl = _host_lens(host_context_lens, context_lens)
    opts = _opts(partition_tokens, path, max_context_len, workgroups_per_cu, kernel_events, hl)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(lib, lib.pa_append_decode(*[ctypes.byref(d) for d in ds], ctypes.c_float(scale),
                                     ctypes.c_int32(block_size), ctypes.byref(opts),
                                     ctypes.c_void_p(ws_ptr) if ws_ptr else None,
                                     ctypes.c_size_t(ws_bytes), _stream(stream)))


def last_launch():
    """Kernels the last library call on this thread enqueued (pa_last_launch), as a list."""
    return load().pa_last_launch().decode().split()


def set_debug(on):
    return bool(load().pa_set_debug(1 if on else 0))
