"""The C ABI without a GPU: libpa.so loads, exports every function include/pa.h
declares, and rejects invalid arguments with the documented status codes
before touching any device memory (the descriptors below point nowhere)."""

import ctypes
import os
import re

import pytest

torch = pytest.importorskip("torch")

from paged_kv_cache_122_amd import _lib as pa  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")
FAKE = 0x7F0000000000  # aligned, never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pa.LIB_PATH):
        pytest.skip("libpa.so not built")
    return pa.load()


def T(shape, dtype, data=FAKE, stride=None):
    d = pa.PaTensor()
    d.data = data
    d.dtype = dtype
    d.ndim = len(shape)
    if stride is None:
        stride, acc = [], 1
        for n in reversed(shape):
            stride.insert(0, acc)
            acc *= n
    for i, n in enumerate(shape):
        d.shape[i] = n
        d.stride[i] = stride[i]
    return d


def decode_args(S=4, Hq=8, Hkv=2, D=128, B=16, NB=64, W=8, qdt=pa.PA_BF16, kdt=pa.PA_BF16,
                out_dt=pa.PA_BF16):
    return dict(
        out=T([S, Hq, D], out_dt), q=T([S, Hq, D], qdt),
        k=T([NB, Hkv, D // 8, B, 8], kdt), v=T([NB, Hkv, B // 4, D, 4], pa.PA_BF16),
        bt=T([S, W], pa.PA_I32), lens=T([S], pa.PA_I32))


def call_decode(lib, a, scale=0.1, block_size=16):
    r = ctypes.byref
    return lib.pa_decode(r(a["out"]), r(a["q"]), r(a["k"]), r(a["v"]), r(a["bt"]), r(a["lens"]),
                         scale, block_size, None)


def call_decode_ex(lib, a, opts, ws=None, ws_bytes=0, block_size=16):
    r = ctypes.byref
    return lib.pa_decode_ex(r(a["out"]), r(a["q"]), r(a["k"]), r(a["v"]), r(a["bt"]), r(a["lens"]),
                            0.1, block_size, r(opts), ws, ws_bytes, None)


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted(pa.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {pa.LIB_PATH}").read()
    exported = set(re.findall(r"\bT (pa_[a-z_]+)\b", out))
    assert exported == set(declared_functions())


def test_validation_errors(lib):
    r = ctypes.byref
    a = decode_args()
    a["out"] = None
    rc = lib.pa_decode(None, r(a["q"]), r(a["k"]), r(a["v"]), r(a["bt"]), r(a["lens"]), 0.1, 16, None)
    assert rc == pa.PA_ERR_INVALID and b"out" in lib.pa_last_error()

    assert call_decode(lib, decode_args(kdt=pa.PA_F32)) == pa.PA_ERR_INVALID
    assert call_decode(lib, decode_args(qdt=pa.PA_F32)) == pa.PA_ERR_INVALID
    assert call_decode(lib, decode_args(out_dt=pa.PA_I32)) == pa.PA_ERR_INVALID
    assert call_decode(lib, decode_args(D=96)) == pa.PA_ERR_UNSUPPORTED
    assert call_decode(lib, decode_args(B=64), block_size=64) == pa.PA_ERR_UNSUPPORTED
    assert call_decode(lib, decode_args(Hq=7)) == pa.PA_ERR_INVALID
    assert call_decode(lib, decode_args(), block_size=8) == pa.PA_ERR_INVALID
    a = decode_args()
    a["lens"] = T([3], pa.PA_I32)
    assert call_decode(lib, a) == pa.PA_ERR_INVALID
    a = decode_args()
    a["k"] = T([64, 2, 16, 16, 8], pa.PA_BF16, stride=[4096 * 2, 2048, 128, 8, 1])  # not contiguous
    assert call_decode(lib, a) == pa.PA_ERR_INVALID
    a = decode_args()
    a["q"] = T([4, 8, 128], pa.PA_BF16, data=FAKE + 2)  # misaligned rows
    assert call_decode(lib, a) == pa.PA_ERR_INVALID
    assert call_decode(lib, decode_args(), scale=float("inf")) == pa.PA_ERR_INVALID

    # options: VALU path takes at most 2 q heads per KV head; partitions are multiples of 32
    assert call_decode_ex(lib, decode_args(), pa.PaDecodeOpts(0, 1, 0)) == pa.PA_ERR_UNSUPPORTED
    assert call_decode_ex(lib, decode_args(), pa.PaDecodeOpts(48, 0, 0)) == pa.PA_ERR_INVALID
    assert call_decode_ex(lib, decode_args(), pa.PaDecodeOpts(0, 3, 0)) == pa.PA_ERR_INVALID
    # W*B = 2048 tokens -> 4 partitions of 512, or the stream-K schedule: a workspace is
    # required, and a missing or short one is rejected before anything is launched
    for part in (512, -2):
        assert call_decode_ex(lib, decode_args(W=128), pa.PaDecodeOpts(part, 0, 0)) == pa.PA_ERR_WORKSPACE
        assert call_decode_ex(lib, decode_args(W=128), pa.PaDecodeOpts(part, 0, 0),
                              ctypes.c_void_p(FAKE), 100) == pa.PA_ERR_WORKSPACE
        assert b"workspace" in lib.pa_last_error()
    assert call_decode_ex(lib, decode_args(), pa.PaDecodeOpts(-3, 0, 0)) == pa.PA_ERR_INVALID
    assert call_decode_ex(lib, decode_args(), pa.PaDecodeOpts(0, 0, 0, 65)) == pa.PA_ERR_INVALID
    assert call_decode_ex(lib, decode_args(), pa.PaDecodeOpts(0, 0, 0, 0, 1)) == pa.PA_ERR_INVALID
    # timing events: both or neither
    assert call_decode_ex(lib, decode_args(), pa.PaDecodeOpts(0, 0, 0, 0, 0, 0x1000, None)) == pa.PA_ERR_INVALID
    assert call_decode_ex(lib, decode_args(), pa.PaDecodeOpts(0, 0, 0, 0, 0, None, 0x1000)) == pa.PA_ERR_INVALID


def test_empty_batch_is_a_no_op(lib):
    assert call_decode(lib, decode_args(S=0)) == pa.PA_OK
    r = ctypes.byref
    k = T([0, 2, 64], pa.PA_BF16)
    slots = T([0], pa.PA_I64)
    kc, vc = T([8, 2, 8, 16, 8], pa.PA_BF16), T([8, 2, 4, 64, 4], pa.PA_BF16)
    assert lib.pa_cache_append(r(k), r(k), r(slots), r(kc), r(vc), None) == pa.PA_OK


def test_append_validation(lib):
    r = ctypes.byref
    kc, vc = T([8, 2, 8, 16, 8], pa.PA_BF16), T([8, 2, 4, 64, 4], pa.PA_BF16)
    k = T([3, 2, 64], pa.PA_BF16)
    assert lib.pa_cache_append(r(k), r(k), r(T([3], pa.PA_I32)), r(kc), r(vc), None) == pa.PA_ERR_INVALID
    assert lib.pa_cache_append(r(k), r(T([3, 2, 32], pa.PA_BF16)), r(T([3], pa.PA_I64)), r(kc), r(vc),
                               None) == pa.PA_ERR_INVALID
    assert lib.pa_cache_append(r(k), r(k), r(T([4], pa.PA_I64)), r(kc), r(vc), None) == pa.PA_ERR_INVALID
    assert lib.pa_cache_append(r(T([3, 3, 64], pa.PA_BF16)), r(k), r(T([3], pa.PA_I64)), r(kc), r(vc),
                               None) == pa.PA_ERR_INVALID
    bad_v = T([8, 2, 4, 64, 2], pa.PA_BF16)
    assert lib.pa_cache_append(r(k), r(k), r(T([3], pa.PA_I64)), r(kc), r(bad_v), None) == pa.PA_ERR_INVALID


def test_workspace_bytes(lib):
    f = lib.pa_decode_workspace_bytes
    up = lambda x: (x + 255) // 256 * 256
    # 64 seqs, 32/8 heads, D 128, contexts up to 2048 tokens -> 4 partitions of 512
    # partitioned: (max, sum) pairs then outputs, fp32, per (seq, q head, partition)
    expect = up(4 * 2 * 64 * 32 * 4) + up(4 * 64 * 32 * 4 * 128)
    assert f(64, 32, 8, 128, 2048, 512) == expect
    assert f(64, 32, 8, 128, 512, 512) == 0        # one partition: no workspace
    assert f(64, 32, 8, 128, 2048, -1) == 0        # never split
    assert f(8, 32, 8, 128, 32768, 512) == up(4 * 2 * 8 * 32 * 64) + up(4 * 8 * 32 * 64 * 128)
    # stream-K: plan (4 + S + 1 ints), then 16-column pieces for (pairs + 4096
    # waves): (max, sum) and outputs
    def stream_bytes(S, Hq, Hkv, D):
        pairs = S * Hkv * -(-(Hq // Hkv) // 16)
        pieces = (pairs + 4096) * 16
        return up(4 * (S + 5)) + up(4 * 2 * pieces) + up(4 * pieces * D)
    for S, Hq, Hkv, D in ((64, 32, 8, 128), (256, 64, 8, 128), (4, 8, 2, 64), (3, 64, 2, 128)):
        assert f(S, Hq, Hkv, D, 2048, -2) == stream_bytes(S, Hq, Hkv, D)
    # automatic schedule, from the shapes alone
    assert f(64, 32, 8, 128, 2048, 0) == 0                                 # 512 pairs: no split
    assert f(128, 40, 40, 128, 2048, 0) == f(128, 40, 40, 128, 2048, 1024)  # MHA: 1024-token parts
    assert f(4, 8, 2, 64, 912, 0) == 0                                      # tiny: no split
    assert f(8, 32, 8, 128, 32768, 0) == stream_bytes(8, 32, 8, 128)        # few long contexts
    assert f(64, 32, 8, 128, 16384, 0) == f(64, 32, 8, 128, 16384, 1024)   # long, many pairs
    assert f(9000, 32, 8, 128, 16384, 0) == up(4 * 2 * 9000 * 32 * 16) + up(4 * 9000 * 32 * 16 * 128)
    # too many sequences for the stream-K prefix: few pairs fall back to 512-token partitions
    assert f(9000, 8, 8, 128, 1024, -2) == 0


def test_schedule_query(lib):
    s = lambda *a: pa.schedule(*a)  # noqa: E731
    assert s(64, 32, 8, 2048) == -1          # 512 (sequence, head group) pairs: no split
    assert s(256, 64, 8, 8192) == -1
    assert s(128, 40, 40, 2048) == 1024      # MHA with many pairs: 1024-token partitions
    assert s(64, 32, 8, 16384) == 1024       # long contexts, many pairs
    assert s(4, 8, 2, 912) == -1             # tiny batch
    assert s(60, 32, 8, 1024) == -1         # few pairs, short tables: no split
    assert s(1, 32, 8, 8192) == 512          # one long context: 512-token partitions (128 workgroups)
    assert s(32, 32, 8, 2048) == 512         # 256 pairs x 4 partitions
    assert s(16, 32, 8, 6016) == 512         # 1536 workgroups
    assert s(16, 32, 8, 32768) == -2         # 8192 workgroups of 512 tokens: stream-K
    assert s(8, 32, 8, 32768) == -2          # few long contexts: stream-K
    assert s(9000, 64, 8, 1024) == -1        # 72000 pairs
    assert s(9000, 2, 1, 1 << 20) == 1024
    with pytest.raises(pa.PaError) as e:
        s(4, 6, 4, 100)
    assert e.value.code == pa.PA_ERR_INVALID
    # every automatic choice is consistent with the workspace size query
    for args in ((64, 32, 8, 2048), (128, 40, 40, 2048), (8, 32, 8, 32768), (64, 32, 8, 16384),
                 (1, 32, 8, 8192), (16, 32, 8, 6016)):
        S, Hq, Hkv, L = args
        assert lib.pa_decode_workspace_bytes(S, Hq, Hkv, 128, L, 0) == \
            lib.pa_decode_workspace_bytes(S, Hq, Hkv, 128, L, s(*args))


def test_copy_blocks_validation(lib):
    """pa_copy_blocks checks its arguments before any launch (fake pointers here)."""
    r = ctypes.byref
    a = decode_args()

    def call(pairs):
        return lib.pa_copy_blocks(r(a["k"]), r(a["v"]), r(pairs), None)

    assert call(T([0, 2], pa.PA_I64)) == pa.PA_OK                        # nothing to copy
    assert call(T([3, 2], pa.PA_I32)) == pa.PA_ERR_INVALID               # int64 pairs
    assert call(T([3, 3], pa.PA_I64)) == pa.PA_ERR_INVALID               # [N, 2]
    assert call(T([3, 2], pa.PA_I64, stride=[4, 1])) == pa.PA_ERR_INVALID  # contiguous rows
    assert call(T([3, 2], pa.PA_I64, data=None)) == pa.PA_ERR_INVALID
    bad = decode_args(kdt=pa.PA_F32)
    assert lib.pa_copy_blocks(r(bad["k"]), r(bad["v"]), r(T([3, 2], pa.PA_I64)), None) == pa.PA_ERR_INVALID


def test_decode_contiguous_validation(lib):
    """pa_decode_contiguous checks shapes before any launch (fake pointers here)."""
    r = ctypes.byref

    def call(S=4, Hq=8, Hkv=2, D=128, T=4, kshape=None, vshape=None, lens=None, scale=0.1):
        out, q = T_([S, Hq, D], pa.PA_BF16), T_([S, Hq, D], pa.PA_BF16)
        k = T_(kshape or [S * Hkv, T, D // 8, 16, 8], pa.PA_BF16)
        v = T_(vshape or [S * Hkv, T, 4, D, 4], pa.PA_BF16)
        ln = T_([lens if lens is not None else S], pa.PA_I32)
        return lib.pa_decode_contiguous(r(out), r(q), r(k), r(v), r(ln), scale, None)

    assert call(S=0, kshape=[0, 4, 16, 16, 8], vshape=[0, 4, 4, 128, 4], lens=0) == pa.PA_OK
    assert call(kshape=[8, 4, 16, 16, 4]) == pa.PA_ERR_INVALID          # last dim 8
    assert call(kshape=[8, 4, 16, 8, 8]) == pa.PA_ERR_INVALID           # 16-token tiles
    assert call(kshape=[7, 4, 16, 16, 8]) == pa.PA_ERR_INVALID          # S * Hkv
    assert call(vshape=[8, 3, 4, 128, 4]) == pa.PA_ERR_INVALID          # matches k
    assert call(D=96, kshape=[8, 4, 12, 16, 8], vshape=[8, 4, 4, 96, 4]) == pa.PA_ERR_UNSUPPORTED
    assert call(Hq=7) == pa.PA_ERR_INVALID
    assert call(lens=3) == pa.PA_ERR_INVALID
    assert call(scale=float("nan")) == pa.PA_ERR_INVALID


T_ = T


def test_decode_multi_validation(lib):
    """pa_decode_multi checks shapes before any launch (fake pointers here: every
    call either fails validation or is a no-op)."""
    r = ctypes.byref

    def call(S=4, T=10, Hq=8, Hkv=2, D=128, B=16, NB=64, W=8, mql=5, scale=0.1, block_size=16,
             kn=None, qs=None, slots=None, out_dt=pa.PA_BF16, qs_dt=pa.PA_I32):
        out, q = T_([T, Hq, D], out_dt), T_([T, Hq, D], pa.PA_BF16)
        k_new = T_(kn or [T, Hkv, D], pa.PA_BF16)
        v_new = T_([T, Hkv, D], pa.PA_BF16)
        sl = T_([slots if slots is not None else T], pa.PA_I64)
        qst = T_([qs if qs is not None else S + 1], qs_dt)
        kc, vc = T_([NB, Hkv, D // 8, B, 8], pa.PA_BF16), T_([NB, Hkv, B // 4, D, 4], pa.PA_BF16)
        bt, ln = T_([S, W], pa.PA_I32), T_([S], pa.PA_I32)
        return lib.pa_decode_multi(r(out), r(q), r(k_new), r(v_new), r(sl), r(qst), r(kc), r(vc),
                                   r(bt), r(ln), scale, block_size, mql, None)

    assert call(S=0) == pa.PA_OK                                   # nothing to do
    assert call(T=0) == pa.PA_OK
    assert call(mql=0) == pa.PA_OK
    assert call(kn=[10, 3, 128]) == pa.PA_ERR_INVALID              # KV heads of the pools
    assert call(kn=[9, 2, 128]) == pa.PA_ERR_INVALID               # one row per q row
    assert call(slots=9) == pa.PA_ERR_INVALID
    assert call(qs=4) == pa.PA_ERR_INVALID                         # S + 1 entries
    assert call(qs_dt=pa.PA_I64) == pa.PA_ERR_INVALID
    assert call(out_dt=pa.PA_I32) == pa.PA_ERR_INVALID
    assert call(Hq=7) == pa.PA_ERR_INVALID
    assert call(block_size=32) == pa.PA_ERR_INVALID
    assert call(mql=-1) == pa.PA_ERR_INVALID
    assert call(mql=1 << 22, Hq=32) == pa.PA_ERR_INVALID           # columns past 2^24
    assert call(scale=float("inf")) == pa.PA_ERR_INVALID
    assert call(D=96) == pa.PA_ERR_UNSUPPORTED                      # pools reject the head size


def test_append_decode_validation(lib):
    """pa_append_decode checks the append's and the decode's arguments, and the
    workspace, before anything is launched (fake pointers here)."""
    r = ctypes.byref

    def call(a=None, kshape=None, slots=None, opts=None, ws=None, ws_bytes=0, kdt=pa.PA_BF16):
        a = a or decode_args()
        S, Hkv, D = a["q"].shape[0], a["k"].shape[1], a["q"].shape[2]
        k = T(kshape or [S, Hkv, D], kdt)
        v = T([S, Hkv, D], pa.PA_BF16)
        sl = T([S if slots is None else slots], pa.PA_I64)
        return lib.pa_append_decode(r(a["out"]), r(a["q"]), r(k), r(v), r(sl), r(a["k"]), r(a["v"]),
                                    r(a["bt"]), r(a["lens"]), 0.1, 16, r(opts) if opts else None, ws,
                                    ws_bytes, None)

    assert call(decode_args(S=0)) == pa.PA_OK                              # nothing to do
    assert call(kshape=[4, 3, 128]) == pa.PA_ERR_INVALID                    # KV heads of the pools
    assert call(kshape=[3, 2, 128]) == pa.PA_ERR_INVALID                    # one new token per sequence
    assert call(kdt=pa.PA_F32) == pa.PA_ERR_INVALID
    assert call(slots=5) == pa.PA_ERR_INVALID
    bad = decode_args()
    bad["lens"] = T([3], pa.PA_I32)
    assert call(bad) == pa.PA_ERR_INVALID                                   # decode arguments too
    # a split schedule needs the caller's workspace: rejected before the append runs
    assert call(decode_args(W=128), opts=pa.PaDecodeOpts(512, 0, 0)) == pa.PA_ERR_WORKSPACE
    assert call(decode_args(W=128), opts=pa.PaDecodeOpts(512, 0, 0), ws=ctypes.c_void_p(FAKE),
                ws_bytes=100) == pa.PA_ERR_WORKSPACE


def test_host_context_lens_marshalling():
    """opts.host_context_lens: the binding hands the library a contiguous int32
    host array with one entry per sequence, or NULL."""
    import numpy as np
    import torch

    lens = torch.zeros(4, dtype=torch.int32)
    assert pa._host_lens(None, lens) is None
    a = pa._host_lens([3, 1, 4, 1], lens)
    assert a.dtype == np.int32 and a.flags["C_CONTIGUOUS"] and a.tolist() == [3, 1, 4, 1]
    b = pa._host_lens(torch.tensor([5, 9, 2, 6], dtype=torch.int64), lens)
    assert b.dtype == np.int32 and b.tolist() == [5, 9, 2, 6]
    strided = np.arange(8, dtype=np.int32)[::2]
    assert pa._host_lens(strided, lens).tolist() == [0, 2, 4, 6]
    with pytest.raises(ValueError):
        pa._host_lens([1, 2, 3], lens)
    with pytest.raises(ValueError):
        pa._host_lens(np.zeros((2, 2), dtype=np.int32), lens)
    o = pa._opts(0, 0, 0, 0, None, a)
    assert o.host_context_lens == a.ctypes.data
    assert pa._opts(0, 0, 0, 0, None, None).host_context_lens is None
    assert ctypes.sizeof(pa.PaDecodeOpts) == 48


def test_decode_multi_ex_validation(lib):
    """pa_decode_multi_ex checks its options and the workspace before any launch
    (fake pointers: every call fails validation or is a no-op)."""
    r = ctypes.byref

    def call(opts=None, ws=None, ws_bytes=0, S=4, T=10, W=8, Hq=8, Hkv=2, D=128, B=16, NB=64, mql=5):
        out, q = T_([T, Hq, D], pa.PA_BF16), T_([T, Hq, D], pa.PA_BF16)
        k_new, v_new = T_([T, Hkv, D], pa.PA_BF16), T_([T, Hkv, D], pa.PA_BF16)
        sl, qst = T_([T], pa.PA_I64), T_([S + 1], pa.PA_I32)
        kc, vc = T_([NB, Hkv, D // 8, B, 8], pa.PA_BF16), T_([NB, Hkv, B // 4, D, 4], pa.PA_BF16)
        bt, ln = T_([S, W], pa.PA_I32), T_([S], pa.PA_I32)
        return lib.pa_decode_multi_ex(r(out), r(q), r(k_new), r(v_new), r(sl), r(qst), r(kc), r(vc), r(bt), r(ln),
                                      0.1, B, mql, r(opts) if opts is not None else None, ws, ws_bytes, None)

    O = pa.PaDecodeOpts
    assert call(O(0, 1, 0)) == pa.PA_ERR_UNSUPPORTED          # VALU: the multi-token kernels are MFMA only
    assert call(O(0, 3, 0)) == pa.PA_ERR_INVALID
    assert call(O(-2, 0, 0)) == pa.PA_ERR_UNSUPPORTED         # no stream-K for several new tokens
    assert call(O(48, 0, 0)) == pa.PA_ERR_INVALID             # not a multiple of 32
    assert call(O(-3, 0, 0)) == pa.PA_ERR_INVALID
    assert call(O(0, 0, -1)) == pa.PA_ERR_INVALID             # max_context_len < 0
    assert call(O(0, 0, 0, 1)) == pa.PA_ERR_INVALID           # workgroups_per_cu
    assert call(O(0, 0, 0, 0, 1)) == pa.PA_ERR_INVALID        # reserved
    assert call(O(0, 0, 0, 0, 0, 0x1000, None)) == pa.PA_ERR_INVALID
    assert call(O(0, 0, 0), S=0) == pa.PA_OK                  # nothing to do
    # 8 (sequence, KV head) pairs over 8192-token tables split: the workspace is checked
    need = lib.pa_decode_multi_workspace_bytes(10, 4, 8, 2, 128, 5, 512 * 16, 0)
    assert need > 0
    assert call(O(0, 0, 0), W=512) == pa.PA_ERR_WORKSPACE
    assert call(O(0, 0, 0), W=512, ws=0x1000, ws_bytes=need - 256) == pa.PA_ERR_WORKSPACE
    assert call(O(0, 0, 0), W=512, ws=0x1010, ws_bytes=need) == pa.PA_ERR_WORKSPACE   # not 256-byte aligned
    assert call(None, W=512) == pa.PA_ERR_WORKSPACE


def test_multi_workspace_bytes(lib):
    f = lib.pa_decode_multi_workspace_bytes
    up = lambda x: (x + 255) // 256 * 256
    # 8 seqs x 5 rows (40), 32 q / 8 kv heads: 20 columns in one workgroup per KV head, 64 pairs; the
    # automatic split cuts 32k-token contexts into partitions of 4096 (about 512 workgroups)
    assert f(40, 8, 32, 8, 128, 5, 32768, 0) == up(4 * 2 * 40 * 32 * 8) + up(4 * 40 * 32 * 8 * 128)
    assert f(40, 8, 32, 8, 128, 5, 32768, 2048) == up(4 * 2 * 40 * 32 * 16) + up(4 * 40 * 32 * 16 * 128)
    assert f(40, 8, 32, 8, 128, 5, 32768, -1) == 0            # never split
    assert f(320, 64, 32, 8, 128, 5, 2048, 0) == 0            # 512 pairs: no split
    assert f(40, 8, 32, 8, 128, 5, 512, 0) == 0               # one partition: no split
    assert f(40, 8, 32, 8, 128, 5, 1024, 1024) == 0           # partition as long as the bound
    assert f(0, 8, 32, 8, 128, 5, 32768, 0) == 0
    assert f(40, 8, 30, 8, 128, 5, 32768, 0) == 0             # heads not a multiple


def test_decode_noalloc_validation(lib):
    """pa_decode_noalloc validates like pa_decode and refuses, before any device
    call, a schedule whose partial results exceed its fixed scratch (fake
    pointers: every call below fails validation)."""
    r = ctypes.byref

    def call(a, block_size=16):
        return lib.pa_decode_noalloc(r(a["out"]), r(a["q"]), r(a["k"]), r(a["v"]), r(a["bt"]), r(a["lens"]),
                                     0.1, block_size, None)

    assert call(decode_args(Hq=7)) == pa.PA_ERR_INVALID
    assert call(decode_args(D=96)) == pa.PA_ERR_UNSUPPORTED
    assert call(decode_args(), block_size=8) == pa.PA_ERR_INVALID
    # 4096 sequences in 32k-token tables: 32 partitions of 1024 tokens per (sequence, q head)
    big = decode_args(S=4096, Hq=32, Hkv=8, W=2048)
    need = lib.pa_decode_workspace_bytes(4096, 32, 8, 128, 2048 * 16, 0)
    assert need > pa.NOALLOC_SCRATCH_BYTES
    assert call(big) == pa.PA_ERR_WORKSPACE
    assert b"scratch" in lib.pa_last_error()
    assert call(decode_args(S=0)) == pa.PA_OK  # nothing to do, no scratch needed


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define PA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == pa.NOALLOC_SCRATCH_BYTES
