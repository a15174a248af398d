"""Benchmark of one paged-decode layer step on one MI355X: slot-mapped append of
this step's K/V and paged decode attention, as one pa_append_decode call (one
launch where the decode schedule is unsplit MFMA, else the append kernel and
then the decode schedule).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]

Prints ONE JSON line.  ``value`` is effective KV-read GB/s of the whole step
(sum_s L_s * Hkv * D * 2 (K and V) * 2 bytes, divided by the event-timed step).  Inputs are resident in HBM; before every timed step a
1 GiB buffer is written so that neither L2 nor the 256 MB Infinity Cache
still holds the pools (the flush is outside the timed region).  All work runs
on one stream of this process and the HIP events are recorded on it; they are
created with hipEventDisableSystemFence, so recording them flushes no cache.
``roofline`` is the step's main kernel alone (on the default workload the
only kernel of the step), timed in as many further flushed steps by events
that the GPU stamps at its start and end, against 8 TB/s.  ``two_call_step``
times the same step as pa_cache_append + pa_decode.  ``paging_control``
times the same decode over an unpaged copy of the cache; ``multi_query`` times
pa_decode_multi (several new tokens per sequence: speculative verification)
on the Llama-3-8B-shaped batch with 5 drafted tokens per sequence, and
``multi_query_long`` on 8 sequences of 32k tokens with 5 drafted tokens each.  ``cpu_baseline`` is the fp64 oracle on a bounded
sample of the same workload, on this host's CPU.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
DEFAULT_CONFIG = "llama3_8b_b64"

# HBM bytes per launch of a step's main kernel, from two rocprofv3
# --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE), each scaled by what
# the counter reads for a plain copy of known size in the same run, and the
# kernel's MFMA busy share of SIMD cycles from a third.  Valid only
# for the kernel sources they were taken on (sha256 of the files below);
# reported as null once those change.
KERNEL_SOURCES = ("paged_kv_cache_122_amd/csrc/pa_kernels.hip",
                  "paged_kv_cache_122_amd/csrc/pa_internal.h")
MEASURED_TRAFFIC = {
    "sources_sha256": "dda88c1be23a894d5f48580224cc48df885709af8c29550d23978e4a1f8933a8",
    # the step's one launch: FETCH_SIZE 133788.2 KiB x 1.9999, WRITE_SIZE 1280.1 KiB x 1.0;
    # MfmaUtil (SQ_VALU_MFMA_BUSY_CYCLES over SIMD cycles) 4.66 %
    "llama3_8b_b64 decode_multi<128,16,1,false>": {"fetch_bytes": 273979547, "write_bytes": 1310784,
                                                   "mfma_busy_pct": 4.66},
    # the verification batch: FETCH_SIZE 140627.6 KiB x 1.9999, WRITE_SIZE 4353.6 KiB x 1.0; MfmaUtil 8.56 %
    "llama3_8b_verify5_b64 decode_multi<128,16,2,false>": {"fetch_bytes": 287985629, "write_bytes": 4458048,
                                                           "mfma_busy_pct": 8.56},
    # long-context verification (split): FETCH_SIZE 524893.5 KiB x 1.9999, WRITE_SIZE 5426.6 KiB x 1.0;
    # MfmaUtil 11.59 %
    "long32k_verify5_b16 decode_multi<128,16,2,true>": {"fetch_bytes": 1074908611, "write_bytes": 5556827,
                                                        "mfma_busy_pct": 11.59},
    # the --config steps' main kernels (bench.py --config X --steps 5 --warmup 2 --no-cpu-baseline
    # --no-control --no-multi --copy-calibration 256, one counter per run):
    # Llama-3-70B-shaped: FETCH_SIZE 442993.4 KiB x 1.9999, WRITE_SIZE 7168.0 KiB x 1.0
    "llama3_70b_b256 decode_multi<128,16,1,false>": {"fetch_bytes": 907196049, "write_bytes": 7340032},
    # OPT-13B-shaped prefix sharing: FETCH_SIZE 852223.5 KiB x 1.9999, WRITE_SIZE 5380.3 KiB x 1.0
    "opt13b_mha_prefix_b128 decode_shared<128,16,true>": {"fetch_bytes": 1745252744, "write_bytes": 5509477},
    # 8 x 32k tokens, B 16: FETCH_SIZE 524706.4 KiB x 1.9999, WRITE_SIZE 1136.2 KiB x 1.0
    "long32k_b16 decode_multi<128,16,1,true>": {"fetch_bytes": 1074533797, "write_bytes": 1163493},
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default=DEFAULT_CONFIG)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--no-multi", action="store_true",
                    help="skip the multi-token (speculative verification) leg")
    ap.add_argument("--no-control", action="store_true",
                    help="skip the unpaged control (pa_decode_contiguous on a copy of the cache)")
    ap.add_argument("--unflushed", action="store_true",
                    help="also time back-to-back steps without the cache flush")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the benchmark, copy a float32 buffer of this many MiB three "
                         "times (a known-size kernel for scaling HBM byte counters)")
    return ap.parse_args()


class TimingEvents:
    """HIP events used only for timing, created with hipEventDisableSystemFence:
    recording one then adds no system-scope cache writeback and invalidation to
    the timed work (a default event does, and a kernel launched with default
    events runs measurably longer).  They live in the HIP runtime torch loaded."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []

    def _check(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def create(self):
        e = self.ct.c_void_p()
        self._check(self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.DISABLE_SYSTEM_FENCE),
                    "hipEventCreateWithFlags")
        self.events.append(e.value)
        return e.value

    def record(self, e, stream):
        self._check(self.hip.hipEventRecord(e, stream.cuda_stream), "hipEventRecord")

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        self._check(self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b), "hipEventElapsedTime")
        return ms.value

    def close(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []


def sources_sha256():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured(config, kernel):
    """The counter figures for this workload's kernel, if taken on these sources."""
    t = MEASURED_TRAFFIC
    key = f"{config} {kernel}"
    if key not in t or t["sources_sha256"] != sources_sha256():
        return None
    return t[key]


def measured_traffic(config, kernel):
    m = measured(config, kernel)
    return None if m is None else m["fetch_bytes"] + m["write_bytes"]


def measured_mfma(config, kernel):
    m = measured(config, kernel)
    return None if m is None else m.get("mfma_busy_pct")


def decode_kernels(w, part, cus):
    """Kernels one automatic pa_decode call launches on this workload."""
    g = w.num_q_heads // w.num_kv_heads
    core = f"decode_{'mfma' if g >= 3 else 'valu'}"
    tmpl = f"<{w.head_dim},{w.block_size}>"
    if part == -2:
        return [core + "_sk" + tmpl, f"combine_sk<{w.head_dim}>"], "stream-K"
    max_len = w.block_tables.shape[1] * w.block_size
    parts = 1 if part == -1 else -(-max_len // part)
    if g >= 3:  # pipeline slots: two once the grid has a workgroup per compute unit
        wgs = w.num_seqs * w.num_kv_heads * -(-g // 16) * parts
        tmpl = f"<{w.head_dim},{w.block_size},{2 if wgs >= cus else 4}>"
    if parts == 1:
        return [core + tmpl], "one workgroup per (sequence, head group), no split"
    wgs = w.num_seqs * w.num_kv_heads * -(-g // 16) * parts
    if g <= 16 and wgs >= cus:  # split schedules read shared partitions once
        return ([f"decode_shared<{w.head_dim},{w.block_size},false>", f"combine_parts<{w.head_dim}>"],
                f"partitions of {part} tokens, shared partitions read once")
    return [core + tmpl, f"combine_parts<{w.head_dim}>"], f"partitions of {part} tokens"


MULTI_CONFIGS = (("llama3_8b_verify5_b64", "decode_multi<128,16,2,false>"),
                 ("long32k_verify5_b16", "decode_multi<128,16,2,true>"))


def multi_query_leg(config, kernel, steps, warmup, tev, stream, flush):
    """pa_decode_multi on a verification batch (5 drafted tokens per sequence):
    the append of the drafted tokens and their causal attention, one launch
    (and a combine when the context is split).  Beside it, pa_decode of one
    token per sequence over the same pools (same KV bytes).  Each call after a
    cache flush, timed by events around it."""
    import numpy as np
    import torch

    from paged_kv_cache_122_amd import _lib as pa
    from paged_kv_cache_122_amd import device as dev
    from paged_kv_cache_122_amd import workloads

    w = workloads.make(config)
    dw = dev.upload(w, "cuda:0")
    counts = np.diff(w.query_start)
    mql = int(counts.max())
    out = torch.empty_like(dw.q)
    first = dw.query_start[:-1].long()
    q1 = dw.q[first].contiguous()
    out1 = torch.empty_like(q1)

    def multi():
        pa.decode_multi(out, dw.q, dw.k_new, dw.v_new, dw.slot_mapping, dw.query_start, dw.k_cache,
                        dw.v_cache, dw.block_tables, dw.context_lens, w.scale, w.block_size, mql,
                        stream=stream)

    def single():
        pa.decode(out1, q1, dw.k_cache, dw.v_cache, dw.block_tables, dw.context_lens, w.scale,
                  w.block_size, stream=stream)

    E = tev.create
    for _ in range(warmup):
        flush.zero_()
        multi()
        single()
    ev = [(E(), E(), E(), E()) for _ in range(steps)]
    for a, b, c, d in ev:
        flush.zero_()
        tev.record(a, stream)
        multi()
        tev.record(b, stream)
        flush.zero_()
        tev.record(c, stream)
        single()
        tev.record(d, stream)
    stream.synchronize()
    multi_ms = [tev.elapsed_ms(a, b) for a, b, _, _ in ev]
    single_ms = [tev.elapsed_ms(c, d) for _, _, c, d in ev]
    # the main kernel alone: pa_decode_multi_ex with the caller's workspace,
    # the host copy of the lengths and GPU-stamped events around the kernel
    T = int(w.q.shape[0])
    span = int(w.block_tables.shape[1]) * w.block_size
    nb = pa.multi_workspace_bytes(T, w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, mql, span, 0)
    ws = pa.alloc_workspace(nb, "cuda:0") if nb else None
    host_lens = np.asarray(w.context_lens, dtype=np.int32)
    kev = [(E(), E()) for _ in range(steps)]
    for a, b in kev:
        flush.zero_()
        pa.decode_multi_ex(out, dw.q, dw.k_new, dw.v_new, dw.slot_mapping, dw.query_start, dw.k_cache,
                           dw.v_cache, dw.block_tables, dw.context_lens, w.scale, w.block_size, mql,
                           workspace=ws, kernel_events=(a, b), host_context_lens=host_lens, stream=stream)
    stream.synchronize()
    kernel_ms = [tev.elapsed_ms(a, b) for a, b in kev]
    new_kv = T * w.num_kv_heads * w.head_dim * 2 * 2
    # K/V of every context token read once (cached ones from the pool, new ones
    # from k_new / v_new), the new K/V written, q read and out written
    algo = w.unique_kv_bytes() + new_kv + 2 * T * w.num_q_heads * w.head_dim * 2
    mean = lambda xs: sum(xs) / len(xs)  # noqa: E731
    t = mean(multi_ms) / 1e3
    tk = mean(kernel_ms) / 1e3
    del dw, ws
    return {
        "workload": w.name,
        "num_seqs": w.num_seqs,
        "new_tokens": T,
        "max_query_len": mql,
        "context_tokens": int(w.context_lens.sum()),
        "call_ms": {"mean": round(mean(multi_ms), 5), "p50": round(percentile(multi_ms, 50), 5)},
        "algorithmic_bytes": algo,
        "achieved_gbs": round(algo / t / 1e9, 2),
        "hbm_frac": round(algo / t / 1e9 / HBM_PEAK_GBS, 4),
        "kernel": kernel,
        "kernel_ms": {"mean": round(mean(kernel_ms), 5), "p50": round(percentile(kernel_ms, 50), 5)},
        "kernel_achieved_gbs": round(algo / tk / 1e9, 2),
        "kernel_hbm_frac": round(algo / tk / 1e9 / HBM_PEAK_GBS, 4),
        "traffic": measured_traffic(w.name, kernel),
        "mfma_busy_pct": measured_mfma(w.name, kernel),
        "tokens_per_s": round(T / t, 1),
        "single_token_decode_same_pools_call_ms": round(mean(single_ms), 5),
        "note": "pa_decode_multi (append fused, causal over cached + drafted tokens) vs pa_decode of "
                "one token per sequence on the same pools, alternating, each after a cache flush, "
                "events around the call (launch included); kernel_ms: the main kernel alone through "
                "pa_decode_multi_ex (caller workspace, host lengths), GPU-stamped events",
    }


def fused_step(w, part, cus):
    """How pa_append_decode (given the host copy of the lengths) runs this
    workload: (append fused into the decode, its kernels, what the schedule
    is, whether the main kernel writes the new tokens).  The unsplit MFMA
    schedule is one launch; a stream-K batch on the MFMA path runs the
    multi-token kernel over partitions sized on the lengths (so that about 512
    workgroups share the tokens), then the row combine; a partitioned batch
    whose grid fills the GPU runs the shared-partition kernel, which takes the
    new token from k / v, and a combine that stores it; anything else appends
    first and decodes as pa_decode_ex does."""
    g = w.num_q_heads // w.num_kv_heads
    sets = 2 if g > 16 else 1
    span = w.block_tables.shape[1] * w.block_size
    unsplit = part == -1 or part >= span
    if g >= 3 and unsplit:
        return True, [f"decode_multi<{w.head_dim},{w.block_size},{sets},false>"], \
            "one launch: the new token stored and attended", True
    if g >= 3 and part == -2:
        row_wgs = w.num_kv_heads * -(-g // (16 * sets))
        tokens = int(sum(min(max(int(x), 0), span) for x in w.context_lens))
        p = max(512, -(-(-(-tokens * row_wgs // 512)) // 256) * 256)
        return True, [f"decode_multi<{w.head_dim},{w.block_size},{sets},true>", f"combine_rows<{w.head_dim}>"], \
            f"partitions of {p} tokens sized on the host's lengths, only those holding tokens launched, " \
            "the new token stored by the last one; then the row combine", True
    if part > 0 and not unsplit and g <= 16 and w.num_seqs * w.num_kv_heads * -(-span // part) >= cus:
        return True, [f"decode_shared<{w.head_dim},{w.block_size},true>", f"combine_append<{w.head_dim},{w.block_size}>"], \
            f"partitions of {part} tokens, shared partitions read once, the new token taken from k / v by its " \
            "last partition; then the combine, which stores the new tokens", False
    return False, [], "append kernel, then the decode schedule", False


def percentile(xs, q):
    xs = sorted(xs)
    if not xs:
        return float("nan")
    k = (len(xs) - 1) * q / 100.0
    lo, hi = int(k), min(int(k) + 1, len(xs) - 1)
    return xs[lo] + (xs[hi] - xs[lo]) * (k - lo)


def cpu_baseline(w, budget_s):
    """Time the fp64 oracle (append + decode), one sequence at a time, in passes
    over the batch, until about budget_s seconds of CPU time are spent."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None

    order = list(range(w.num_seqs))
    kst, vst = w.stores()
    t_total, tokens, done = 0.0, 0, 0
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    try:
        if ctx:
            ctx.__enter__()
        passes = 0
        while t_total < budget_s:
            passes += 1
            t0 = time.perf_counter()
            oracle.copy_blocks(w.copies, kst, vst)  # the step's copy-on-write copies, if any
            t_total += time.perf_counter() - t0
            for s in order:
                t0 = time.perf_counter()
                oracle.cache_append(w.k_new[s:s + 1], w.v_new[s:s + 1], w.slot_mapping[s:s + 1], kst, vst,
                                    w.block_size)
                oracle.paged_decode(w.q, kst, vst, w.block_tables, w.context_lens, w.scale, w.block_size,
                                    seqs=[s])
                t_total += time.perf_counter() - t0
                tokens += int(w.context_lens[s])
                done += 1
                if t_total >= budget_s:
                    break
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    kv_bytes = tokens * w.num_kv_heads * w.head_dim * 2 * 2
    return {
        "value": round(kv_bytes / t_total / 1e9, 6),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "seqs_per_s": round(done / t_total, 4),
        "sample": f"{done} sequence-steps ({passes} pass(es) over the {w.num_seqs}-sequence batch, "
                  f"{tokens} context tokens), fp64 numpy oracle append + decode, one BLAS thread, "
                  f"{t_total:.1f} s",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the decode path shards by sequence or KV head with no exchange, see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from paged_kv_cache_122_amd import _lib as pa
    from paged_kv_cache_122_amd import device as dev
    from paged_kv_cache_122_amd import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    pa.load()
    torch.cuda.set_device(0)

    w = workloads.make(args.config)
    dw = dev.upload(w, "cuda:0")
    out = torch.empty_like(dw.q)
    eff_bytes = w.effective_kv_bytes()
    # bytes the kernel must bring from HBM: a physical block shared by several
    # sequences (a common prefix) counts once
    algo_bytes = w.unique_kv_bytes()
    max_len = int(w.block_tables.shape[1]) * w.block_size
    part = pa.schedule(w.num_seqs, w.num_q_heads, w.num_kv_heads, max_len)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    kernels, schedule = decode_kernels(w, part, cus)
    fused, fused_kernels, step_kind, writes_new = fused_step(w, part, cus)
    new_kv_bytes = w.num_seqs * w.num_kv_heads * w.head_dim * 2 * 2
    if fused:
        # the main launch reads the context (the new token from k / v); in one-launch steps it
        # also writes the new token (else the combine that follows does)
        kernels, schedule = fused_kernels, step_kind
        if writes_new:
            algo_bytes += new_kv_bytes
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.Stream()  # default priority
    torch.cuda.synchronize()

    has_copies = int(w.copies.shape[0]) > 0

    def append():
        # the step's copy-on-write copies (if any) go first, then the append
        if has_copies:
            pa.copy_blocks(dw.k_cache, dw.v_cache, dw.copies, stream=stream)
        pa.cache_append(dw.k_new, dw.v_new, dw.slot_mapping, dw.k_cache, dw.v_cache, stream=stream)

    # the call pa_decode makes, with a workspace of our own so that the main
    # kernel can be bracketed by GPU-timed events
    ws_bytes = pa.workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, max_len, 0)
    ws = pa.alloc_workspace(ws_bytes, "cuda:0") if ws_bytes else None

    # the host copy of the lengths that a serving engine keeps (it computes
    # them); unsplit schedules rank the sequences from it on the host
    host_lens = np.asarray(w.context_lens, dtype=np.int32)

    def decode(kernel_events=None):
        pa.decode_ex(out, dw.q, dw.k_cache, dw.v_cache, dw.block_tables, dw.context_lens, w.scale,
                     w.block_size, workspace=ws, kernel_events=kernel_events, host_context_lens=host_lens,
                     stream=stream)

    def step(kernel_events=None):
        # the step's copy-on-write copies (if any), then append + decode in one call
        if has_copies:
            pa.copy_blocks(dw.k_cache, dw.v_cache, dw.copies, stream=stream)
        pa.append_decode(out, dw.q, dw.k_new, dw.v_new, dw.slot_mapping, dw.k_cache, dw.v_cache,
                         dw.block_tables, dw.context_lens, w.scale, w.block_size, workspace=ws,
                         kernel_events=kernel_events, host_context_lens=host_lens, stream=stream)

    tev = TimingEvents()
    E = tev.create
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            flush.zero_()
            step()
        stream.synchronize()

        ev = [(E(), E()) for _ in range(args.steps)]
        kev = [(E(), E()) for _ in range(args.steps)]
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        for e0, e1 in ev:
            flush.zero_()
            tev.record(e0, stream)
            step()
            tev.record(e1, stream)
        stream.synchronize()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        step_ms = [tev.elapsed_ms(a, b) for a, b in ev]

        # the same steps again with the main kernel bracketed by events that the
        # GPU stamps at its own start and end (such a launch costs the stream a
        # few microseconds more, so it is kept out of the steps above)
        for k in kev:
            flush.zero_()
            step(kernel_events=k)
        stream.synchronize()
        kernel_ms = [tev.elapsed_ms(a, b) for a, b in kev]

        # the step as two calls: pa_cache_append, then pa_decode's schedule
        tw = [(E(), E(), E()) for _ in range(args.steps)]
        for e0, e1, e2 in tw:
            flush.zero_()
            tev.record(e0, stream)
            append()
            tev.record(e1, stream)
            decode()
            tev.record(e2, stream)
        stream.synchronize()
        append_ms = [tev.elapsed_ms(a, b) for a, b, _ in tw]
        decode_ms = [tev.elapsed_ms(b, c) for _, b, c in tw]
        two_ms = [tev.elapsed_ms(a, c) for a, _, c in tw]

        hot_ms = []
        if args.unflushed:  # back-to-back steps (caches may hold part of the pools)
            hot = [(E(), E()) for _ in range(args.steps)]
            for a, b in hot:
                tev.record(a, stream)
                step()
                tev.record(b, stream)
            stream.synchronize()
            hot_ms = [tev.elapsed_ms(a, b) for a, b in hot]

        # paging control: the same decode over an unpaged copy of the cache
        # (taken after the append, so both see the same tokens), timed the same
        # way as the paged call above
        contig_ms, unsplit_ms = [], []
        if not args.no_control:
            kc, vc = dev.contiguous_copy(dw, w)
            out_c = torch.empty_like(out)
            cev = [(E(), E(), E(), E()) for _ in range(args.steps)]
            for a, b, c, d in cev:
                flush.zero_()
                tev.record(a, stream)
                pa.decode_contiguous(out_c, dw.q, kc, vc, dw.context_lens, w.scale, stream=stream)
                tev.record(b, stream)
                flush.zero_()
                tev.record(c, stream)  # the paged kernel with the control's schedule
                pa.decode_ex(out_c, dw.q, dw.k_cache, dw.v_cache, dw.block_tables, dw.context_lens,
                             w.scale, w.block_size, partition_tokens=-1, path=2, stream=stream)
                tev.record(d, stream)
            stream.synchronize()
            contig_ms = [tev.elapsed_ms(a, b) for a, b, _, _ in cev]
            unsplit_ms = [tev.elapsed_ms(c, d) for _, _, c, d in cev]
            del kc, vc, out_c

        multi = []
        if not args.no_multi:
            multi = [multi_query_leg(c, k, args.steps, args.warmup, tev, stream, flush) for c, k in MULTI_CONFIGS]

        tev.close()

        if args.copy_calibration > 0:
            n = args.copy_calibration << 18  # float32 elements
            src = torch.ones(n, dtype=torch.float32, device="cuda:0")
            dst = torch.empty_like(src)
            for _ in range(3):
                torch.neg(src, out=dst)
            stream.synchronize()
            del src, dst

    mean = lambda xs: sum(xs) / len(xs)  # noqa: E731
    t_step = mean(step_ms) / 1e3
    t_kernel = mean(kernel_ms) / 1e3
    value = eff_bytes / t_step / 1e9
    achieved = algo_bytes / t_kernel / 1e9
    line = {
        "metric": "paged decode-attention effective KV GB/s vs HBM peak; seqs/s per layer-step",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mean(step_ms), 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "num_seqs": w.num_seqs,
            "num_q_heads": w.num_q_heads,
            "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim,
            "block_size": w.block_size,
            "num_blocks": w.num_blocks,
            "context_tokens": int(w.context_lens.sum()),
            "max_context_len": int(w.context_lens.max()),
            "effective_kv_bytes": eff_bytes,
            "unique_kv_bytes": w.unique_kv_bytes(),
            "seed": w.seed,
            "step": ("pa_copy_blocks (copy-on-write) + " if has_copies else "")
                    + "pa_append_decode (" + step_kind
                    + "), with a host copy of the lengths"
                    + (" (the sequences ranked on the host)" if kernels[0].endswith(",false>") and "multi" in kernels[0]
                       else "")
                    + ", caches flushed before each step",
            "cow_copies": int(w.copies.shape[0]),
            "schedule": schedule,
        },
        "seqs_per_s": round(w.num_seqs / t_step, 1),
        "hbm_frac_step": round(value / HBM_PEAK_GBS, 4),
        "main_kernel_ms": {"mean": round(mean(kernel_ms), 5),
                           "p10": round(percentile(kernel_ms, 10), 5),
                           "p50": round(percentile(kernel_ms, 50), 5),
                           "p90": round(percentile(kernel_ms, 90), 5)},
        "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 4),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(w.name, kernels[0]),
            "mfma_busy_pct": measured_mfma(w.name, kernels[0]),
            "kernels": kernels,
            "algorithmic_bytes": algo_bytes,
            "timed": f"HIP events (created with hipEventDisableSystemFence) stamped by the GPU "
                     f"at the start and end of {kernels[0]} (hipExtLaunchKernel), {args.steps} "
                     "further steps, caches flushed",
        },
    }
    if contig_ms:
        line["paging_control"] = {
            "contiguous_call_ms": round(mean(contig_ms), 5),
            "paged_same_schedule_call_ms": round(mean(unsplit_ms), 5),
            "paged_over_contiguous": round(mean(unsplit_ms) / mean(contig_ms) - 1.0, 4),
            "paged_auto_call_ms": round(mean(decode_ms), 5),
            "note": "pa_decode_contiguous on an unpaged copy of the cache (per sequence and KV head a "
                    "run of 16-token tiles, no block table) vs the paged kernel with the same "
                    "schedule (one workgroup per sequence and head group, MFMA), alternating, each "
                    "after a cache flush and timed by events around the call",
        }
    line["two_call_step"] = {
        "step_ms": {"mean": round(mean(two_ms), 5), "p50": round(percentile(two_ms, 50), 5)},
        "value": round(eff_bytes / (mean(two_ms) / 1e3) / 1e9, 2),
        "unit": "GB/s",
        "append_call_ms": {"mean": round(mean(append_ms), 5), "p50": round(percentile(append_ms, 50), 5)},
        "decode_call_ms": {"mean": round(mean(decode_ms), 5), "p10": round(percentile(decode_ms, 10), 5),
                           "p50": round(percentile(decode_ms, 50), 5),
                           "p90": round(percentile(decode_ms, 90), 5)},
        "note": "the same step as " + ("pa_copy_blocks + " if has_copies else "") + "pa_cache_append + "
                "pa_decode (the append kernel, then the decode schedule), flushed, events around the calls",
    }
    if multi:
        line["multi_query"] = multi[0]
        line["multi_query_long"] = multi[1]
    if hot_ms:
        line["unflushed_step_ms"] = {"mean": round(mean(hot_ms), 5),
                                     "p50": round(percentile(hot_ms, 50), 5),
                                     "gbs": round(eff_bytes / (mean(hot_ms) / 1e3) / 1e9, 2)}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
