"""Benchmark of one paged-decode layer step on one MI355X: slot-mapped append of
this step's K/V and paged decode attention, as one pa_append_decode call (one
launch where the decode schedule is unsplit MFMA; the shared-partition kernel
and a combine on partitioned batches; the split multi-token kernel and a row
combine on few long contexts).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
                    [--configs all|none|NAME,...] [--no-cpu-baseline]

Prints ONE JSON line.  The headline (``value``, ``roofline``) is the
Llama-3-8B-shaped batch (``--config`` changes it); ``configs`` holds one row per
seeded configuration, every one timed the same way in the same run.  ``value`` is
effective KV-read GB/s of the whole step (sum_s L_s * Hkv * D * 2 (K and V) * 2
bytes, divided by the event-timed step).  Inputs are resident in HBM; before
every timed step a 1 GiB buffer is read so that neither L2 nor the 256 MB
Infinity Cache still holds the pools (the flush is outside the timed region).
The buffer is read, not written: a written one leaves the caches full of dirty
lines, and their write-back then lands in the timed kernel.
All work runs on one stream of this process and the HIP events are recorded on
it; they are created with hipEventDisableSystemFence, so recording them flushes
no cache.  ``roofline`` is the step's main kernel alone, timed in as many
further flushed steps by events that the GPU stamps at its start and end,
against 8 TB/s.  ``two_call_step`` times the headline step as pa_cache_append +
pa_decode.  ``fixed_cost`` times the headline's shapes with one token per
sequence (what a launch costs with next to no bytes).  ``paging_control`` times
the same decode over an unpaged copy of the
cache; ``multi_query`` times pa_decode_multi (several new tokens per sequence:
speculative verification) on the Llama-3-8B-shaped batch with 5 drafted tokens
per sequence, and ``multi_query_long`` on 8 sequences of 32k tokens with 5
drafted tokens each.  ``cpu_baseline`` is the fp64 oracle on a bounded sample of
the headline workload, in worker processes on this host's cores.
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
# every seeded configuration, one row each in ``configs``
CONFIG_ROWS = ("tiny_gqa4_d64", "llama3_8b_b64", "llama3_70b_b256", "opt13b_mha_prefix_b128",
               "long32k_b8", "long32k_b16", "long32k_b32", "opt13b_cow_fork_b128")
# worker processes of the CPU baseline: this host's cores, at most 16 (a
# one-GPU share of a multi-GPU host's cores)
CPU_WORKERS_MAX = 16

# HBM bytes per launch of a step's main kernel, from two rocprofv3 --pmc runs
# of this script (FETCH_SIZE, then WRITE_SIZE), each scaled by what the counter
# reads for a plain copy of known size in the same run, and the kernel's MFMA
# busy share of SIMD cycles from a third.  They are copied here from the
# summaries under profiles/ (named per entry), not measured in the run that
# prints them, and hold only for the sources they were taken on (sha256 of the
# files below, which include the host code that picks the schedule); reported
# as null once those change.
KERNEL_SOURCES = ("paged_kv_cache_122_amd/csrc/pa_kernels.hip",
                  "paged_kv_cache_122_amd/csrc/pa_internal.h",
                  "paged_kv_cache_122_amd/csrc/pa_api.cpp")
MEASURED_TRAFFIC = {
    "sources_sha256": "9e14632f8f2a079c3b2a889faf4f3756d356c09ae4096541ebf01ba752bfcfb0",
    "tiny_gqa4_d64 decode_multi<64,16,1,false>": {"fetch_bytes": 760356, "write_bytes": 10240, "mfma_busy_pct": 0.04,
        "source": "profiles/decode_multi_tiny_gqa4_d64_kernel_trace.md"},
    "llama3_8b_b64 decode_multi<128,16,1,false>": {"fetch_bytes": 274016918, "write_bytes": 1310770, "mfma_busy_pct": 7.8,
        "source": "profiles/decode_multi_llama3_8b_b64_kernel_trace.md"},
    "llama3_8b_verify5_b64 decode_multi<128,16,2,false>": {"fetch_bytes": 288020869, "write_bytes": 4459629, "mfma_busy_pct": 15.44,
        "source": "profiles/decode_multi_llama3_8b_verify5_b64_kernel_trace.md"},
    "long32k_verify5_b16 decode_multi<128,16,2,true>": {"fetch_bytes": 1074923221, "write_bytes": 5559133, "mfma_busy_pct": 19.58,
        "source": "profiles/decode_multi_long32k_verify5_b16_kernel_trace.md"},
    "llama3_70b_b256 decode_multi<128,16,1,false>": {"fetch_bytes": 907152096, "write_bytes": 7340032, "mfma_busy_pct": 9.49,
        "source": "profiles/decode_multi_llama3_70b_b256_kernel_trace.md"},
    "opt13b_mha_prefix_b128 decode_shared<128,16,true>": {"fetch_bytes": 1745314486, "write_bytes": 5525000, "mfma_busy_pct": 9.68,
        "source": "profiles/decode_shared_opt13b_mha_prefix_b128_kernel_trace.md"},
    "long32k_b8 decode_multi<128,8,1,true>": {"fetch_bytes": 1075070705, "write_bytes": 1163264, "mfma_busy_pct": 9.93,
        "source": "profiles/decode_multi_long32k_b8_kernel_trace.md"},
    "long32k_b16 decode_multi<128,16,1,true>": {"fetch_bytes": 1074517722, "write_bytes": 1163469, "mfma_busy_pct": 9.86,
        "source": "profiles/decode_multi_long32k_b16_kernel_trace.md"},
    "long32k_b32 decode_multi<128,32,1,true>": {"fetch_bytes": 1074262929, "write_bytes": 1163456, "mfma_busy_pct": 10.0,
        "source": "profiles/decode_multi_long32k_b32_kernel_trace.md"},
    "opt13b_cow_fork_b128 decode_shared<128,16,true>": {"fetch_bytes": 350439439, "write_bytes": 1310720, "mfma_busy_pct": 7.55,
        "source": "profiles/decode_shared_opt13b_cow_fork_b128_kernel_trace.md"},
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default=DEFAULT_CONFIG, help="the headline workload")
    ap.add_argument("--configs", default="all",
                    help="rows of the configs object: all, none, or a comma-separated list")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="seconds each CPU baseline worker spends on the oracle")
    ap.add_argument("--no-multi", action="store_true",
                    help="skip the multi-token (speculative verification) leg")
    ap.add_argument("--no-fixed-cost", action="store_true",
                    help="skip the one-token-per-sequence step (the launch's fixed cost)")
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


class CacheFlush:
    """Evicts the pools from L2 and the Infinity Cache by reading a 1 GiB
    buffer that is written once, here.  Reading leaves only clean lines behind;
    a buffer written before each step would leave up to the caches' size in
    dirty lines, whose write-back to HBM would then run inside the timed kernel
    (on the Llama-3-70B-shaped batch, 154.3 us after a written flush against
    148.2 after a read one and 147.5 with no flush at all, whose 900 MB of
    pools no cache holds anyway)."""

    def __init__(self):
        import torch

        self.buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        self.out = torch.empty((), dtype=torch.float32, device="cuda:0")

    def __call__(self):
        import torch

        torch.sum(self.buf, dim=0, out=self.out)

    def written(self):
        """The flush that writes the buffer instead (for comparison only)."""
        self.buf.fill_(1.0)


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


def counter_fields(config, kernel):
    """traffic (fetched + written bytes per launch), MFMA busy share and where
    they come from, or nulls when no summary holds them for these sources."""
    m = measured(config, kernel)
    if m is None:
        return {"traffic": None, "mfma_busy_pct": None, "traffic_source": None}
    return {"traffic": m["fetch_bytes"] + m["write_bytes"], "mfma_busy_pct": m.get("mfma_busy_pct"),
            "traffic_source": m["source"] + " (rocprofv3 counter passes, copied here; not measured in this run)"}


def mean(xs):
    return sum(xs) / len(xs)


def percentile(xs, q):
    xs = sorted(xs)
    if not xs:
        return float("nan")
    k = (len(xs) - 1) * q / 100.0
    lo, hi = int(k), min(int(k) + 1, len(xs) - 1)
    return xs[lo] + (xs[hi] - xs[lo]) * (k - lo)


def stats_us(ms):
    return {"mean": round(mean(ms) * 1e3, 2), "p10": round(percentile(ms, 10) * 1e3, 2),
            "p50": round(percentile(ms, 50) * 1e3, 2), "p90": round(percentile(ms, 90) * 1e3, 2)}


def describe_launch(kernels, part):
    """What a step's launches do, read from the kernel names the library
    reports (pa_last_launch) and the automatic partition choice."""
    main = next((k for k in kernels if not k.startswith(("copy_kernel", "append_kernel"))), "")
    split = "stream-K" if part == -2 else (f"partitions of {part} tokens" if part > 0 else "no split")
    if main.startswith("decode_multi") and main.endswith(",false>"):
        text = "one launch: the new token stored and attended, one workgroup per (sequence, head group)"
    elif main.startswith("decode_multi"):
        text = ("partitions sized on the host's lengths, only those holding tokens launched, the new token "
                "stored by the last one; then the row combine")
    elif main.startswith("decode_shared") and main.endswith(",true>"):
        text = (f"{split}; runs of consecutive sequences read their common blocks once, the new token taken "
                "from k / v by its last partition; then the combine, which stores the new tokens")
    elif main.startswith("decode_shared"):
        text = f"{split}; runs of consecutive sequences read their common blocks once"
    elif "_sk" in main:
        text = "stream-K: equal token ranges per wave of a persistent grid, then the piece combine"
    else:
        text = split + ("" if len(kernels) < 2 or not kernels[-1].startswith("combine") else "; then the combine")
    if kernels and kernels[0].startswith("append_kernel"):
        text = "append kernel, then " + text
    return text


class Step:
    """One layer step of a workload on the GPU, as a serving engine would run
    it: the step's copy-on-write copies (if any), then pa_append_decode with the
    caller's workspace and a host copy of the lengths."""

    def __init__(self, w, stream, partition_tokens=0):
        import numpy as np
        import torch

        from paged_kv_cache_122_amd import _lib as pa
        from paged_kv_cache_122_amd import device as dev

        self.pa, self.w, self.stream = pa, w, stream
        self.partition_tokens = partition_tokens  # 0: the automatic schedule
        self.dw = dev.upload(w, "cuda:0")
        self.out = torch.empty_like(self.dw.q)
        self.has_copies = int(w.copies.shape[0]) > 0
        max_len = int(w.block_tables.shape[1]) * w.block_size
        self.part = partition_tokens or pa.schedule(w.num_seqs, w.num_q_heads, w.num_kv_heads, max_len)
        nb = pa.workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, max_len, partition_tokens)
        self.ws = pa.alloc_workspace(nb, "cuda:0") if nb else None
        self.host_lens = np.asarray(w.context_lens, dtype=np.int32)
        # the kernels the step launches, as the library reports them (one
        # call; the bench's warm-up repeats it); the main kernel is the first
        # one after the copy-on-write copies and a separate append
        self()
        launched = pa.last_launch()
        self.kernels = [k for k in launched if not k.startswith(("copy_kernel", "append_kernel"))]
        if not self.kernels:
            raise RuntimeError(f"{w.name}: the step launched no decode kernel ({launched})")
        self.kernels_all = launched
        self.schedule = describe_launch(launched, self.part)
        # bytes the main kernel must move: a physical block shared by several
        # sequences (a common prefix) counts once; the multi-token kernel also
        # writes the new tokens (a separate append kernel, or the combine after
        # the shared-partition kernel, writes them otherwise)
        self.algo_bytes = w.unique_kv_bytes()
        if self.kernels[0].startswith("decode_multi"):
            self.algo_bytes += w.num_seqs * w.num_kv_heads * w.head_dim * 2 * 2

    def copies(self):
        if self.has_copies:
            self.pa.copy_blocks(self.dw.k_cache, self.dw.v_cache, self.dw.copies, stream=self.stream)

    def __call__(self, kernel_events=None):
        dw, w = self.dw, self.w
        self.copies()  # pa_last_launch then names the step's own call alone
        self.pa.append_decode(self.out, dw.q, dw.k_new, dw.v_new, dw.slot_mapping, dw.k_cache, dw.v_cache,
                              dw.block_tables, dw.context_lens, w.scale, w.block_size, workspace=self.ws,
                              kernel_events=kernel_events, host_context_lens=self.host_lens,
                              partition_tokens=self.partition_tokens, stream=self.stream)

    def append(self):
        dw = self.dw
        self.copies()
        self.pa.cache_append(dw.k_new, dw.v_new, dw.slot_mapping, dw.k_cache, dw.v_cache, stream=self.stream)

    def decode(self):
        """The call pa_decode makes (same schedule), with the step's workspace."""
        dw, w = self.dw, self.w
        self.pa.decode_ex(self.out, dw.q, dw.k_cache, dw.v_cache, dw.block_tables, dw.context_lens, w.scale,
                          w.block_size, workspace=self.ws, host_context_lens=self.host_lens,
                          partition_tokens=self.partition_tokens, stream=self.stream)

    def step_desc(self):
        return (("pa_copy_blocks (copy-on-write) + " if self.has_copies else "")
                + "pa_append_decode (" + self.schedule + "), with a host copy of the lengths"
                + (" (the sequences ranked on the host)"
                   if self.kernels[0].endswith(",false>") and "multi" in self.kernels[0] else "")
                + ", caches flushed before each step")


def time_steps(st, steps, warmup, tev, flush):
    """(step ms, main-kernel ms) over `steps` flushed steps each: the step
    between events around the call, then the main kernel alone between events
    the GPU stamps at its start and end (a launch that carries them costs the
    stream a few microseconds more, so it is kept out of the step timing)."""
    stream = st.stream
    for _ in range(warmup):
        flush()
        st()
    stream.synchronize()
    ev = [(tev.create(), tev.create()) for _ in range(steps)]
    kev = [(tev.create(), tev.create()) for _ in range(steps)]
    for a, b in ev:
        flush()
        tev.record(a, stream)
        st()
        tev.record(b, stream)
    stream.synchronize()
    step_ms = [tev.elapsed_ms(a, b) for a, b in ev]
    for k in kev:
        flush()
        st(kernel_events=k)
    stream.synchronize()
    kernel_ms = [tev.elapsed_ms(a, b) for a, b in kev]
    return step_ms, kernel_ms


def config_row(st, step_ms, kernel_ms):
    """One row of ``configs``: the step of this workload and its main kernel."""
    w = st.w
    eff = w.effective_kv_bytes()
    t, tk = mean(step_ms) / 1e3, mean(kernel_ms) / 1e3
    row = {
        "num_seqs": w.num_seqs, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
        "head_dim": w.head_dim, "block_size": w.block_size,
        "context_tokens": int(w.context_lens.sum()), "max_context_len": int(w.context_lens.max()),
        "step_us": stats_us(step_ms),
        "value": round(eff / t / 1e9, 2),
        "unit": "GB/s",
        "seqs_per_s": round(w.num_seqs / t, 1),
        "kernel": st.kernels[0],
        "kernels": st.kernels_all,
        "kernel_us": stats_us(kernel_ms),
        "effective_kv_bytes": eff,
        "unique_kv_bytes": w.unique_kv_bytes(),
        "algorithmic_bytes": st.algo_bytes,
        "kernel_gbs": round(st.algo_bytes / tk / 1e9, 2),
        "kernel_frac": round(st.algo_bytes / tk / 1e9 / HBM_PEAK_GBS, 4),
        "step_frac_unique": round(w.unique_kv_bytes() / t / 1e9 / HBM_PEAK_GBS, 4),
        "schedule": st.schedule,
        "cow_copies": int(w.copies.shape[0]),
    }
    row.update(counter_fields(w.name, st.kernels[0]))
    return row


MULTI_CONFIGS = ("llama3_8b_verify5_b64", "long32k_verify5_b16")


def multi_query_leg(config, steps, warmup, tev, stream, flush):
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
        flush()
        multi()
        single()
    ev = [(E(), E(), E(), E()) for _ in range(steps)]
    for a, b, c, d in ev:
        flush()
        tev.record(a, stream)
        multi()
        tev.record(b, stream)
        flush()
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
        flush()
        pa.decode_multi_ex(out, dw.q, dw.k_new, dw.v_new, dw.slot_mapping, dw.query_start, dw.k_cache,
                           dw.v_cache, dw.block_tables, dw.context_lens, w.scale, w.block_size, mql,
                           workspace=ws, kernel_events=(a, b), host_context_lens=host_lens, stream=stream)
    stream.synchronize()
    kernel_ms = [tev.elapsed_ms(a, b) for a, b in kev]
    kernels = pa.last_launch()
    new_kv = T * w.num_kv_heads * w.head_dim * 2 * 2
    # K/V of every context token read once (cached ones from the pool, new ones
    # from k_new / v_new), the new K/V written, q read and out written
    algo = w.unique_kv_bytes() + new_kv + 2 * T * w.num_q_heads * w.head_dim * 2
    t = mean(multi_ms) / 1e3
    tk = mean(kernel_ms) / 1e3
    del dw, ws
    row = {
        "workload": w.name,
        "num_seqs": w.num_seqs,
        "new_tokens": T,
        "max_query_len": mql,
        "context_tokens": int(w.context_lens.sum()),
        "call_us": stats_us(multi_ms),
        "algorithmic_bytes": algo,
        "achieved_gbs": round(algo / t / 1e9, 2),
        "hbm_frac": round(algo / t / 1e9 / HBM_PEAK_GBS, 4),
        "kernel": kernels[0],
        "kernels": kernels,
        "kernel_us": stats_us(kernel_ms),
        "kernel_achieved_gbs": round(algo / tk / 1e9, 2),
        "kernel_hbm_frac": round(algo / tk / 1e9 / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(T / t, 1),
        "single_token_decode_same_pools_call_us": round(mean(single_ms) * 1e3, 2),
        "note": "pa_decode_multi (append fused, causal over cached + drafted tokens) vs pa_decode of "
                "one token per sequence on the same pools, alternating, each after a cache flush, "
                "events around the call (launch included); kernel_us: the main kernel alone through "
                "pa_decode_multi_ex (caller workspace, host lengths), GPU-stamped events",
    }
    row.update(counter_fields(w.name, kernels[0]))
    return row


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle in worker processes forked before this process
# touches the GPU; each inherits the headline workload and times the oracle's
# append + decode on its share of the sequences.
# ---------------------------------------------------------------------------
_CPU_WORKLOAD = None


def _cpu_worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)  # one BLAS thread per worker process
    except ImportError:  # pragma: no cover
        pass


def _cpu_share(job):
    """Oracle append + decode over this worker's sequences, in passes, until
    `budget` seconds are spent; returns (context tokens, sequence-steps, seconds)."""
    import oracle
    from paged_kv_cache_122_amd.workloads import BlockStore

    seqs, budget = job
    w = _CPU_WORKLOAD
    # this process's own (copy-on-write) view of the pools: re-appending a token
    # writes the same value again
    kst = BlockStore(w.owned, w.k_blocks, w.num_blocks)
    vst = BlockStore(w.owned, w.v_blocks, w.num_blocks)
    spent, tokens, done = 0.0, 0, 0
    if len(w.copies):
        oracle.copy_blocks(w.copies, kst, vst)
    while spent < budget and seqs:
        for s in seqs:
            t0 = time.perf_counter()
            oracle.cache_append(w.k_new[s:s + 1], w.v_new[s:s + 1], w.slot_mapping[s:s + 1], kst, vst,
                                w.block_size)
            oracle.paged_decode(w.q, kst, vst, w.block_tables, w.context_lens, w.scale, w.block_size, seqs=[s])
            spent += time.perf_counter() - t0
            tokens += int(w.context_lens[s])
            done += 1
            if spent >= budget:
                break
    return tokens, done, spent


def start_cpu_pool(w):
    """Fork the baseline's worker processes now, before the GPU is initialised
    in this process (they never touch it)."""
    import multiprocessing

    global _CPU_WORKLOAD
    _CPU_WORKLOAD = w
    affinity = len(os.sched_getaffinity(0))
    n = max(1, min(affinity, CPU_WORKERS_MAX, w.num_seqs))
    pool = multiprocessing.get_context("fork").Pool(n, initializer=_cpu_worker_init)
    return pool, n, affinity


def cpu_baseline(pool, n, affinity, w, budget_s):
    """Sequences dealt round robin over the workers; each worker loops over its
    share for budget_s seconds.  Rate = sum over workers of their own rates
    (they run at the same time, one per core)."""
    jobs = [(list(range(i, w.num_seqs, n)), budget_s) for i in range(n)]
    wall0 = time.perf_counter()
    res = pool.map(_cpu_share, jobs)
    wall = time.perf_counter() - wall0
    pool.close()
    pool.join()
    bpt = w.num_kv_heads * w.head_dim * 2 * 2
    gbs = sum(tok * bpt / t for tok, _, t in res if t > 0) / 1e9
    seqs_s = sum(d / t for _, d, t in res if t > 0)
    done = sum(d for _, d, _ in res)
    tokens = sum(tok for tok, _, _ in res)
    return {
        "value": round(gbs, 6),
        "unit": "GB/s",
        "cores": n,
        "kind": "oracle",
        "seqs_per_s": round(seqs_s, 3),
        "host_affinity_cores": affinity,
        "sample": f"{done} sequence-steps of the {w.num_seqs}-sequence {w.name} batch ({tokens} context "
                  f"tokens): fp64 numpy oracle append + decode, one sequence at a time, in {n} worker "
                  f"processes with one BLAS thread each, the sequences dealt round robin, about "
                  f"{budget_s:.0f} s per worker ({wall:.1f} s wall); rate = sum of the workers' rates",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the decode path shards by sequence or KV head with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    from paged_kv_cache_122_amd import workloads

    if args.configs == "all":
        rows = list(CONFIG_ROWS)
    elif args.configs == "none":
        rows = []
    else:
        rows = [c for c in args.configs.split(",") if c]
        bad = [c for c in rows if c not in workloads.CONFIGS]
        if bad:
            print(f"bench.py: unknown configs {bad}", file=sys.stderr)
            sys.exit(2)

    w = workloads.make(args.config)
    pool = None
    if not args.no_cpu_baseline:
        pool, n_workers, affinity = start_cpu_pool(w)

    import torch

    from paged_kv_cache_122_amd import _lib as pa
    from paged_kv_cache_122_amd import device as dev

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    pa.load()
    torch.cuda.set_device(0)
    flush = CacheFlush()
    stream = torch.cuda.Stream()  # default priority
    torch.cuda.synchronize()
    eff_bytes = w.effective_kv_bytes()

    tev = TimingEvents()
    E = tev.create
    with torch.cuda.stream(stream):
        st = Step(w, stream)
        step_ms, kernel_ms = time_steps(st, args.steps, args.warmup, tev, flush)
        print(f"bench: {w.name} step {mean(step_ms) * 1e3:.1f} us, kernel {mean(kernel_ms) * 1e3:.1f} us",
              file=sys.stderr, flush=True)
        # the same main kernel after a flush that writes the buffer instead of
        # reading it, for comparison: a written flush leaves dirty lines whose
        # write-back lands in the timed kernel
        _, written_kernel_ms = time_steps(st, args.steps, 0, tev, flush.written)

        # the step as two calls: pa_cache_append, then pa_decode's schedule
        tw = [(E(), E(), E()) for _ in range(args.steps)]
        for e0, e1, e2 in tw:
            flush()
            tev.record(e0, stream)
            st.append()
            tev.record(e1, stream)
            st.decode()
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
                st()
                tev.record(b, stream)
            stream.synchronize()
            hot_ms = [tev.elapsed_ms(a, b) for a, b in hot]

        # paging control: the same decode over an unpaged copy of the cache
        # (taken after the append, so both see the same tokens), timed the same
        # way as the paged call above
        contig_ms, unsplit_ms = [], []
        if not args.no_control:
            kc, vc = dev.contiguous_copy(st.dw, w)
            out_c = torch.empty_like(st.out)
            dw = st.dw
            cev = [(E(), E(), E(), E()) for _ in range(args.steps)]
            for a, b, c, d in cev:
                flush()
                tev.record(a, stream)
                pa.decode_contiguous(out_c, dw.q, kc, vc, dw.context_lens, w.scale, stream=stream)
                tev.record(b, stream)
                flush()
                tev.record(c, stream)  # the paged kernel with the control's schedule
                pa.decode_ex(out_c, dw.q, dw.k_cache, dw.v_cache, dw.block_tables, dw.context_lens,
                             w.scale, w.block_size, partition_tokens=-1, path=2, stream=stream)
                tev.record(d, stream)
            stream.synchronize()
            contig_ms = [tev.elapsed_ms(a, b) for a, b, _, _ in cev]
            unsplit_ms = [tev.elapsed_ms(c, d) for _, _, c, d in cev]
            del kc, vc, out_c
        # the fixed cost of the step: the same shapes, grid and schedule family
        # with one token per sequence (a few bytes each), timed the same way
        fixed = None
        if not args.no_fixed_cost:
            fw = workloads.random_workload(w.seed, [1] * w.num_seqs, num_q_heads=w.num_q_heads,
                                           num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                                           block_size=w.block_size, name=f"{w.name}_one_token")
            fst = Step(fw, stream)
            fsm, fkm = time_steps(fst, args.steps, args.warmup, tev, flush)
            # a launch of any kernel: a one-element fill between the same
            # kind of events as the step
            one = torch.zeros(1, dtype=torch.float32, device="cuda:0")
            fev = [(E(), E()) for _ in range(args.steps)]
            for a, b in fev:
                flush()
                tev.record(a, stream)
                one.fill_(1.0)
                tev.record(b, stream)
            stream.synchronize()
            fill_ms = [tev.elapsed_ms(a, b) for a, b in fev]
            fixed = {"workload": f"{w.name}'s shapes ({w.num_seqs} sequences, {w.num_q_heads} q / "
                                 f"{w.num_kv_heads} kv heads, D {w.head_dim}, B {w.block_size}) with one token "
                                 "per sequence",
                     "kernels": fst.kernels_all, "step_us": stats_us(fsm), "kernel_us": stats_us(fkm),
                     "one_element_fill_us": stats_us(fill_ms),
                     "note": "what a launch of the step costs with next to no bytes: dispatch, the table fetch, "
                             "one tile, the cross-wave combine, the output and the append; GPU-stamped events "
                             "around the kernel as for the roofline. one_element_fill_us: a one-element torch "
                             "fill between events around the call, as step_us is timed: the cost of launching "
                             "any kernel"}
            del fst, fw
        head_row = config_row(st, step_ms, kernel_ms)
        head_kernels, head_schedule, head_algo, head_desc = st.kernels_all, st.schedule, st.algo_bytes, st.step_desc()
        head_main = st.kernels[0]
        del st
        torch.cuda.empty_cache()

        multi = []
        if not args.no_multi:
            multi = [multi_query_leg(c, args.steps, args.warmup, tev, stream, flush) for c in MULTI_CONFIGS]
            torch.cuda.empty_cache()

        # every seeded configuration, timed the same way
        configs = {}
        for name in rows:
            if name == w.name:
                configs[name] = head_row
                continue
            cw = workloads.make(name)
            cst = Step(cw, stream)
            sm, km = time_steps(cst, args.steps, args.warmup, tev, flush)
            configs[name] = config_row(cst, sm, km)
            print(f"bench: {name} step {mean(sm) * 1e3:.1f} us, kernel {mean(km) * 1e3:.1f} us",
                  file=sys.stderr, flush=True)
            del cst, cw
            torch.cuda.empty_cache()

        tev.close()

        if args.copy_calibration > 0:
            n = args.copy_calibration << 18  # float32 elements
            src = torch.ones(n, dtype=torch.float32, device="cuda:0")
            dst = torch.empty_like(src)
            for _ in range(3):
                torch.neg(src, out=dst)
            stream.synchronize()
            del src, dst

    t_step = mean(step_ms) / 1e3
    t_kernel = mean(kernel_ms) / 1e3
    value = eff_bytes / t_step / 1e9
    achieved = head_algo / t_kernel / 1e9
    cf = counter_fields(w.name, head_main)
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
            "step": head_desc,
            "cow_copies": int(w.copies.shape[0]),
            "schedule": head_schedule,
        },
        "seqs_per_s": round(w.num_seqs / t_step, 1),
        "hbm_frac_step": round(value / HBM_PEAK_GBS, 4),
        "main_kernel_ms": {"mean": round(mean(kernel_ms), 5),
                           "p10": round(percentile(kernel_ms, 10), 5),
                           "p50": round(percentile(kernel_ms, 50), 5),
                           "p90": round(percentile(kernel_ms, 90), 5)},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": cf["traffic"],
            "traffic_source": cf["traffic_source"],
            "mfma_busy_pct": cf["mfma_busy_pct"],
            "kernels": head_kernels,
            "algorithmic_bytes": head_algo,
            "kernel": head_main,
            "timed": f"HIP events (created with hipEventDisableSystemFence) stamped by the GPU "
                     f"at the start and end of {head_main} (hipExtLaunchKernel), {args.steps} "
                     "further steps, caches flushed by reading a 1 GiB buffer",
        },
    }
    line["written_flush"] = {
        "kernel_us": stats_us(written_kernel_ms),
        "frac": round(head_algo / (mean(written_kernel_ms) / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "note": f"{head_main} timed as for the roofline, but after writing the 1 GiB flush buffer instead of "
                "reading it: the caches then hold dirty lines whose write-back runs inside the timed kernel; "
                "for comparison only",
    }
    if contig_ms:
        line["paging_control"] = {
            "contiguous_call_us": round(mean(contig_ms) * 1e3, 2),
            "paged_same_schedule_call_us": round(mean(unsplit_ms) * 1e3, 2),
            "paged_over_contiguous": round(mean(unsplit_ms) / mean(contig_ms) - 1.0, 4),
            "paged_auto_call_us": round(mean(decode_ms) * 1e3, 2),
            "note": "pa_decode_contiguous on an unpaged copy of the cache (per sequence and KV head a "
                    "run of 16-token tiles, no block table) vs the paged kernel with the same "
                    "schedule (one workgroup per sequence and head group, MFMA), alternating, each "
                    "after a cache flush and timed by events around the call",
        }
    if fixed is not None:
        line["fixed_cost"] = fixed
    line["two_call_step"] = {
        "step_us": stats_us(two_ms),
        "value": round(eff_bytes / (mean(two_ms) / 1e3) / 1e9, 2),
        "unit": "GB/s",
        "append_call_us": stats_us(append_ms),
        "decode_call_us": stats_us(decode_ms),
        "note": "the same step as " + ("pa_copy_blocks + " if int(w.copies.shape[0]) else "") + "pa_cache_append + "
                "pa_decode (the append kernel, then the decode schedule), flushed, events around the calls",
    }
    if multi:
        line["multi_query"] = multi[0]
        line["multi_query_long"] = multi[1]
    if hot_ms:
        line["unflushed_step_us"] = {**stats_us(hot_ms), "gbs": round(eff_bytes / (mean(hot_ms) / 1e3) / 1e9, 2)}
    if configs:
        line["configs"] = configs
        line["configs_note"] = (
            "every seeded configuration, each step (pa_append_decode with the caller's workspace and a host "
            "copy of the lengths, after the step's copy-on-write copies) timed by events around it over "
            f"{args.steps} flushed steps after {args.warmup} warm-up steps, and its main kernel alone by "
            "GPU-stamped events over as many more; value = effective (logical) KV bytes / step; kernel_frac "
            "= algorithmic bytes (unique KV bytes, plus the new tokens where that kernel writes them) / "
            "kernel time / 8 TB/s")
    if pool is not None:
        line["cpu_baseline"] = cpu_baseline(pool, n_workers, affinity, w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
