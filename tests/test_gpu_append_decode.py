"""GPU checks of pa_append_decode, the decode step in one call: the appended
pools are bit-exact against the oracle's append, the attention matches the fp64
oracle (max|err| <= 1e-2, relative RMS <= 2e-3), on the fused one-launch path
(unsplit MFMA schedules), on the partitioned schedule whose shared-partition
kernel takes the append (one launch and the combine), and on the
append-then-decode path (VALU, small split batches, stream-K), where it equals
pa_cache_append + pa_decode_ex bit for bit."""

import numpy as np
import pytest

import oracle
from gpu_util import assert_close, need_gpu, oracle_step, sample_seqs
from paged_kv_cache_122_amd import workloads

pytestmark = pytest.mark.gpu

# (config, options, sequences the oracle checks): fused path first, then the
# append-then-decode schedules
CASES = [
    ("tiny_gqa4_d64", {}, 64),
    ("llama3_8b_b64", {}, 24),
    ("llama3_70b_b256", {}, 16),
    ("llama3_8b_b64", {"partition_tokens": 512}, 16),
    ("long32k_b16", {}, 4),
    ("opt13b_mha_prefix_b128", {}, 12),
]


def _run(pa, dw, w, out, opts, kernel_events=None):
    torch = need_gpu()
    maxlen = w.table_width * w.block_size
    nb = pa.workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, maxlen,
                            opts.get("partition_tokens", 0))
    ws = pa.alloc_workspace(nb, "cuda") if nb else None
    pa.append_decode(out, dw.q, dw.k_new, dw.v_new, dw.slot_mapping, dw.k_cache, dw.v_cache, dw.block_tables,
                     dw.context_lens, w.scale, w.block_size, workspace=ws, kernel_events=kernel_events, **opts)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name,opts,n_check", CASES, ids=[f"{c[0]}-{c[1]}" for c in CASES])
def test_append_decode_parity(name, opts, n_check):
    torch = need_gpu()
    from paged_kv_cache_122_amd import _lib as pa
    from paged_kv_cache_122_amd import device as dev

    w = workloads.make(name)
    print(f"[{name} {opts}] S={w.num_seqs}", flush=True)
    dw = dev.upload(w)
    seqs = sample_seqs(w, n_check)
    kst, vst, ref = oracle_step(w, seqs)
    out = torch.empty(dw.q.shape, dtype=torch.float32, device="cuda")
    _run(pa, dw, w, out, opts)
    assert np.array_equal(dev.bf16_bits(dw.k_cache[dw.owned]), kst.blocks), "K pool differs"
    assert np.array_equal(dev.bf16_bits(dw.v_cache[dw.owned]), vst.blocks), "V pool differs"
    a, r = assert_close(out.double().cpu().numpy()[seqs], ref[seqs], name)
    print(f"[{name} {opts}] max|err| {a:.2e} rel RMS {r:.2e}", flush=True)
    del dw
    torch.cuda.empty_cache()


def test_append_decode_equals_two_calls_where_unfused():
    """Stream-K, VALU and small partitioned batches (the deep pipeline) run the
    append kernel, then pa_decode_ex's own kernels: the output equals the two
    separate calls bit for bit."""
    torch = need_gpu()
    from paged_kv_cache_122_amd import _lib as pa
    from paged_kv_cache_122_amd import device as dev

    for name, opts in (("opt13b_mha_prefix_b128", {"path": 1}),
                       ("tiny_gqa4_d64", {"partition_tokens": 32}), ("long32k_b16", {})):
        w = workloads.make(name)
        dw1, dw2 = dev.upload(w), dev.upload(w)
        o1, o2 = torch.empty_like(dw1.q), torch.empty_like(dw2.q)
        _run(pa, dw1, w, o1, opts)
        maxlen = w.table_width * w.block_size
        nb = pa.workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, maxlen,
                                opts.get("partition_tokens", 0))
        ws = pa.alloc_workspace(nb, "cuda") if nb else None
        pa.cache_append(dw2.k_new, dw2.v_new, dw2.slot_mapping, dw2.k_cache, dw2.v_cache)
        pa.decode_ex(o2, dw2.q, dw2.k_cache, dw2.v_cache, dw2.block_tables, dw2.context_lens, w.scale,
                     w.block_size, workspace=ws, **opts)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), name
        assert torch.equal(dw1.k_cache.view(torch.int16), dw2.k_cache.view(torch.int16)), name
        del dw1, dw2
        torch.cuda.empty_cache()


def test_append_decode_events_and_contracts():
    """Kernel events time the fused kernel (or the decode kernel); debug mode
    rejects a slot that is not the table's slot of the new position."""
    torch = need_gpu()
    from paged_kv_cache_122_amd import _lib as pa
    from paged_kv_cache_122_amd import device as dev

    w = workloads.make("tiny_gqa4_d64")
    dw = dev.upload(w)
    out = torch.empty_like(dw.q)
    for opts in ({}, {"partition_tokens": 32}):
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        _run(pa, dw, w, out, opts, kernel_events=ev)
        assert ev[0].elapsed_time(ev[1]) > 0.0
    old = pa.set_debug(True)
    try:
        _run(pa, dw, w, out, {})  # valid
        bad = dw.slot_mapping.clone()
        bad[0] += 1
        with pytest.raises(pa.PaError) as e:
            pa.append_decode(out, dw.q, dw.k_new, dw.v_new, bad, dw.k_cache, dw.v_cache, dw.block_tables,
                             dw.context_lens, w.scale, w.block_size)
        assert e.value.code == pa.PA_ERR_CONTRACT
        # no token (context length 0) but a slot to store it in
        lens = dw.context_lens.clone()
        lens[0] = 0
        with pytest.raises(pa.PaError) as e:
            pa.append_decode(out, dw.q, dw.k_new, dw.v_new, dw.slot_mapping, dw.k_cache, dw.v_cache,
                             dw.block_tables, lens, w.scale, w.block_size)
        assert e.value.code == pa.PA_ERR_CONTRACT
    finally:
        pa.set_debug(old)


def test_append_decode_empty_contexts():
    """Sequences with no tokens (length 0, slot -1) beside others: their rows are
    zeros and nothing is stored for them, on the one-launch path."""
    torch = need_gpu()
    from paged_kv_cache_122_amd import _lib as pa
    from paged_kv_cache_122_amd import device as dev

    rng = np.random.Generator(np.random.PCG64(77))
    lens = [0, 33, 0, 200, 1]
    nb = 40
    _, tables = workloads.place_independent(rng, lens, 16, nb)
    w = workloads.build_workload("empty_contexts", 77, rng, num_q_heads=8, num_kv_heads=2, head_dim=128,
                                 block_size=16, num_blocks=nb, tables=tables, context_lens=lens, width=16)
    assert list(w.slot_mapping[[0, 2]]) == [-1, -1]
    dw = dev.upload(w)
    kst, vst, ref = oracle_step(w)
    out = torch.full(dw.q.shape, float("nan"), dtype=torch.float32, device="cuda")
    _run(pa, dw, w, out, {})
    assert np.array_equal(dev.bf16_bits(dw.k_cache[dw.owned]), kst.blocks)
    assert np.array_equal(dev.bf16_bits(dw.v_cache[dw.owned]), vst.blocks)
    got = out.double().cpu().numpy()
    assert np.all(got[[0, 2]] == 0.0)
    assert_close(got, ref, "empty_contexts")


@pytest.mark.parametrize("b,d,hq,hkv", [(8, 128, 16, 4), (32, 64, 24, 2), (16, 64, 8, 8)])
def test_append_decode_block_sizes(b, d, hq, hkv):
    """The one-launch path at every block size (and MHA, which takes the
    append kernel and the VALU decode): 12 sequences of U[1, 900] tokens."""
    torch = need_gpu()
    from paged_kv_cache_122_amd import _lib as pa
    from paged_kv_cache_122_amd import device as dev

    rng = np.random.Generator(np.random.PCG64(900 + b + d + hq))
    lens = rng.integers(1, 900, size=12, endpoint=True).tolist()
    nb = int(1.2 * sum(-(-L // b) for L in lens)) + 4
    _, tables = workloads.place_independent(rng, lens, b, nb)
    w = workloads.build_workload(f"ad_b{b}", 900 + b, rng, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                                 block_size=b, num_blocks=nb, tables=tables, context_lens=lens,
                                 width=max(len(t) for t in tables))
    dw = dev.upload(w)
    kst, vst, ref = oracle_step(w)
    out = torch.empty(dw.q.shape, dtype=torch.float32, device="cuda")
    _run(pa, dw, w, out, {})
    assert np.array_equal(dev.bf16_bits(dw.k_cache[dw.owned]), kst.blocks)
    assert np.array_equal(dev.bf16_bits(dw.v_cache[dw.owned]), vst.blocks)
    assert_close(out.double().cpu().numpy(), ref, f"ad_b{b}")


@pytest.mark.parametrize("part", [256, 32])
@pytest.mark.parametrize("g,d,b", [(1, 128, 16), (4, 64, 8), (16, 128, 32)], ids=["mha", "gqa4_d64_b8", "gqa16_b32"])
def test_append_decode_shared_step_edges(g, d, b, part):
    """The partitioned step whose shared-partition kernel takes the append, at
    partitions of 256 tokens (and of 32, so that the combine joins up to 35
    pieces of a row, more than one batch of its loads): contexts of one token
    (nothing read from the pool), lengths on and either side of partition
    boundaries (the new token alone in the last partition, or ending it),
    empty sequences (slot -1) and random ones; 40 sequences x 8 KV heads, so
    the schedule does not take the deep pipeline.  Pools bit-exact, every row
    against the oracle, and the route is the shared step and its combine."""
    torch = need_gpu()
    from paged_kv_cache_122_amd import _lib as pa
    from paged_kv_cache_122_amd import device as dev

    rng = np.random.Generator(np.random.PCG64(1300 + g + d + b))
    edges = [1, 2, 255, 256, 257, 511, 512, 513, 768, 1024, 0, 0, 16, 17]
    lens = edges + rng.integers(1, 1100, size=40 - len(edges), endpoint=True).tolist()
    nb = int(1.2 * sum(-(-L // b) for L in lens)) + 4
    _, tables = workloads.place_independent(rng, lens, b, nb)
    w = workloads.build_workload(f"shared_step_g{g}", 1300 + g, rng, num_q_heads=8 * g, num_kv_heads=8, head_dim=d,
                                 block_size=b, num_blocks=nb, tables=tables, context_lens=lens,
                                 width=max(len(t) for t in tables))
    print(f"[shared_step G={g} D={d} B={b} part={part}] S={w.num_seqs}", flush=True)
    dw = dev.upload(w)
    kst, vst, ref = oracle_step(w)
    out = torch.full(dw.q.shape, float("nan"), dtype=torch.float32, device="cuda")
    _run(pa, dw, w, out, {"partition_tokens": part})
    route = pa.last_launch()
    assert route[0].startswith("decode_shared<") and route[-1].startswith("combine_append<"), route
    assert np.array_equal(dev.bf16_bits(dw.k_cache[dw.owned]), kst.blocks), "K pool differs"
    assert np.array_equal(dev.bf16_bits(dw.v_cache[dw.owned]), vst.blocks), "V pool differs"
    got = out.double().cpu().numpy()
    assert np.all(got[[10, 11]] == 0.0)
    a, r = assert_close(got, ref, f"shared_step_g{g}")
    print(f"[shared_step G={g}] max|err| {a:.2e} rel RMS {r:.2e}", flush=True)
