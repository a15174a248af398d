"""GPU checks beyond the named configurations: edge lengths, every supported
geometry, both compute paths, split-K variants, invariances the pages fix
(physical placement does not matter; one token returns v0), determinism,
strided operands, workspace and debug-mode contracts."""

import numpy as np
import pytest

import oracle
from gpu_util import assert_close, assert_close_bf16, need_gpu, oracle_step
from paged_kv_cache_122_amd import workloads

pytestmark = pytest.mark.gpu

EDGE_LENS = [1, 2, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 255, 511, 512, 513, 1000, 1024, 1537]


def _setup(w):
    from paged_kv_cache_122_amd import device as dev
    dw = dev.upload(w)
    from paged_kv_cache_122_amd import _lib as pa
    pa.cache_append(dw.k_new, dw.v_new, dw.slot_mapping, dw.k_cache, dw.v_cache)
    return dw


def _decode(torch, w, dw, out_dtype=None, **opts):
    from paged_kv_cache_122_amd import _lib as pa
    out = torch.empty(dw.q.shape, dtype=out_dtype or torch.bfloat16, device=dw.q.device)
    if opts:
        ws = None
        nbytes = pa.workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                    opts.get("max_context_len") or w.table_width * w.block_size,
                                    opts.get("partition_tokens", 0))
        if nbytes:
            ws = pa.alloc_workspace(nbytes, dw.q.device)
        pa.decode_ex(out, dw.q, dw.k_cache, dw.v_cache, dw.block_tables, dw.context_lens, w.scale,
                     w.block_size, workspace=ws, **opts)
    else:
        pa.decode(out, dw.q, dw.k_cache, dw.v_cache, dw.block_tables, dw.context_lens, w.scale,
                  w.block_size)
    torch.cuda.synchronize()
    return out


def _as_f64(torch, out):
    from paged_kv_cache_122_amd import device as dev
    if out.dtype == torch.float32:
        return out.double().cpu().numpy()
    return oracle.bf16_bits_to_f64(dev.bf16_bits(out))


GEOMS = [(D, B, Hq, Hkv) for D in (64, 128) for B in (8, 16, 32)
         for (Hq, Hkv) in ((4, 4), (4, 2), (6, 2), (8, 2), (16, 2), (32, 1))]


@pytest.mark.parametrize("D,B,Hq,Hkv", GEOMS, ids=[f"D{g[0]}-B{g[1]}-G{g[2]//g[3]}" for g in GEOMS])
def test_edge_lengths_every_geometry(D, B, Hq, Hkv):
    torch = need_gpu()
    w = workloads.random_workload(7 + D + B + Hq, EDGE_LENS, num_q_heads=Hq, num_kv_heads=Hkv,
                                  head_dim=D, block_size=B)
    print(f"geometry D={D} B={B} Hq={Hq} Hkv={Hkv}", flush=True)
    dw = _setup(w)
    _, _, ref = oracle_step(w)
    assert_close_bf16(_as_f64(torch, _decode(torch, w, dw)), ref, "bf16 out")
    assert_close(_as_f64(torch, _decode(torch, w, dw, torch.float32)), ref, "f32 out",
                 max_abs=1e-4, rel_rms=1e-4)


@pytest.mark.parametrize("part", [32, 64, 96, 512, -1, -2])
def test_split_variants(part):
    torch = need_gpu()
    w = workloads.random_workload(31, [3000, 1, 700, 2049, 64], num_q_heads=16, num_kv_heads=4,
                                  head_dim=128, block_size=16)
    dw = _setup(w)
    _, _, ref = oracle_step(w)
    assert_close_bf16(_as_f64(torch, _decode(torch, w, dw, partition_tokens=part)), ref, f"part {part}")
    assert_close(_as_f64(torch, _decode(torch, w, dw, torch.float32, partition_tokens=part)), ref,
                 f"part {part} f32", max_abs=1e-4, rel_rms=1e-4)


STREAM_CASES = [
    # (lens, Hq, Hkv, D, B, workgroups_per_cu)
    ([3000, 1, 700, 2049, 64], 16, 4, 128, 16, 1),     # tiny per-wave ranges: every pair split
    ([3000, 1, 700, 2049, 64], 16, 4, 128, 16, 8),
    ([20000, 30000], 32, 8, 128, 32, 1),               # ranges longer than 64 tiles
    ([0, 17, 0, 5000, 0], 8, 2, 64, 8, 2),             # empty contexts between live ones
    ([0, 0, 0], 8, 2, 64, 16, 2),                      # nothing to read at all
    ([33, 900, 4100, 2], 4, 4, 128, 16, 1),            # MHA (VALU) pieces
    ([33, 900, 4100, 2], 8, 4, 64, 8, 4),              # two heads per KV head (VALU)
    ([700, 1, 2500], 64, 2, 128, 16, 2),               # 32 heads per KV head: two column groups
]


@pytest.mark.parametrize("case", STREAM_CASES, ids=[f"stream{i}" for i in range(len(STREAM_CASES))])
def test_stream_schedule(case):
    torch = need_gpu()
    lens, Hq, Hkv, D, B, wpc = case
    w = workloads.random_workload(71 + len(lens) + wpc, lens, num_q_heads=Hq, num_kv_heads=Hkv,
                                  head_dim=D, block_size=B)
    dw = _setup(w)
    _, _, ref = oracle_step(w)
    got = _decode(torch, w, dw, torch.float32, partition_tokens=-2, workgroups_per_cu=wpc)
    assert_close(_as_f64(torch, got), ref, f"stream-K wpc={wpc}", max_abs=1e-4, rel_rms=1e-4)
    got16 = _decode(torch, w, dw, partition_tokens=-2, workgroups_per_cu=wpc)
    assert_close_bf16(_as_f64(torch, got16), ref, f"stream-K bf16 wpc={wpc}")
    for s, L in enumerate(lens):
        if L == 0:
            assert torch.all(got[s] == 0)


@pytest.mark.parametrize("G", [1, 2])
def test_valu_and_mfma_paths_agree(G):
    torch = need_gpu()
    w = workloads.random_workload(41, [5, 300, 1500], num_q_heads=4 * G, num_kv_heads=4,
                                  head_dim=128, block_size=16)
    dw = _setup(w)
    _, _, ref = oracle_step(w)
    valu = _decode(torch, w, dw, torch.float32, path=1)
    mfma = _decode(torch, w, dw, torch.float32, path=2)
    assert_close(_as_f64(torch, valu), ref, "valu", max_abs=1e-4, rel_rms=1e-4)
    assert_close(_as_f64(torch, mfma), ref, "mfma", max_abs=1e-4, rel_rms=1e-4)


def test_context_len_one_returns_v0_bit_exact():
    torch = need_gpu()
    from paged_kv_cache_122_amd import device as dev
    for Hq, Hkv in ((8, 2), (4, 4)):
        w = workloads.random_workload(51, [1, 1, 1, 1], num_q_heads=Hq, num_kv_heads=Hkv,
                                      head_dim=64, block_size=16)
        dw = _setup(w)
        out = dev.bf16_bits(_decode(torch, w, dw))
        G = Hq // Hkv
        assert np.array_equal(out, np.repeat(w.v_new, G, axis=1))


def test_empty_context_gives_zeros():
    torch = need_gpu()
    w = workloads.random_workload(52, [0, 40, 0], num_q_heads=8, num_kv_heads=2, head_dim=128,
                                  block_size=16)
    dw = _setup(w)
    out = _as_f64(torch, _decode(torch, w, dw))
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    _, _, ref = oracle_step(w)
    assert_close_bf16(out[1], ref[1], "middle row")


def test_block_permutation_gives_identical_bits():
    torch = need_gpu()
    from paged_kv_cache_122_amd import device as dev
    w = workloads.random_workload(53, [600, 33, 1200, 17], num_q_heads=32, num_kv_heads=8,
                                  head_dim=128, block_size=16)
    dw = _setup(w)
    ref = dev.bf16_bits(_decode(torch, w, dw))
    perm = torch.randperm(w.num_blocks, generator=torch.Generator().manual_seed(5)).to(dw.q.device)
    k2 = torch.empty_like(dw.k_cache)
    v2 = torch.empty_like(dw.v_cache)
    k2[perm] = dw.k_cache
    v2[perm] = dw.v_cache
    bt = dw.block_tables.long()
    bt2 = torch.where(bt >= 0, perm[bt.clamp(min=0)], bt).to(torch.int32)
    dw.k_cache, dw.v_cache, dw.block_tables = k2, v2, bt2
    assert np.array_equal(dev.bf16_bits(_decode(torch, w, dw)), ref)


@pytest.mark.parametrize("part", [0, 512, -2])
def test_runs_are_bitwise_deterministic(part):
    torch = need_gpu()
    from paged_kv_cache_122_amd import device as dev
    w = workloads.random_workload(54, [4000, 2500, 100], num_q_heads=32, num_kv_heads=8,
                                  head_dim=128, block_size=16)
    dw = _setup(w)
    a = dev.bf16_bits(_decode(torch, w, dw, partition_tokens=part))
    for _ in range(3):
        assert np.array_equal(dev.bf16_bits(_decode(torch, w, dw, partition_tokens=part)), a)


def test_strided_q_and_out():
    torch = need_gpu()
    w = workloads.random_workload(55, [77, 300], num_q_heads=8, num_kv_heads=2, head_dim=128,
                                  block_size=16)
    dw = _setup(w)
    from paged_kv_cache_122_amd import _lib as pa
    S, Hq, D = dw.q.shape
    big_q = torch.zeros(S, Hq + 4, D, dtype=torch.bfloat16, device=dw.q.device)
    big_q[:, 2:2 + Hq] = dw.q
    q_view = big_q[:, 2:2 + Hq]
    big_out = torch.zeros(S, Hq, D + 64, dtype=torch.float32, device=dw.q.device)
    out_view = big_out[:, :, :D]
    pa.decode(out_view, q_view, dw.k_cache, dw.v_cache, dw.block_tables, dw.context_lens, w.scale,
              w.block_size)
    torch.cuda.synchronize()
    _, _, ref = oracle_step(w)
    assert_close(out_view.double().cpu().numpy(), ref, "strided", max_abs=1e-4, rel_rms=1e-4)
    assert torch.all(big_out[:, :, D:] == 0)


def test_decode_ex_matches_decode_and_checks_workspace():
    torch = need_gpu()
    from paged_kv_cache_122_amd import _lib as pa
    from paged_kv_cache_122_amd import device as dev
    w = workloads.random_workload(56, [1500, 900, 2048], num_q_heads=32, num_kv_heads=8,
                                  head_dim=128, block_size=16)
    dw = _setup(w)
    a = dev.bf16_bits(_decode(torch, w, dw))
    b = dev.bf16_bits(_decode(torch, w, dw, workgroups_per_cu=0))  # same schedule, caller workspace
    assert np.array_equal(a, b)
    out = torch.empty_like(dw.q)
    for part in (512, -2):
        with pytest.raises(pa.PaError) as e:
            pa.decode_ex(out, dw.q, dw.k_cache, dw.v_cache, dw.block_tables, dw.context_lens, w.scale,
                         w.block_size, partition_tokens=part,
                         workspace=torch.zeros(64, dtype=torch.uint8, device=dw.q.device))
        assert e.value.code == pa.PA_ERR_WORKSPACE


def test_workspace_reuse_across_layouts():
    """Regression: a split call whose counters sit where an earlier, differently
    sized call left partial results (library workspace and one reused
    caller workspace) must still combine correctly."""
    torch = need_gpu()
    from paged_kv_cache_122_amd import _lib as pa
    big = workloads.random_workload(61, [3000] * 24, num_q_heads=64, num_kv_heads=8, head_dim=128,
                                    block_size=16)
    small = workloads.random_workload(62, [1500, 2000, 1100] * 8, num_q_heads=40, num_kv_heads=40,
                                      head_dim=128, block_size=16)
    dbig, dsmall = _setup(big), _setup(small)
    _, _, ref_small = oracle_step(small)
    _decode(torch, big, dbig)                     # library workspace, large layout
    assert_close_bf16(_as_f64(torch, _decode(torch, small, dsmall)), ref_small, "library workspace")
    nbytes = max(pa.workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                    w.table_width * w.block_size) for w in (big, small))
    ws = pa.alloc_workspace(nbytes, dbig.q.device)
    for w, dw in ((big, dbig), (small, dsmall)):
        out = torch.empty_like(dw.q)
        pa.decode_ex(out, dw.q, dw.k_cache, dw.v_cache, dw.block_tables, dw.context_lens, w.scale,
                     w.block_size, workspace=ws)
    torch.cuda.synchronize()
    assert_close_bf16(_as_f64(torch, out), ref_small, "caller workspace")


def test_debug_mode_contracts():
    torch = need_gpu()
    from paged_kv_cache_122_amd import _lib as pa
    w = workloads.random_workload(57, [40, 20], num_q_heads=4, num_kv_heads=2, head_dim=64,
                                  block_size=16)
    dw = _setup(w)
    out = torch.empty_like(dw.q)
    prev = pa.set_debug(True)
    try:
        pa.decode(out, dw.q, dw.k_cache, dw.v_cache, dw.block_tables, dw.context_lens, w.scale, 16)
        bad = dw.block_tables.clone()
        bad[0, 1] = w.num_blocks
        with pytest.raises(pa.PaError) as e:
            pa.decode(out, dw.q, dw.k_cache, dw.v_cache, bad, dw.context_lens, w.scale, 16)
        assert e.value.code == pa.PA_ERR_CONTRACT
        bad = dw.block_tables.clone()
        bad[1, 0] = -1
        with pytest.raises(pa.PaError) as e:
            pa.decode(out, dw.q, dw.k_cache, dw.v_cache, bad, dw.context_lens, w.scale, 16)
        assert e.value.code == pa.PA_ERR_CONTRACT
        lens = dw.context_lens.clone()
        lens[0] = w.table_width * 16 + 1
        with pytest.raises(pa.PaError) as e:
            pa.decode(out, dw.q, dw.k_cache, dw.v_cache, dw.block_tables, lens, w.scale, 16)
        assert e.value.code == pa.PA_ERR_CONTRACT
        dup = dw.slot_mapping.clone()
        dup[1] = dup[0]
        with pytest.raises(pa.PaError) as e:
            pa.cache_append(dw.k_new, dw.v_new, dup, dw.k_cache, dw.v_cache)
        assert e.value.code == pa.PA_ERR_CONTRACT
        oob = dw.slot_mapping.clone()
        oob[0] = w.num_blocks * 16
        with pytest.raises(pa.PaError) as e:
            pa.cache_append(dw.k_new, dw.v_new, oob, dw.k_cache, dw.v_cache)
        assert e.value.code == pa.PA_ERR_CONTRACT
        dev_ = dw.q.device
        for pairs in ([[1, 5], [2, 5]],            # a destination twice
                      [[1, 5], [5, 6]],            # a destination that is also a source
                      [[1, w.num_blocks]]):        # outside the pool
            with pytest.raises(pa.PaError) as e:
                pa.copy_blocks(dw.k_cache, dw.v_cache, torch.tensor(pairs, dtype=torch.int64, device=dev_))
            assert e.value.code == pa.PA_ERR_CONTRACT
    finally:
        pa.set_debug(prev)
    torch.cuda.synchronize()


def test_negative_slots_are_skipped():
    torch = need_gpu()
    from paged_kv_cache_122_amd import _lib as pa
    w = workloads.random_workload(58, [10, 30], num_q_heads=4, num_kv_heads=2, head_dim=64,
                                  block_size=8)
    from paged_kv_cache_122_amd import device as dev
    dw = dev.upload(w)
    before_k = dw.k_cache.clone()
    before_v = dw.v_cache.clone()
    skip = torch.full_like(dw.slot_mapping, -1)
    pa.cache_append(dw.k_new, dw.v_new, skip, dw.k_cache, dw.v_cache)
    torch.cuda.synchronize()
    assert torch.equal(dw.k_cache.view(torch.int16), before_k.view(torch.int16))
    assert torch.equal(dw.v_cache.view(torch.int16), before_v.view(torch.int16))


@pytest.mark.gpu
@pytest.mark.parametrize("part", [-1, 512, -2])
def test_kernel_timing_events(part):
    """Timing events change nothing in the result and bracket the decode kernel."""
    torch = need_gpu()
    from paged_kv_cache_122_amd import device as dev
    w = workloads.random_workload(57, [3000, 1200, 64, 700], num_q_heads=32, num_kv_heads=8,
                                  head_dim=128, block_size=16)
    dw = _setup(w)
    ref = dev.bf16_bits(_decode(torch, w, dw, partition_tokens=part))
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    call0, call1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(2):
        call0.record()
        got = _decode(torch, w, dw, partition_tokens=part, kernel_events=(start, stop))
        call1.record()
        torch.cuda.synchronize()
        assert np.array_equal(dev.bf16_bits(got), ref)
        t_kernel, t_call = start.elapsed_time(stop), call0.elapsed_time(call1)
        assert 0.0 < t_kernel <= t_call + 1e-3, (t_kernel, t_call)


@pytest.mark.gpu
@pytest.mark.parametrize("S", [5, 256, 257, 300])
@pytest.mark.parametrize("part", [-1, 64])
def test_longest_first_order_covers_every_sequence(S, part):
    """Partitioned grids hand rows to sequences in decreasing length order (the
    identity order past 256 sequences): with many ties and empty contexts every
    sequence must still be computed exactly once and land in its own row."""
    torch = need_gpu()
    rng = np.random.default_rng(900 + S)
    lens = rng.choice([0, 1, 16, 17, 100, 100, 100, 250], size=S)
    w = workloads.random_workload(901 + S, lens, num_q_heads=8, num_kv_heads=2, head_dim=64,
                                  block_size=16)
    print(f"S={S} part={part}", flush=True)
    dw = _setup(w)
    _, _, ref = oracle_step(w)
    assert_close_bf16(_as_f64(torch, _decode(torch, w, dw, partition_tokens=part)), ref, "bf16 out")



@pytest.mark.parametrize("D,B,Hkv", [(128, 16, 8), (64, 8, 2), (128, 32, 40)])
def test_copy_blocks_bit_exact(D, B, Hkv):
    """Random batches of block copies match the oracle's copy bit for bit; rows
    naming a block outside the pool are skipped (pool unchanged)."""
    torch = need_gpu()
    from paged_kv_cache_122_amd import _lib as pa
    from paged_kv_cache_122_amd import device as dev
    rng = np.random.default_rng(D + B + Hkv)
    w = workloads.random_workload(71 + B, rng.integers(1, 200, size=24), num_q_heads=Hkv, num_kv_heads=Hkv,
                                  head_dim=D, block_size=B)
    dw = dev.upload(w)
    owned = w.owned
    src = rng.choice(owned, size=min(12, len(owned) // 2), replace=False)
    rest = np.setdiff1d(np.arange(w.num_blocks), src)
    dst = rng.choice(rest, size=len(src), replace=False)
    pairs = np.stack([src, dst], 1).astype(np.int64)
    # the oracle's pools cover every block here: start from the device's contents
    k_all = dev.bf16_bits(dw.k_cache).copy()
    v_all = dev.bf16_bits(dw.v_cache).copy()
    oracle.copy_blocks(pairs, k_all, v_all)
    pa.copy_blocks(dw.k_cache, dw.v_cache, torch.from_numpy(pairs).to(dw.q.device))
    torch.cuda.synchronize()
    assert np.array_equal(dev.bf16_bits(dw.k_cache), k_all)
    assert np.array_equal(dev.bf16_bits(dw.v_cache), v_all)
    # out-of-range rows do nothing
    pa.copy_blocks(dw.k_cache, dw.v_cache,
                   torch.tensor([[-1, int(dst[0])], [int(src[0]), w.num_blocks], [int(src[0]), -5]],
                                dtype=torch.int64, device=dw.q.device))
    torch.cuda.synchronize()
    assert np.array_equal(dev.bf16_bits(dw.k_cache), k_all)
    assert np.array_equal(dev.bf16_bits(dw.v_cache), v_all)


@pytest.mark.parametrize("D,B,Hq,Hkv", [(128, 16, 32, 8), (64, 32, 8, 2), (128, 8, 64, 8), (64, 16, 4, 4)])
def test_contiguous_control(D, B, Hq, Hkv):
    """The unpaged control equals the paged decode's unsplit MFMA schedule bit for
    bit (same tiles in the same order), and the oracle on the unpaged layout."""
    torch = need_gpu()
    from paged_kv_cache_122_amd import _lib as pa
    from paged_kv_cache_122_amd import device as dev
    lens = [0, 1, 15, 16, 17, 100, 511, 1000, 1024, 3] * 3
    w = workloads.random_workload(81 + D + B, lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                  block_size=B)
    print(f"contiguous D={D} B={B} Hq={Hq} Hkv={Hkv}", flush=True)
    dw = _setup(w)
    paged = _decode(torch, w, dw, partition_tokens=-1, path=2)
    k, v = dev.contiguous_copy(dw, w)
    out = torch.empty_like(dw.q)
    pa.decode_contiguous(out, dw.q, k, v, dw.context_lens, w.scale)
    torch.cuda.synchronize()
    assert np.array_equal(dev.bf16_bits(out), dev.bf16_bits(paged))
    ref = oracle.contiguous_decode(w.q, dev.bf16_bits(k), dev.bf16_bits(v), w.context_lens, w.scale)
    assert_close_bf16(_as_f64(torch, out), ref, "contiguous")
    out32 = torch.empty(dw.q.shape, dtype=torch.float32, device=dw.q.device)
    pa.decode_contiguous(out32, dw.q, k, v, dw.context_lens, w.scale)
    torch.cuda.synchronize()
    assert_close(_as_f64(torch, out32), ref, "contiguous f32", max_abs=1e-4, rel_rms=1e-4)
