"""Host logic against the values the pages print (tests/golden/page_values.json):
sizing formulas, block counts, the block manager and copy-on-write."""

import json
import os

import numpy as np
import pytest

from paged_kv_cache_122_amd import layout, sizing, workloads
from paged_kv_cache_122_amd.blockpool import (BlockPool, Sequence, fork, free, reserve_slot, reserve_slots,
                                              slot_of_position)

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))
GiB = 2 ** 30
MiB = 2 ** 20


@pytest.mark.parametrize("case", GOLDEN["kv_bytes_per_token"])
def test_token_cache_bytes(case):
    got = sizing.token_cache_bytes(case["layers"], case["kv_heads"], case["head_dim"], case["dtype_bytes"])
    assert got == case["bytes"]


def test_sevydevy_script_outputs():
    per_token = sizing.token_cache_bytes(32, 8, 128, 2)
    assert per_token * 8192 / GiB == GOLDEN["gib_for_8192_tokens_32_layer_model"]["gib"]
    c = GOLDEN["blocks_in_60_gib"]
    blocks = 60 * GiB // (per_token * c["block_size"])
    assert blocks == c["blocks"]
    assert blocks * c["block_size"] == c["tokens"]


def test_block_bytes_and_pool_capacity():
    c = GOLDEN["block_bytes_llama3_70b"]
    per_layer = sizing.block_bytes(c["block_size"], c["kv_heads"], c["head_dim"], c["dtype_bytes"])
    assert per_layer == c["bytes_per_layer"]
    all_layers = sizing.block_bytes(c["block_size"], c["kv_heads"], c["head_dim"], c["dtype_bytes"], c["layers"])
    assert all_layers / MiB == c["mib_all_layers"]
    blocks = c["pool_gib"] * GiB // all_layers
    assert blocks == c["blocks"]
    assert blocks * c["block_size"] == c["tokens"]


@pytest.mark.parametrize("case", GOLDEN["block_table_bytes"])
def test_block_table_bytes(case):
    if "max_model_len" in case:
        assert sizing.blocks_for_tokens(case["max_model_len"], case["block_size"]) == case["max_blocks_per_seq"]
        assert case["num_seqs"] * case["max_blocks_per_seq"] == case["numel"]
    assert sizing.block_table_bytes(case["num_seqs"], case["max_blocks_per_seq"]) == case["bytes"]


@pytest.mark.parametrize("case", GOLDEN["block_counts"])
def test_block_counts(case):
    assert sizing.blocks_for_tokens(case["tokens"], case["block_size"]) == case["blocks"]
    if "last_block_used" in case:
        assert sizing.tail_fill(case["tokens"], case["block_size"]) == case["last_block_used"]
    if "block_table" in case:
        # token -> (logical block, offset) -> physical slot, per the page's example
        B = case["block_size"]
        table = case["block_table"]
        for i, (lo, hi) in enumerate(case["logical_block_tokens"]):
            for t in (lo, hi):
                assert slot_of_position(table, t, B) == table[i] * B + (t - lo)


def test_tail_waste_bound():
    for B in (8, 16, 32):
        for L in range(1, 200):
            waste = sizing.blocks_for_tokens(L, B) * B - L
            assert 0 <= waste <= B - 1
            assert sizing.tail_fill(L, B) == B - waste


def test_block_manager_demo():
    c = GOLDEN["block_manager_demo"]
    pool = BlockPool(c["total_blocks"], c["block_size"])
    seq = Sequence()
    new_at, got_blocks = [], []
    for t in range(c["tokens"]):
        before = len(seq.table)
        reserve_slot(pool, seq)
        if len(seq.table) > before:
            new_at.append(t)
            got_blocks.append(seq.table[-1])
    assert new_at == c["new_block_at_tokens"]
    assert got_blocks == c["blocks_allocated"]
    free(pool, seq)
    assert pool.blocks_in_use() == 0
    assert pool.num_free() == c["total_blocks"]


def test_copy_on_write_script():
    c = GOLDEN["cow_script"]
    pool = BlockPool(c["free_blocks"], c["block_size"])
    prompt = Sequence()
    reserve_slots(pool, prompt, c["prompt_tokens"])
    assert len(prompt.table) == 63
    samples = [fork(pool, prompt) for _ in range(c["samples"])]
    for b in prompt.table:          # the parent itself is done
        pool.release(b)
    for _ in range(c["tokens_per_sample"]):
        for s in samples:
            reserve_slot(pool, s)
    assert pool.blocks_in_use() == c["blocks_in_use"]
    assert pool.ref[prompt.table[0]] == c["first_block_shared_by"]
    assert [s.table[62] for s in samples] == c["last_prompt_block_per_sample"]
    unshared = c["samples"] * sizing.blocks_for_tokens(c["prompt_tokens"] + c["tokens_per_sample"], c["block_size"])
    assert unshared == c["blocks_without_sharing"]
    assert round(100 * (1 - c["blocks_in_use"] / unshared)) == c["saving_percent"]
    # three samples copied the shared tail block (8 filled slots each); the last kept it
    assert [(src, n) for src, _, n in pool.pending_copies] == [(62, 8)] * 3


def test_system_prompt_sharing():
    c = GOLDEN["system_prompt_sharing"]
    B = c["block_size"]
    full = c["prompt_tokens"] // B
    assert full == c["shared_full_blocks"]
    assert full * B == c["tokens_in_full_blocks"]
    assert c["prompt_tokens"] - full * B == c["recomputed_tail_tokens"]
    assert full + c["chats"] == c["blocks_with_sharing"]
    assert c["chats"] * sizing.blocks_for_tokens(c["prompt_tokens"], B) == c["blocks_without_sharing"]
    assert (c["prompt_tokens"] // 128) * 128 == c["block_size_128_tokens_in_full_blocks"]


def test_layout_pack_roundtrip_and_tiles():
    rng = np.random.default_rng(0)
    for B in (8, 16, 32):
        for D in (64, 128):
            x = rng.integers(0, 2 ** 16, size=(3, 2, B, D), dtype=np.uint16)
            pk, pv = layout.pack_k(x), layout.pack_v(x)
            assert pk.shape == layout.k_cache_shape(3, 2, D, B)
            assert pv.shape == layout.v_cache_shape(3, 2, D, B)
            assert np.array_equal(layout.unpack_k(pk), x)
            assert np.array_equal(layout.unpack_v(pv), x)
            # element positions follow the documented formula
            for (b, h, t, d) in [(0, 0, 0, 0), (2, 1, B - 1, D - 1), (1, 0, 5 % B, 37)]:
                assert pk[b, h, d // 8, t, d % 8] == x[b, h, t, d]
                assert pv[b, h, t // 4, d, t % 4] == x[b, h, t, d]
            # one (block, head) tile is one contiguous chunk of B*D elements
            assert pk[1, 1].size == B * D and pk[1, 1].flags["C_CONTIGUOUS"]


def test_f32_to_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        rng.uniform(-1e30, 1e30, 1000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3e-39], dtype=np.float32)])
    ours = workloads.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_tiny_workload_structure():
    w = workloads.tiny_gqa()
    assert w.context_lens.tolist() == [1, 17, 100, 900]
    assert (w.block_tables >= 0).sum() == 1 + 2 + 7 + 57
    assert w.block_tables.shape == (4, 57)
    assert len(set(w.owned.tolist())) == 67 and w.owned.max() < 128
    for s in range(4):
        L = int(w.context_lens[s])
        t = w.block_tables[s]
        assert w.slot_mapping[s] == t[(L - 1) // 16] * 16 + (L - 1) % 16
        assert (t[sizing.blocks_for_tokens(L, 16):] == -1).all()
    # the slot the append will write is poisoned before the append
    kstore, vstore = w.stores()
    for s in range(4):
        blk, off = divmod(int(w.slot_mapping[s]), 16)
        assert (kstore[blk][:, :, off, :] == workloads.NAN_BF16).all()
        assert (vstore[blk][:, off // 4, :, off % 4] == workloads.NAN_BF16).all()


def test_prefix_sharing_workload_structure():
    w = workloads.opt13b_prefix_sharing()
    assert w.num_seqs == 128
    shared = w.block_tables[:, :64]
    for g in range(16):
        rows = shared[g * 8:(g + 1) * 8]
        assert (rows == rows[0]).all()
    assert len(set(shared.ravel().tolist())) == 16 * 64
    ref = dict(zip(w.owned.tolist(), w.refcount.tolist()))
    assert all(ref[int(b)] == 8 for b in shared.ravel())
    tails = w.context_lens - 1024
    assert tails.min() >= 16 and tails.max() <= 1024
    # this step's token lands in a private block
    for s in range(128):
        assert ref[int(w.slot_mapping[s]) // 16] == 1
    assert w.unique_kv_bytes() < w.effective_kv_bytes()


def test_cow_fork_workload_copies_the_shared_partial_block():
    """Forking 8 samples from a 1,000-token prompt: the last block (8 of 16
    tokens) is shared, so the first token of every sample but the last writer
    goes to a fresh copy (the chenyuan1125 essay; the sevydevy CoW script's rule
    that a shared last block is copied before a write)."""
    import oracle
    w = workloads.make("opt13b_cow_fork_b128")
    B = w.block_size
    assert w.copies.shape == (16 * 7, 2)
    assert np.all(w.context_lens == 1001)
    kst, vst = w.stores()
    # before the copies every destination is poison
    for _, dst in w.copies:
        assert np.all(kst[int(dst)] == workloads.NAN_BF16)
    oracle.copy_blocks(w.copies, kst, vst)
    oracle.cache_append(w.k_new, w.v_new, w.slot_mapping, kst, vst, B)
    for g in range(16):
        ctx = []
        for j in range(8):
            s = 8 * g + j
            K, V = oracle.gather_sequence(kst, vst, w.block_tables[s], int(w.context_lens[s]), B)
            assert np.all(np.isfinite(K)) and np.all(np.isfinite(V))
            ctx.append((K, V))
            # the new token sits at position 1000 of this sample alone
            assert np.array_equal(K[:, 1000], oracle.bf16_bits_to_f64(w.k_new[s]))
        for K, V in ctx[1:]:  # the prompt is the same for every sample of a group
            assert np.array_equal(K[:, :1000], ctx[0][0][:, :1000])
            assert np.array_equal(V[:, :1000], ctx[0][1][:, :1000])
    # skipping the copies leaves the copied samples reading poison
    kst2, vst2 = w.stores()
    oracle.cache_append(w.k_new, w.v_new, w.slot_mapping, kst2, vst2, B)
    K, _ = oracle.gather_sequence(kst2, vst2, w.block_tables[0], 1001, B)
    assert np.isnan(K[:, 992:1000]).all()


@pytest.mark.parametrize("B", [8, 16, 32])
def test_contiguous_copy_matches_a_plain_rearrangement(B):
    """The device-side gather that builds the unpaged control cache (torch on the
    CPU here) equals a token-by-token numpy rearrangement of the blocks, on every
    token inside a context."""
    torch = pytest.importorskip("torch")
    import oracle
    from paged_kv_cache_122_amd import device as dev
    from test_oracle import _contiguous_copy
    w = workloads.random_workload(5 + B, [1, 9, 16, 17, 40, 77], num_q_heads=4, num_kv_heads=2,
                                  head_dim=64, block_size=B)
    dw = dev.upload(w, "cpu")
    kst, vst = w.stores()
    k_ref, v_ref = _contiguous_copy(w, kst, vst)
    k, v = dev.contiguous_copy(dw, w)
    k, v = dev.bf16_bits(k), dev.bf16_bits(v)
    assert k.shape[1] >= k_ref.shape[1]
    for s in range(w.num_seqs):
        L = int(w.context_lens[s])
        for h in range(w.num_kv_heads):
            r = s * w.num_kv_heads + h
            for t in range(L):
                assert np.array_equal(k[r, t // 16, :, t % 16, :], k_ref[r, t // 16, :, t % 16, :])
                assert np.array_equal(v[r, t // 16, (t % 16) // 4, :, t % 4],
                                      v_ref[r, t // 16, (t % 16) // 4, :, t % 4])


# -- prefix cache ---------------------------------------------------------------
def test_prefix_cache_page_example():
    """First Principles, section 9: two requests sharing a 32-token prefix share
    P0 and P1 (refcount 2); the rest is private; P1's hash chains P0's."""
    from paged_kv_cache_122_amd.prefix_cache import ROOT_HASH, PrefixCache, block_hash
    pool = BlockPool(16, 16)
    cache = PrefixCache(pool)
    prefix = list(range(1000, 1032))
    r1, hits1 = cache.allocate_prompt(prefix + list(range(20)))       # 52 tokens: 4 blocks
    r2, hits2 = cache.allocate_prompt(prefix + list(range(50, 60)))   # 42 tokens: 3 blocks
    assert (hits1, hits2) == (0, 2)
    assert r1.table[:2] == r2.table[:2] and len(r1.table) == 4 and len(r2.table) == 3
    assert set(r1.table[2:]).isdisjoint(r2.table[2:])
    assert [pool.ref[b] for b in r1.table] == [2, 2, 1, 1]
    h0 = block_hash(ROOT_HASH, prefix[:16])
    assert cache.hash_of[r1.table[1]] == block_hash(h0, prefix[16:])
    # the same 16 tokens after a different prefix are a different block
    assert block_hash(ROOT_HASH, prefix[16:]) != block_hash(h0, prefix[16:])
    assert pool.blocks_in_use() == 5


@pytest.mark.parametrize("B,shared_tokens", [(16, 992), (128, 896)])
def test_prefix_cache_system_prompt(B, shared_tokens):
    """sevydevy: 50 chats with the same 1,000-token system prompt; only full
    blocks are shared (62 of 16 tokens = 992 tokens, or 7 of 128 = 896), each
    chat keeps a private tail: 112 blocks instead of 3,150 at B = 16."""
    from paged_kv_cache_122_amd.prefix_cache import PrefixCache
    pool = BlockPool(4000, B)
    cache = PrefixCache(pool)
    prompt = [7 * i % 50021 for i in range(1000)]
    chats = [cache.allocate_prompt(prompt)[0] for _ in range(50)]
    n_full = shared_tokens // B
    assert pool.blocks_in_use() == n_full + 50
    if B == 16:
        assert pool.blocks_in_use() == 112 and 50 * len(chats[0].table) == 3150
    assert all(c.table[:n_full] == chats[0].table[:n_full] for c in chats)


def test_prefix_cache_salt_and_eviction():
    """A cache salt keeps tenants apart; a freed block stays findable until the
    pool reuses it (least recently freed first), then a lookup misses."""
    from paged_kv_cache_122_amd.prefix_cache import PrefixCache
    pool = BlockPool(6, 16)
    cache = PrefixCache(pool)
    toks = list(range(48))                                          # 3 full blocks
    a, _ = cache.allocate_prompt(toks, salt=b"tenant-a")
    b, hits = cache.allocate_prompt(toks, salt=b"tenant-b")
    assert hits == 0 and set(a.table).isdisjoint(b.table)
    a_blocks = list(a.table)
    free(pool, a)                                                   # refcounts 0, still registered
    c, hits = cache.allocate_prompt(toks, salt=b"tenant-a")
    assert hits == 3 and c.table == a_blocks and pool.num_free() == 0
    free(pool, c)
    free(pool, b)
    # reuse the whole pool: every block is handed out again and loses its hash
    d = Sequence()
    reserve_slots(pool, d, 16 * 6)
    free(pool, d)
    e, hits = cache.allocate_prompt(toks, salt=b"tenant-a")
    assert hits == 0 and pool.blocks_in_use() == 3
