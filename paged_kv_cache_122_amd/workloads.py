"""Seeded synthetic decode workloads: block pools, block tables, slot mappings
and bf16 values.

This module is the one thing both the HIP path and the fp64 oracle consume.  It
holds no attention arithmetic: it draws lengths and values, places blocks with
the host block manager, and poisons every slot a kernel must not read.

Recipe (all draws from one ``numpy.random.Generator(PCG64(seed))``, in this
order): context lengths -> a permutation of the pool that becomes the free-list
order (random block placement) -> q ``[S, Hq, D]`` -> this step's k ``[S, Hkv,
D]`` -> its v.  Pool values are drawn for the owned blocks only, in ascending
physical-id order, in chunks of ``max(1, 2**22 // (Hkv*B*D))`` blocks of
logical shape ``[Hkv, B, D]``; chunk ``c0`` (first owned index) of pool ``which`` (0 = K, 1 = V) uses its
own stream ``PCG64(SeedSequence([seed, which, c0]))``, so chunks can be drawn in
parallel and the result does not depend on the thread count.  Values are
N(0, 1) float32 rounded to bf16 (round-to-nearest-even).

Conventions: ``context_lens[s]`` counts this step's token, which the append
writes at position ``L - 1`` (slot ``slot_mapping[s]``; -1 when ``L == 0``).
Before the append, that position and every position ``>= L`` of the sequence's
blocks hold NaN, as does every block no sequence owns.  Unused block-table
entries hold -1.
"""

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

from . import layout
from .blockpool import BlockPool, Sequence, fork, free, reserve_slot, reserve_slots, slot_of_position
from .sizing import blocks_for_tokens, effective_kv_bytes

NAN_BF16 = 0x7FC0
_CHUNK_VALUES = 1 << 22        # values per generation chunk


def f32_to_bf16_bits(x):
    """float32 -> bf16 bit patterns, round-to-nearest-even (finite inputs)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.reshape(-1).view(np.uint32)
    out = np.empty(b.shape, dtype=np.uint16)
    step = 1 << 20                      # cache-sized chunks
    for i in range(0, b.size, step):
        c = b[i:i + step]
        t = (c >> np.uint32(16)) & np.uint32(1)
        t += np.uint32(0x7FFF)
        t += c
        t >>= np.uint32(16)
        out[i:i + step] = t
    return out.reshape(x.shape)


def _bf16_normal(rng, shape):
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


class BlockStore:
    """Owned blocks of a pool, indexable by physical block id (axis 0).

    Reading a block nobody owns raises: no correct reader ever touches one."""

    def __init__(self, owned, blocks, num_blocks):
        self.owned = np.asarray(owned, dtype=np.int64)
        self.blocks = blocks
        self.index = np.full(int(num_blocks), -1, dtype=np.int64)
        self.index[self.owned] = np.arange(len(self.owned))

    def __getitem__(self, b):
        idx = self.index[b]
        if np.any(np.asarray(idx) < 0):
            raise KeyError(f"physical block {b} is not owned by any sequence")
        return self.blocks[idx]

    def __len__(self):
        return len(self.index)


@dataclass
class Workload:
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    context_lens: np.ndarray      # int32 [S]
    block_tables: np.ndarray      # int32 [S, W], -1 padded
    slot_mapping: np.ndarray      # int64 [S]
    q: np.ndarray                 # uint16 [S, Hq, D]
    k_new: np.ndarray             # uint16 [S, Hkv, D]
    v_new: np.ndarray             # uint16 [S, Hkv, D]
    owned: np.ndarray             # int64 [n], ascending physical ids
    k_blocks: np.ndarray          # uint16 [n, Hkv, D/8, B, 8]
    v_blocks: np.ndarray          # uint16 [n, Hkv, B/4, D, 4]
    refcount: np.ndarray          # int32 [n]
    meta: dict = field(default_factory=dict)
    # copy-on-write copies this step performs before its append, int64 [N, 2]
    # (src, dst); every dst block holds NaN until the copy
    copies: np.ndarray = field(default_factory=lambda: np.zeros((0, 2), dtype=np.int64))
    # rows of q / k_new / v_new / slot_mapping per sequence, int32 [S + 1]: one
    # new token each unless a step brings several (chunked prefill,
    # speculative verification)
    query_start: np.ndarray = None

    @property
    def num_seqs(self):
        return int(self.context_lens.shape[0])

    @property
    def table_width(self):
        return int(self.block_tables.shape[1])

    def effective_kv_bytes(self):
        return effective_kv_bytes(self.context_lens, self.num_kv_heads, self.head_dim, 2)

    def unique_kv_bytes(self):
        """K + V bytes of distinct physical token slots read (shared blocks once)."""
        B = self.block_size
        seen = {}
        for s in range(self.num_seqs):
            L = int(self.context_lens[s])
            for i in range(blocks_for_tokens(L, B)):
                b = int(self.block_tables[s, i])
                seen[b] = max(seen.get(b, 0), min(B, L - i * B))
        return sum(seen.values()) * self.num_kv_heads * self.head_dim * 2 * 2

    def stores(self):
        """Fresh (writable) copies of the pre-append pools as BlockStores."""
        return (BlockStore(self.owned, self.k_blocks.copy(), self.num_blocks),
                BlockStore(self.owned, self.v_blocks.copy(), self.num_blocks))


def build_workload(name, seed, rng, *, num_q_heads, num_kv_heads, head_dim, block_size,
                   num_blocks, tables, context_lens, width, meta=None, copies=None, new_tokens=None):
    """Fill values for a placed workload.  ``tables`` are lists of physical ids
    covering ``ceil(L/B)`` blocks per sequence; ``rng`` continues the stream.
    ``copies`` are the pool's pending copy-on-write copies ``(src, dst, valid)``
    of this step: ``src`` holds ``valid`` tokens, ``dst`` holds NaN until copied.
    ``new_tokens[s]`` (default 1) of the ``L`` tokens of sequence ``s`` arrive
    this step: the pool holds the first ``L - new_tokens[s]``."""
    S = len(context_lens)
    Hq, Hkv, D, B = int(num_q_heads), int(num_kv_heads), int(head_dim), int(block_size)
    if Hq % Hkv or D not in layout.SUPPORTED_HEAD_DIMS or B not in layout.SUPPORTED_BLOCK_SIZES:
        raise ValueError("unsupported head / block geometry")
    lens = np.asarray(context_lens, dtype=np.int32)
    news = np.ones(S, dtype=np.int64) if new_tokens is None else np.asarray(new_tokens, dtype=np.int64)
    if np.any(news < 0) or np.any(news > np.maximum(lens, 1)):
        raise ValueError("new tokens must lie inside the context")
    qstart = np.zeros(S + 1, dtype=np.int32)
    qstart[1:] = np.cumsum(news)
    T = int(qstart[-1])
    bt = np.full((S, int(width)), -1, dtype=np.int32)
    slots = np.full(T, -1, dtype=np.int64)
    valid_before = {}
    users = {}
    for s in range(S):
        L = int(lens[s])
        n = int(news[s])
        t = list(tables[s])
        if len(t) != blocks_for_tokens(L, B) or len(t) > width:
            raise ValueError("block table does not match context length")
        bt[s, :len(t)] = t
        if L > 0:
            for i in range(n):
                slots[qstart[s] + i] = slot_of_position(t, L - n + i, B)
        for i, b in enumerate(t):
            n_prev = min(B, max(0, (L - n) - i * B))
            valid_before[b] = max(valid_before.get(b, 0), n_prev)
            users[b] = users.get(b, 0) + 1
    copies = [tuple(int(x) for x in c) for c in (copies or [])]
    for src, _dst, valid in copies:
        valid_before[src] = max(valid_before.get(src, 0), valid)
        users.setdefault(src, 0)

    q = _bf16_normal(rng, (T, Hq, D))
    k_new = _bf16_normal(rng, (T, Hkv, D))
    v_new = _bf16_normal(rng, (T, Hkv, D))

    owned = np.array(sorted(valid_before), dtype=np.int64)
    n = len(owned)
    fill = np.array([valid_before[int(b)] for b in owned], dtype=np.int64)
    k_blocks = np.empty((n,) + layout.k_cache_shape(1, Hkv, D, B)[1:], dtype=np.uint16)
    v_blocks = np.empty((n,) + layout.v_cache_shape(1, Hkv, D, B)[1:], dtype=np.uint16)

    chunk = max(1, _CHUNK_VALUES // (Hkv * B * D))

    def fill_chunk(which, c0):
        c1 = min(n, c0 + chunk)
        crng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, which, c0])))
        vals = _bf16_normal(crng, (c1 - c0, Hkv, B, D))
        for r in np.nonzero(fill[c0:c1] < B)[0]:               # partly filled blocks only
            vals[r, :, fill[c0 + r]:, :] = NAN_BF16
        if which == 0:
            k_blocks[c0:c1] = layout.pack_k(vals)
        else:
            v_blocks[c0:c1] = layout.pack_v(vals)

    jobs = [(which, c0) for which in (0, 1) for c0 in range(0, n, chunk)]
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(lambda j: fill_chunk(*j), jobs))
    pools = [k_blocks, v_blocks]
    pos = {int(b): i for i, b in enumerate(owned)}
    for _src, dst, _valid in copies:  # not yet copied: poison
        k_blocks[pos[dst]] = NAN_BF16
        v_blocks[pos[dst]] = NAN_BF16

    return Workload(
        name=name, seed=int(seed), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=B,
        num_blocks=int(num_blocks), scale=1.0 / float(np.sqrt(D)), context_lens=lens,
        block_tables=bt, slot_mapping=slots, q=q, k_new=k_new, v_new=v_new, owned=owned,
        k_blocks=pools[0], v_blocks=pools[1],
        refcount=np.array([users[int(b)] for b in owned], dtype=np.int32), meta=dict(meta or {}),
        copies=np.array([(c[0], c[1]) for c in copies], dtype=np.int64).reshape(-1, 2),
        query_start=qstart)


def place_independent(rng, context_lens, block_size, num_blocks):
    """Random placement: the free list is a seeded permutation of the pool and
    every sequence takes its blocks on demand, one token at a time."""
    pool = BlockPool(num_blocks, block_size, free_order=rng.permutation(int(num_blocks)))
    tables = []
    for L in context_lens:
        seq = Sequence()
        reserve_slots(pool, seq, int(L))
        tables.append(seq.table)
    return pool, tables


def random_workload(seed, context_lens, *, num_q_heads, num_kv_heads, head_dim, block_size,
                    num_blocks=None, width=None, name="random"):
    """Independent sequences with the given lengths; pool = needed + 10 % unless given."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = [int(x) for x in context_lens]
    need = sum(blocks_for_tokens(L, block_size) for L in lens)
    if num_blocks is None:
        num_blocks = max(1, int(np.ceil(1.1 * need)))
    if width is None:
        width = max(1, max(blocks_for_tokens(L, block_size) for L in lens))
    _, tables = place_independent(rng, lens, block_size, num_blocks)
    return build_workload(name, seed, rng, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                          head_dim=head_dim, block_size=block_size, num_blocks=num_blocks,
                          tables=tables, context_lens=lens, width=width)


# ---------------------------------------------------------------------------
# the five named configurations
# ---------------------------------------------------------------------------
def tiny_gqa():
    """4 seqs, L = {1, 17, 100, 900}, 8 q / 2 kv heads, D 64, B 16, pool 128."""
    seed = 1001
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = [1, 17, 100, 900]
    _, tables = place_independent(rng, lens, 16, 128)
    return build_workload("tiny_gqa4_d64", seed, rng, num_q_heads=8, num_kv_heads=2, head_dim=64,
                          block_size=16, num_blocks=128, tables=tables, context_lens=lens,
                          width=blocks_for_tokens(900, 16))


def llama3_8b_layer():
    """64 seqs, 32 q / 8 kv heads, D 128, B 16, L ~ U[128, 2048], pool needed + 10 %."""
    seed = 1002
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(128, 2048, size=64, endpoint=True).tolist()
    need = sum(blocks_for_tokens(L, 16) for L in lens)
    nb = int(np.ceil(1.1 * need))
    _, tables = place_independent(rng, lens, 16, nb)
    return build_workload("llama3_8b_b64", seed, rng, num_q_heads=32, num_kv_heads=8,
                          head_dim=128, block_size=16, num_blocks=nb, tables=tables,
                          context_lens=lens, width=2048 // 16)


def llama3_70b_layer():
    """256 seqs, 64 q / 8 kv heads, D 128, B 16, L = clip(rint(600 e^Z), 16, 8192),
    blocks scattered over a 200,000-block pool."""
    seed = 1003
    rng = np.random.Generator(np.random.PCG64(seed))
    z = rng.standard_normal(256)
    lens = np.clip(np.rint(600.0 * np.exp(z)), 16, 8192).astype(np.int64).tolist()
    _, tables = place_independent(rng, lens, 16, 200_000)
    return build_workload("llama3_70b_b256", seed, rng, num_q_heads=64, num_kv_heads=8,
                          head_dim=128, block_size=16, num_blocks=200_000, tables=tables,
                          context_lens=lens, width=8192 // 16)


def opt13b_prefix_sharing():
    """128 seqs in 16 groups of 8; each group shares a 1,024-token prompt (64 full
    blocks, refcount 8) and each seq has a private tail of U[16, 1024] tokens.
    40 q = 40 kv heads, D 128, B 16, pool needed + 10 %."""
    seed = 1004
    B, prompt, groups, per = 16, 1024, 16, 8
    rng = np.random.Generator(np.random.PCG64(seed))
    tails = rng.integers(16, 1024, size=groups * per, endpoint=True).tolist()
    need = groups * blocks_for_tokens(prompt, B) + sum(blocks_for_tokens(t, B) for t in tails)
    nb = int(np.ceil(1.1 * need))
    pool = BlockPool(nb, B, free_order=rng.permutation(nb))
    tables, lens = [], []
    for g in range(groups):
        parent = Sequence()
        reserve_slots(pool, parent, prompt)
        children = [fork(pool, parent) for _ in range(per)]
        free(pool, parent)
        for j, child in enumerate(children):
            reserve_slots(pool, child, tails[g * per + j])
            tables.append(child.table)
            lens.append(child.length)
    if pool.pending_copies:
        raise AssertionError("a 1,024-token prompt fills whole blocks: no copy-on-write expected")
    return build_workload("opt13b_mha_prefix_b128", seed, rng, num_q_heads=40, num_kv_heads=40,
                          head_dim=128, block_size=B, num_blocks=nb, tables=tables,
                          context_lens=lens, width=(prompt + 1024) // B,
                          meta={"groups": groups, "per_group": per, "shared_blocks": prompt // B})


def opt13b_cow_fork():
    """Parallel sampling right after the prompt: 16 prompts of 1,000 tokens (62
    full blocks and a last block holding 8 of 16 tokens), each forked into 8
    samples that share every block.  This step each sample appends its first
    token; the shared last block is copied for every sample but the last
    writer, which by then holds its only reference (7 copies per prompt).
    40 q = 40 kv heads, D 128, B 16, pool needed + 10 %."""
    seed = 1008
    B, prompt, groups, per = 16, 1000, 16, 8
    rng = np.random.Generator(np.random.PCG64(seed))
    need = groups * (blocks_for_tokens(prompt, B) + per - 1)
    nb = int(np.ceil(1.1 * need))
    pool = BlockPool(nb, B, free_order=rng.permutation(nb))
    tables, lens = [], []
    for _ in range(groups):
        parent = Sequence()
        reserve_slots(pool, parent, prompt)
        children = [fork(pool, parent) for _ in range(per)]
        free(pool, parent)
        for child in children:
            reserve_slot(pool, child)  # this step's token
            tables.append(child.table)
            lens.append(child.length)
    copies = list(pool.pending_copies)
    if len(copies) != groups * (per - 1):
        raise AssertionError("every sample but the last writer copies the shared block")
    return build_workload("opt13b_cow_fork_b128", seed, rng, num_q_heads=40, num_kv_heads=40,
                          head_dim=128, block_size=B, num_blocks=nb, tables=tables,
                          context_lens=lens, width=blocks_for_tokens(prompt + 1, B),
                          meta={"groups": groups, "per_group": per}, copies=copies)


def multi_query_workload(seed, old_lens, new_counts, *, num_q_heads, num_kv_heads, head_dim,
                         block_size, name="multi_query", width=None):
    """Sequences with ``old_lens[s]`` cached tokens and ``new_counts[s]`` tokens
    arriving this step (context ``old + new``); random placement, pool needed
    + 10 %."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B = int(block_size)
    lens = [int(o) + int(n) for o, n in zip(old_lens, new_counts)]
    need = sum(blocks_for_tokens(L, B) for L in lens)
    nb = max(1, int(np.ceil(1.1 * need)))
    _, tables = place_independent(rng, lens, B, nb)
    width = width or max(1, max(blocks_for_tokens(L, B) for L in lens))
    return build_workload(name, seed, rng, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                          head_dim=head_dim, block_size=B, num_blocks=nb, tables=tables,
                          context_lens=lens, width=width, new_tokens=list(new_counts))


def llama3_8b_verify5():
    """Speculative verification on the Llama-3-8B-shaped batch: 64 seqs with
    U[128, 2048] cached tokens, each verifying 5 drafted tokens this step
    (32 q / 8 kv heads, D 128, B 16)."""
    seed = 1009
    rng = np.random.Generator(np.random.PCG64(seed))
    old = rng.integers(128, 2048, size=64, endpoint=True).tolist()
    return multi_query_workload(seed, old, [5] * 64, num_q_heads=32, num_kv_heads=8, head_dim=128,
                                block_size=16, name="llama3_8b_verify5_b64",
                                width=blocks_for_tokens(2048 + 5, 16))


def long32k_verify5():
    """Speculative verification over long contexts: 8 seqs x 32,763 cached tokens,
    each verifying 5 drafted tokens (32 q / 8 kv heads, D 128, B 16)."""
    seed = 1010
    return multi_query_workload(seed, [32768 - 5] * 8, [5] * 8, num_q_heads=32, num_kv_heads=8, head_dim=128,
                                block_size=16, name="long32k_verify5_b16")


def long_context(block_size):
    """8 seqs x 32,768 tokens, 32 q / 8 kv heads, D 128, B in {8, 16, 32},
    random placement, pool needed + 10 %."""
    seed = {8: 1005, 16: 1006, 32: 1007}[int(block_size)]
    B = int(block_size)
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = [32768] * 8
    need = 8 * (32768 // B)
    nb = int(np.ceil(1.1 * need))
    _, tables = place_independent(rng, lens, B, nb)
    return build_workload(f"long32k_b{B}", seed, rng, num_q_heads=32, num_kv_heads=8,
                          head_dim=128, block_size=B, num_blocks=nb, tables=tables,
                          context_lens=lens, width=32768 // B)


CONFIGS = {
    "tiny_gqa4_d64": tiny_gqa,
    "llama3_8b_b64": llama3_8b_layer,
    "llama3_70b_b256": llama3_70b_layer,
    "opt13b_mha_prefix_b128": opt13b_prefix_sharing,
    "long32k_b8": lambda: long_context(8),
    "long32k_b16": lambda: long_context(16),
    "long32k_b32": lambda: long_context(32),
    "opt13b_cow_fork_b128": opt13b_cow_fork,
    "llama3_8b_verify5_b64": llama3_8b_verify5,
    "long32k_verify5_b16": long32k_verify5,
}


def make(name):
    return CONFIGS[name]()
