"""Device-side plumbing with torch: pool allocation in the library's layout
and upload of a seeded workload.  No arithmetic on values."""

from dataclasses import dataclass

import numpy as np
import torch

from . import layout


def bf16_tensor(bits, device):
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 tensor on ``device``."""
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).view(torch.bfloat16).to(device)


def bf16_bits(t):
    """torch bf16 tensor -> uint16 numpy bit patterns (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def alloc_pools(num_blocks, num_kv_heads, head_dim, block_size, device, fill=float("nan")):
    """K and V pools in the library layout, every element set to ``fill``."""
    k = torch.full(layout.k_cache_shape(num_blocks, num_kv_heads, head_dim, block_size), fill,
                   dtype=torch.bfloat16, device=device)
    v = torch.full(layout.v_cache_shape(num_blocks, num_kv_heads, head_dim, block_size), fill,
                   dtype=torch.bfloat16, device=device)
    return k, v


@dataclass
class DeviceWorkload:
    q: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    slot_mapping: torch.Tensor
    block_tables: torch.Tensor
    context_lens: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    owned: torch.Tensor
    copies: torch.Tensor   # int64 [N, 2] copy-on-write (src, dst) of this step
    query_start: torch.Tensor = None  # int32 [S + 1] rows of q / k_new / v_new per sequence


def upload(w, device="cuda"):
    """Copy a workloads.Workload to the GPU: unowned pool blocks hold NaN."""
    k_cache, v_cache = alloc_pools(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size, device)
    owned = torch.from_numpy(w.owned).to(device)
    if len(w.owned):
        k_cache[owned] = bf16_tensor(w.k_blocks, device)
        v_cache[owned] = bf16_tensor(w.v_blocks, device)
    return DeviceWorkload(
        q=bf16_tensor(w.q, device), k_new=bf16_tensor(w.k_new, device),
        v_new=bf16_tensor(w.v_new, device),
        slot_mapping=torch.from_numpy(w.slot_mapping).to(device),
        block_tables=torch.from_numpy(w.block_tables).to(device),
        context_lens=torch.from_numpy(w.context_lens).to(device),
        k_cache=k_cache, v_cache=v_cache, owned=owned,
        copies=torch.from_numpy(np.ascontiguousarray(w.copies, dtype=np.int64)).to(device),
        query_start=torch.from_numpy(np.ascontiguousarray(w.query_start, dtype=np.int32)).to(device))


def contiguous_copy(dw, w):
    """The pools of a device workload without paging, for pa_decode_contiguous:
    (sequence, KV head) region s*Hkv + h holds that sequence's tokens in logical
    order as a run of 16-token tiles (K [S*Hkv, T, D/8, 16, 8], V [S*Hkv, T, 4,
    D, 4], T = table width * B / 16 rounded up).  A gather of whole blocks
    through the tables; sentinel entries read block 0, whose tokens lie past
    the context and are never used."""
    S, W, B = w.num_seqs, w.table_width, w.block_size
    Hkv, D = w.num_kv_heads, w.head_dim
    bt = dw.block_tables[:, :W].long().clamp(min=0)
    if B == 8 and W % 2:                                   # whole 16-token tiles
        bt = torch.nn.functional.pad(bt, (0, 1))
        W += 1
    k = dw.k_cache[bt].permute(0, 2, 1, 3, 4, 5)         # [S, Hkv, W, D/8, B, 8]
    v = dw.v_cache[bt].permute(0, 2, 1, 3, 4, 5)         # [S, Hkv, W, B/4, D, 4]
    if B == 32:   # two tiles per block
        k = k.reshape(S, Hkv, W, D // 8, 2, 16, 8).permute(0, 1, 2, 4, 3, 5, 6)
    elif B == 8:  # two blocks per tile
        k = k.reshape(S, Hkv, W // 2, 2, D // 8, 8, 8).permute(0, 1, 2, 4, 3, 5, 6)
    T = W * B // 16
    k = k.reshape(S * Hkv, T, D // 8, 16, 8)
    v = v.reshape(S * Hkv, T, 4, D, 4)
    return k.contiguous(), v.contiguous()
