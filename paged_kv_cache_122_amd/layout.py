"""Physical layout of the paged K/V pools, and logical <-> packed conversion.

The pages agree that the cache is a per-layer pool of fixed-size blocks indexed
by physical block id ("PagedAttention from First Principles", section 5) but
give three incompatible element orders inside a block (section 5's vLLM shapes
and pseudocode shapes, the hungchun0201 digest's kernel sketch, section 7's
prose).  This library fixes its own, chosen so that one (block, kv-head) tile is
a single contiguous ``B * D * 2``-byte chunk and so that a 64-lane wavefront
reads it with 16-byte loads that are already in MFMA operand order:

* K pool ``[num_blocks, num_kv_heads, D/8, B, 8]``: token ``t``, dim ``d`` of a
  block at ``[h, d // 8, t, d % 8]`` -- 8-dim groups, token-minor, so 16 lanes
  holding 16 consecutive tokens of one 8-dim group read 256 contiguous bytes.
* V pool ``[num_blocks, num_kv_heads, B/4, D, 4]``: token ``t``, dim ``d`` at
  ``[h, t // 4, d, t % 4]`` -- 4-token groups, dim-major, so a lane holding two
  adjacent dims of 4 consecutive tokens reads 16 contiguous bytes and 16 lanes
  read 256 contiguous bytes.

``pack_*`` / ``unpack_*`` convert between the logical block view
``[..., num_kv_heads, B, D]`` and these layouts; they work on numpy arrays and
on torch tensors (views where possible, no arithmetic on values).
"""

SUPPORTED_HEAD_DIMS = (64, 128)
SUPPORTED_BLOCK_SIZES = (8, 16, 32)


def k_cache_shape(num_blocks, num_kv_heads, head_dim, block_size):
    return (int(num_blocks), int(num_kv_heads), int(head_dim) // 8, int(block_size), 8)


def v_cache_shape(num_blocks, num_kv_heads, head_dim, block_size):
    return (int(num_blocks), int(num_kv_heads), int(block_size) // 4, int(head_dim), 4)


def _permute(x, order):
    if hasattr(x, "permute"):
        return x.permute(*order)
    return x.transpose(order)


def _contig(x):
    if hasattr(x, "contiguous"):
        return x.contiguous()
    import numpy as np

    return np.ascontiguousarray(x)


def pack_k(k_logical):
    """[..., H, B, D] -> [..., H, D/8, B, 8]"""
    *lead, H, B, D = k_logical.shape
    n = len(lead)
    x = k_logical.reshape(*lead, H, B, D // 8, 8)
    order = list(range(n)) + [n, n + 2, n + 1, n + 3]
    return _contig(_permute(x, order))


def unpack_k(k_packed):
    """[..., H, D/8, B, 8] -> [..., H, B, D]"""
    *lead, H, D8, B, _ = k_packed.shape
    n = len(lead)
    order = list(range(n)) + [n, n + 2, n + 1, n + 3]
    return _contig(_permute(k_packed, order)).reshape(*lead, H, B, D8 * 8)


def pack_v(v_logical):
    """[..., H, B, D] -> [..., H, B/4, D, 4]"""
    *lead, H, B, D = v_logical.shape
    n = len(lead)
    x = v_logical.reshape(*lead, H, B // 4, 4, D)
    order = list(range(n)) + [n, n + 1, n + 3, n + 2]
    return _contig(_permute(x, order))


def unpack_v(v_packed):
    """[..., H, B/4, D, 4] -> [..., H, B, D]"""
    *lead, H, B4, D, _ = v_packed.shape
    n = len(lead)
    order = list(range(n)) + [n, n + 1, n + 3, n + 2]
    return _contig(_permute(v_packed, order)).reshape(*lead, H, B4 * 4, D)
