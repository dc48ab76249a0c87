"""Host-side views of the paged cache layout (include/mla.h, cache_pool).

A pool is [num_blocks][block_size][row_width] elements.  fp8 and fp32 pools
are token-major (row t of a block is token t).  bf16 pools store each block
as sub-blocks of 32 tokens (the whole block when block_size is not a
multiple of 32), each channel-major: element (token t, channel c) of a block
sits at ((t // sub) * row_width + c) * sub + t % sub.

``pool_rows`` turns a pool (numpy array or torch tensor) into token rows
[num_blocks * block_size, row_width]; ``rows_to_pool`` is its inverse.  Both
only move elements.
"""

from __future__ import annotations

SUB = 32


def sub_block(block_size: int) -> int:
    return SUB if block_size % SUB == 0 else block_size


def _is_channel_major(cache_dtype) -> bool:
    return cache_dtype in ("bf16", 1)


def pool_rows(pool, cache_dtype):
    """Token rows [num_blocks * block_size, row_width] of a pool."""
    nblk, bs, D = pool.shape
    if not _is_channel_major(cache_dtype):
        return pool.reshape(nblk * bs, D)
    sub = sub_block(bs)
    x = pool.reshape(nblk, bs // sub, D, sub)
    x = x.permute(0, 1, 3, 2) if hasattr(x, "permute") else x.transpose(0, 1, 3, 2)
    return x.reshape(nblk * bs, D)


def rows_to_pool(rows, block_size: int, cache_dtype):
    """A pool [num_blocks, block_size, row_width] holding the given token rows."""
    n, D = rows.shape
    nblk = n // block_size
    if not _is_channel_major(cache_dtype):
        return rows.reshape(nblk, block_size, D)
    sub = sub_block(block_size)
    x = rows.reshape(nblk, block_size // sub, sub, D)
    if hasattr(x, "permute"):
        return x.permute(0, 1, 3, 2).contiguous().reshape(nblk, block_size, D)
    import numpy as np
    return np.ascontiguousarray(x.transpose(0, 1, 3, 2)).reshape(nblk, block_size, D)
