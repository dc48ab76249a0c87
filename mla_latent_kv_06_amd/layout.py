"""Host-side views of the paged cache layout (include/mla.h, cache_pool).

A pool is [num_blocks][block_size][row_width] elements, token-major for every
cache dtype: row t of a block is token t, and element (token t, channel c) of
a block sits at t * row_width + c.

``pool_rows`` turns a pool (numpy array or torch tensor) into token rows
[num_blocks * block_size, row_width]; ``rows_to_pool`` is its inverse.  Both
only move elements.
"""

from __future__ import annotations


def pool_rows(pool, cache_dtype=None):
    """Token rows [num_blocks * block_size, row_width] of a pool (any dtype)."""
    nblk, bs, D = pool.shape
    return pool.reshape(nblk * bs, D)


def rows_to_pool(rows, block_size: int, cache_dtype=None):
    """A pool [num_blocks, block_size, row_width] holding the given token rows."""
    n, D = rows.shape
    return rows.reshape(n // block_size, block_size, D)
