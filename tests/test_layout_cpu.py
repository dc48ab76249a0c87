"""The host-side pool views (``mla_latent_kv_06_amd.layout``) against the block
layout include/mla.h states for cache_pool, element by element with plain
loops: every cache dtype is token-major -- element (token t, channel c) of a
block at t * D + c.  The GPU tests feed the oracle through these views, so
they are pinned here against the stated formula rather than against
themselves."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from mla_latent_kv_06_amd import layout


def stated_offset(t, c, D):
    return t * D + c


@pytest.mark.parametrize("bs,D,dtype", [(64, 7, "bf16"), (96, 5, "bf16"), (48, 3, "bf16"),
                                        (16, 9, "bf16"), (64, 6, "fp8"), (32, 4, "f32")])
def test_pool_rows_follows_the_stated_layout(bs, D, dtype):
    nblk = 3
    rng = np.random.default_rng(7)
    pool = rng.integers(0, 60000, size=(nblk, bs, D)).astype(np.uint16)
    flat = pool.reshape(nblk, bs * D)
    want = np.empty((nblk * bs, D), np.uint16)
    for blk in range(nblk):
        for t in range(bs):
            for c in range(D):
                want[blk * bs + t, c] = flat[blk, stated_offset(t, c, D)]
    got = layout.pool_rows(pool, dtype)
    assert np.array_equal(got, want)
    # torch tensors take the same path
    assert np.array_equal(layout.pool_rows(torch.from_numpy(pool.astype(np.int32)), dtype).numpy(),
                          want.astype(np.int32))
    # and rows_to_pool is its inverse, for numpy and torch
    back = layout.rows_to_pool(want, bs, dtype)
    assert back.shape == pool.shape and np.array_equal(back, pool)
    back_t = layout.rows_to_pool(torch.from_numpy(want.astype(np.int32)), bs, dtype)
    assert np.array_equal(back_t.numpy(), pool.astype(np.int32))


def test_planted_transpose_is_caught():
    """A channel-major reading of a block differs from the stated layout, so
    the element-by-element check above would catch a transposed view."""
    bs, D = 64, 5
    pool = np.arange(2 * bs * D, dtype=np.uint16).reshape(2, bs, D)
    transposed = pool.reshape(2, D, bs).transpose(0, 2, 1).reshape(-1, D)
    assert not np.array_equal(layout.pool_rows(pool, "bf16"), transposed)
