"""The cache's state and its device-side contract.

* Checkpoint / resume: the pool, the block table and seq_lens are the whole
  state of a decode.  Saved to host files and loaded into fresh device
  buffers (elsewhere in memory, blocks renumbered), they must give bitwise
  the same decode, and the same pool after one more append.
* mla_check_block_table: finds planted out-of-range block ids and lengths,
  and reports nothing on a valid table.  (The decode itself is never run on
  a bad table: it would read outside the pool.)
"""

from __future__ import annotations

import os

import numpy as np
import pytest
import torch

from mla_latent_kv_06_amd import layout, synth
from tests import casebuild
from tests.casebuild import build_case

pytestmark = pytest.mark.gpu
W = synth.WORKLOADS


def announce(*what):
    print("[gpu-case]", *what, flush=True)


def G():
    from tests import gpu_util
    return gpu_util


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8"])
def test_save_restore_reproduces_decode_and_append_bitwise(cache_dtype, tmp_path):
    from mla_latent_kv_06_amd import binding as b
    wl = W["v3_b64_ctx1k8k_paged_bf16"].replace(name="v3_state", batch=3, ctx_lo=100, ctx_hi=400,
                                                cache_dtype=cache_dtype)
    announce("save/restore", cache_dtype)
    case = build_case(wl)
    dc = G().DeviceCase(case)
    dc.append()
    out1, lse1 = dc.decode(num_splits=0)
    torch.cuda.synchronize()
    # save: pool (+ scales), block table, lengths, to host files
    path = os.path.join(tmp_path, "state.npz")
    pool_np, scale_np = dc.pool_host()
    arrays = dict(pool=pool_np, table=dc.block_table.cpu().numpy(), lens=dc.seq_lens.cpu().numpy())
    if scale_np is not None:
        arrays["scale"] = scale_np
    np.savez(path, **arrays)
    # restore into fresh buffers: blocks in reverse order behind 3 spare blocks
    st = np.load(path)
    nblk = st["pool"].shape[0]
    perm = np.arange(nblk)[::-1] + 3                       # old block i -> new block perm[i]
    new_pool = np.zeros((nblk + 3,) + st["pool"].shape[1:], dtype=st["pool"].dtype)
    new_pool[perm] = st["pool"]
    table = st["table"].copy()
    table[table >= 0] = perm[table[table >= 0]]
    pool_d = torch.from_numpy(new_pool.view(np.int16) if cache_dtype == "bf16" else new_pool).to(G().DEV)
    if cache_dtype == "bf16":
        pool_d = pool_d.view(torch.bfloat16)
    scale_d = None
    if "scale" in st:
        sc = np.zeros((nblk + 3,) + st["scale"].shape[1:], dtype=np.float32)
        sc[perm] = st["scale"]
        scale_d = torch.from_numpy(sc).to(G().DEV)
    table_d = torch.from_numpy(table).to(G().DEV)
    lens_d = torch.from_numpy(st["lens"]).to(G().DEV)
    out2, lse2 = b.decode(dc.dims, dc.q_nope, dc.q_pe, dc.w_uk, dc.w_uv, pool_d, scale_d, table_d, lens_d,
                          num_splits=0)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1.view(torch.int32), lse2.view(torch.int32))
    # one more token on both states: the pools stay equal block for block.
    # (Checked on the host first: every sequence's next position lies in a
    # block its table already holds.)
    assert all(int(L) % wl.block_size != 0 for L in case.seq_lens)
    start = dc.seq_lens.clone()
    b.append(dc.dims, dc.h, dc.w_kv_a, dc.gamma, dc.block_table, start, dc.pool, dc.scale,
             rms_eps=casebuild.RMS_EPS, rope_base=casebuild.ROPE_BASE)
    b.append(dc.dims, dc.h, dc.w_kv_a, dc.gamma, table_d, start, pool_d, scale_d,
             rms_eps=casebuild.RMS_EPS, rope_base=casebuild.ROPE_BASE)
    torch.cuda.synchronize()
    old = dc.pool.view(torch.uint8).cpu().numpy()
    new = pool_d.view(torch.uint8).cpu().numpy()
    assert np.array_equal(new[perm], old)
    if scale_d is not None:
        assert np.array_equal(scale_d.cpu().numpy()[perm].view(np.int32), dc.scale.cpu().numpy().view(np.int32))


def test_check_block_table_reports_planted_violations():
    from mla_latent_kv_06_amd import binding as b
    wl = W["v3_b64_ctx1k8k_paged_bf16"].replace(name="v3_check", batch=5, ctx_lo=100, ctx_hi=900)
    announce("check_block_table")
    case = build_case(wl, fill=[])
    dims = b.Dims.from_workload(wl)
    table = torch.from_numpy(case.block_table).to(G().DEV)
    lens = torch.from_numpy(case.seq_lens).to(G().DEV)
    assert b.check_block_table(dims, table, lens, case.num_blocks) == (0, -1, -1)
    # a pool that ends just below the highest block id in use: that one entry is out of range
    used = [(bb, k) for bb in range(wl.batch) for k in range(case.block_table.shape[1])
            if k * 64 < case.seq_lens[bb]]
    top = max(int(case.block_table[bb, k]) for bb, k in used)
    hit = [(bb, k) for bb, k in used if case.block_table[bb, k] == top]
    assert b.check_block_table(dims, table, lens, top) == (1, hit[0][0], hit[0][1])
    # planted: a negative id, an id past the pool, a length past the table
    t2 = case.block_table.copy()
    t2[1, 0] = -5
    t2[3, 1] = 10 ** 6
    l2 = case.seq_lens.copy()
    l2[4] = case.block_table.shape[1] * 64 + 1
    n, fb, fk = b.check_block_table(dims, torch.from_numpy(t2).to(G().DEV), torch.from_numpy(l2).to(G().DEV),
                                    case.num_blocks)
    # the length also makes sequence 4's unused table entries (-1) count
    need4 = case.block_table.shape[1]
    used4 = (case.seq_lens[4] + 63) // 64
    assert (fb, fk) == (1, 0)
    assert n == 2 + 1 + (need4 - used4)
