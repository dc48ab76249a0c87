"""Device-side helpers for the GPU tests: upload a host case, call the library
through the binding, read results back."""

from __future__ import annotations

import numpy as np
import torch

from tests import casebuild

DEV = torch.device("cuda:0")


def binding():
    from mla_latent_kv_06_amd import binding as b
    return b


def up_act(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def up_pool(case: casebuild.Case):
    pool = case.pool
    if case.wl.cache_dtype == "bf16":
        t = torch.from_numpy(pool.view(np.int16)).view(torch.bfloat16).to(DEV)
    elif case.wl.cache_dtype == "fp8":
        t = torch.from_numpy(pool).to(DEV)
    else:
        t = torch.from_numpy(pool).to(DEV)
    sc = None if case.scale is None else torch.from_numpy(case.scale).to(DEV)
    return t, sc


def down_pool(t: torch.Tensor, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class DeviceCase:
    """A case's tensors on the GPU."""

    def __init__(self, case: casebuild.Case):
        b = binding()
        wl = case.wl
        self.case = case
        self.dims = b.Dims.from_workload(wl)
        self.q_nope = up_act(case.q_nope, wl.act_dtype)
        self.q_pe = up_act(case.q_pe, wl.act_dtype)
        self.w_uk = up_act(case.w_uk, wl.act_dtype)
        self.w_uv = up_act(case.w_uv, wl.act_dtype)
        self.pool, self.scale = up_pool(case)
        self.block_table = torch.from_numpy(case.block_table).to(DEV)
        self.seq_lens = torch.from_numpy(case.seq_lens).to(DEV)
        if case.h is not None:
            self.h = up_act(case.h, wl.act_dtype)
            self.w_kv_a = up_act(case.w_kv_a, wl.act_dtype)
            self.gamma = up_act(case.gamma, wl.act_dtype)
            self.start_pos = torch.from_numpy(case.cached.astype(np.int32)).to(DEV)

    def decode(self, num_splits=None, stages=None, workspace=None, out=None, lse=None):
        b = binding()
        ns = self.case.wl.num_splits if num_splits is None else num_splits
        kw = {} if stages is None else {"stages": stages}
        return b.decode(self.dims, self.q_nope, self.q_pe, self.w_uk, self.w_uv, self.pool,
                        self.scale, self.block_table, self.seq_lens, num_splits=ns,
                        workspace=workspace, out=out, lse=lse, **kw)

    def append(self):
        b = binding()
        b.append(self.dims, self.h, self.w_kv_a, self.gamma, self.block_table, self.start_pos,
                 self.pool, self.scale, rms_eps=casebuild.RMS_EPS, rope_base=casebuild.ROPE_BASE)

    def pool_host(self):
        torch.cuda.synchronize()
        p = down_pool(self.pool, self.case.wl.cache_dtype)
        s = None if self.scale is None else self.scale.cpu().numpy()
        return p, s


def to_np(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.float().cpu().numpy().astype(np.float64)
