"""GPU check of mla_decode_absorbed_noalloc (the decode on the library's static
scratch, for callers that cannot allocate) against mla_decode_absorbed with a
caller workspace: the same kernels on the same inputs, so the outputs must be
bitwise equal.  Two calls in a row, the second with a smaller batch, so that
the second runs on scratch the first left behind; each result is also held to
the oracle's bf16 bars."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from mla_latent_kv_06_amd import synth
from tests.casebuild import build_case, error_stats

pytestmark = pytest.mark.gpu

MID = synth.WORKLOADS["v3_b64_ctx1k8k_paged_bf16"].replace(
    name="v3_noalloc", batch=6, ctx_lo=40, ctx_hi=700, append=False)


@pytest.mark.parametrize("splits", [0, 3])
def test_noalloc_matches_workspace_decode_twice(splits):
    from mla_latent_kv_06_amd import binding as b
    from tests import gpu_util
    for batch in (6, 2):
        wl = MID.replace(batch=batch)
        print("[gpu-case] noalloc batch", batch, "splits", splits, flush=True)
        case = build_case(wl, seed=batch)
        dc = gpu_util.DeviceCase(case)
        ref_out, ref_lse = dc.decode(num_splits=splits)
        out = torch.full_like(ref_out, float("nan"))
        lse = torch.full_like(ref_lse, float("nan"))
        b.decode_noalloc(dc.dims, dc.q_nope, dc.q_pe, dc.w_uk, dc.w_uv, dc.pool, dc.scale,
                         dc.block_table, dc.seq_lens, out, lse, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        assert torch.equal(lse, ref_lse)
        ref, ref_l = case.oracle_decode()
        got = gpu_util.to_np(out)
        max_abs, rel = error_stats(got, ref)
        print(f"noalloc batch {batch}: max-abs {max_abs:.3e} rel-L2 {rel:.3e}", flush=True)
        assert max_abs <= 2e-2 and rel <= 5e-3
        assert np.max(np.abs(gpu_util.to_np(lse) - ref_l)) <= 1e-2


def test_noalloc_rejects_oversized_calls():
    from mla_latent_kv_06_amd import binding as b
    wl = MID.replace(batch=130)
    dims = b.Dims.from_workload(wl)
    dev = torch.device("cuda:0")
    z = lambda *s, dt=torch.bfloat16: torch.zeros(*s, dtype=dt, device=dev)
    with pytest.raises(b.MLAError) as e:
        b.decode_noalloc(dims, z(130, 1, 128, 128), z(130, 1, 128, 64), z(128, 128, 512),
                         z(128, 128, 512), z(1, 64, 576), None, z(130, 1, dt=torch.int32),
                         z(130, dt=torch.int32), z(130, 1, 128, 128))
    assert "WORKSPACE_TOO_SMALL" in str(e.value)
