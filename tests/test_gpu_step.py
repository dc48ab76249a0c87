"""GPU checks of mla_decode_step: the step's cache append followed by the
absorbed decode in one call must give, bit for bit, what mla_cache_append
then mla_decode_absorbed give on the same inputs -- the output, the lse and
every byte of the pool -- and the oracle's result within the decode's bars.

Cases: bf16 cache with one query row (balanced schedule and a fixed split
count), fp8 cache with two query rows, and the portable kernels (a small
head shape with f32 activations), where the finalize and the absorption are
not fused.  The stages run one at a time compose to the full call.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from mla_latent_kv_06_amd import synth
from tests import casebuild
from tests.casebuild import build_case, error_stats

pytestmark = pytest.mark.gpu
W = synth.WORKLOADS


def announce(*what):
    print("[gpu-case]", *what, flush=True)


def G():
    from tests import gpu_util
    return gpu_util


def two_copies(case):
    """Two independent device copies of the case (pool included)."""
    return G().DeviceCase(case), G().DeviceCase(case)


def step(dc, num_splits, stages=None):
    from mla_latent_kv_06_amd import binding as b
    kw = {} if stages is None else {"stages": stages}
    return b.decode_step(dc.dims, dc.h, dc.w_kv_a, dc.gamma, dc.start_pos, dc.q_nope, dc.q_pe,
                         dc.w_uk, dc.w_uv, dc.pool, dc.scale, dc.block_table, dc.seq_lens,
                         num_splits=num_splits, rms_eps=casebuild.RMS_EPS,
                         rope_base=casebuild.ROPE_BASE, **kw)


def assert_same(ref_dc, ref_out, ref_lse, dc, out, lse, tag):
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                       ref_out.view(torch.int16) if ref_out.dtype == torch.bfloat16 else ref_out), tag
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), tag
    assert torch.equal(dc.pool.view(torch.uint8), ref_dc.pool.view(torch.uint8)), tag
    if dc.scale is not None:
        assert torch.equal(dc.scale.view(torch.int32), ref_dc.scale.view(torch.int32)), tag


CASES = {
    "bf16_q1": W["v3_b64_ctx1k8k_paged_bf16"].replace(name="v3_step_bf16", batch=5, ctx_lo=40,
                                                      ctx_hi=700),
    "fp8_q2": W["v3_b64_ctx1k8k_paged_bf16"].replace(name="v3_step_fp8", batch=4, ctx_lo=1,
                                                     ctx_hi=500, cache_dtype="fp8", q_len=2),
}


@pytest.mark.parametrize("name,splits", [("bf16_q1", 0), ("bf16_q1", 3), ("fp8_q2", 0)])
def test_step_equals_append_then_decode(name, splits):
    wl = CASES[name]
    announce("decode_step", wl.name, "q_len", wl.q_len, "splits", splits)
    case = build_case(wl)
    ref, dc = two_copies(case)
    ref.append()
    ref_out, ref_lse = ref.decode(num_splits=splits)
    out, lse = step(dc, splits)
    assert_same(ref, ref_out, ref_lse, dc, out, lse, f"{name} splits={splits}")
    # and the oracle, on the pool the step left
    after, after_scale = dc.pool_host()
    o_ref, l_ref = case.oracle_decode(pool=after, scale=after_scale)
    got = G().to_np(out)
    max_abs, rel = error_stats(got, o_ref)
    vis = np.isfinite(l_ref)
    d_lse = float(np.max(np.abs(G().to_np(lse)[vis] - l_ref[vis])))
    print(f"decode_step {name} splits={splits}: max-abs {max_abs:.3e} rel-L2 {rel:.3e} lse {d_lse:.3e}",
          flush=True)
    bar = 6e-2 if wl.cache_dtype == "fp8" else 2e-2
    assert max_abs <= bar and d_lse <= 1e-2
    if wl.cache_dtype != "fp8":
        assert rel <= 5e-3


def test_step_stages_compose():
    from mla_latent_kv_06_amd import binding as b
    wl = CASES["bf16_q1"]
    announce("decode_step stages", wl.name)
    case = build_case(wl)
    ref, dc = two_copies(case)
    ref_out, ref_lse = step(ref, 0)
    out, lse = step(dc, 0, stages=b.STEP_PROJECT | b.STEP_FINALIZE_ABSORB)
    step(dc, 0, stages=b.STEP_SPLIT_KV)
    # the combine writes into the caller's out / lse: run it on the same tensors
    b.decode_step(dc.dims, dc.h, dc.w_kv_a, dc.gamma, dc.start_pos, dc.q_nope, dc.q_pe, dc.w_uk,
                  dc.w_uv, dc.pool, dc.scale, dc.block_table, dc.seq_lens, num_splits=0,
                  rms_eps=casebuild.RMS_EPS, rope_base=casebuild.ROPE_BASE, out=out, lse=lse,
                  stages=b.STEP_COMBINE)
    assert_same(ref, ref_out, ref_lse, dc, out, lse, "stages")


def test_step_portable_path():
    """A small head shape with f32 activations: unfused launches, same results."""
    wl = W["tiny_f32"].replace(name="tiny_step", append=True, batch=2, ctx_lo=5, ctx_hi=70,
                               d_model=64)
    announce("decode_step portable", wl.name)
    case = build_case(wl)
    ref, dc = two_copies(case)
    ref.append()
    ref_out, ref_lse = ref.decode(num_splits=2)
    out, lse = step(dc, 2)
    assert_same(ref, ref_out, ref_lse, dc, out, lse, "portable")
