"""mla_decode_step captured into a HIP graph (torch.cuda.CUDAGraph on a
capturing stream): the library only enqueues kernels on the caller's stream,
so the whole step -- append projection, finalize + query absorption,
split-KV, combine -- replays from the graph.  Each replay, with eager work
between replays, must give bit for bit the output, lse and pool of the same
step run eagerly on a copy of the inputs (the replayed append rewrites the
same token's slot with the same values)."""

from __future__ import annotations

import pytest
import torch

from mla_latent_kv_06_amd import synth
from tests import casebuild
from tests.casebuild import build_case

pytestmark = pytest.mark.gpu
W = synth.WORKLOADS


def G():
    from tests import gpu_util
    return gpu_util


def step_call(dc, **kw):
    from mla_latent_kv_06_amd import binding as b
    return b.decode_step(dc.dims, dc.h, dc.w_kv_a, dc.gamma, dc.start_pos, dc.q_nope, dc.q_pe,
                         dc.w_uk, dc.w_uv, dc.pool, dc.scale, dc.block_table, dc.seq_lens,
                         num_splits=0, rms_eps=casebuild.RMS_EPS, rope_base=casebuild.ROPE_BASE, **kw)


CASES = {
    "bf16_q1": W["v3_b64_ctx1k8k_paged_bf16"].replace(name="v3_graph_bf16", batch=6, ctx_lo=30,
                                                      ctx_hi=900),
    "fp8_q2": W["v3_b64_ctx1k8k_paged_bf16"].replace(name="v3_graph_fp8", batch=3, ctx_lo=2,
                                                     ctx_hi=400, cache_dtype="fp8", q_len=2),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_step_replays_from_a_graph(name):
    from mla_latent_kv_06_amd import binding as b
    wl = CASES[name]
    print("[gpu-case] decode_step graph", wl.name, "q_len", wl.q_len, flush=True)
    case = build_case(wl)
    ref, dc = G().DeviceCase(case), G().DeviceCase(case)
    ref_out, ref_lse = step_call(ref)
    torch.cuda.synchronize()

    # buffers the graph writes, allocated before capture
    out = torch.empty_like(ref_out)
    lse = torch.empty_like(ref_lse)
    ws = torch.empty(b.step_workspace_size(dc.dims, wl.batch, wl.q_len, wl.d_model), dtype=torch.uint8,
                     device=ref_out.device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):              # one eager run on the capturing stream first
        step_call(dc, out=out, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step_call(dc, out=out, lse=lse, workspace=ws)
    for rep in range(3):
        out.fill_(float("nan"))                # eager work between replays
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same_out = torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        same_lse = torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
        same_pool = torch.equal(dc.pool.view(torch.uint8), ref.pool.view(torch.uint8))
        print(f"replay {rep}: out {same_out} lse {same_lse} pool {same_pool}", flush=True)
        assert same_out and same_lse and same_pool
        if dc.scale is not None:
            assert torch.equal(dc.scale.view(torch.int32), ref.scale.view(torch.int32))
