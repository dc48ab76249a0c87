"""GPU parity of mla_query_project (the query path) against the CPU oracle's
``query_rows``, and of the query path followed by the decode against
``query_rows`` followed by ``decode_naive``.

Bars.  The kernels round c_Q to bf16 between the two products (relative 2^-9
per element, which reaches q as about 2^-9.8 of its RMS, up to ~5 sigma over
millions of elements) and round q to bf16 on output (2^-9 relative).  Element
by element: |q - ref| <= 2^-8 |ref| + 2^-6 rms(ref); over the tensor: rel-L2
<= 5e-3 (the bf16 bar of the decode).  The end-to-end check uses the decode's
bars (output max-abs 2e-2 and rel-L2 5e-3, lse 1e-2).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from mla_latent_kv_06_amd import synth
from tests import casebuild
from tests.casebuild import build_case, error_stats

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
V3 = W["v3_b64_ctx8k_paged_bf16"]
DEV = "cuda:0"


def announce(*what):
    print("[gpu-case]", *what, flush=True)


def bf(x):
    """float draws -> (bf16 bits, float64 of the stored bf16 values)."""
    bits = casebuild.to_bf16_bits(x)
    return bits, oracle.bf16_bits_to_f64(bits)


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


class QueryCase:
    def __init__(self, wl, q_lora, gamma=True, start=None, seed=0):
        self.wl, self.q_lora = wl, q_lora
        B, Sq, d = wl.batch, wl.q_len, wl.d_model
        self.h_bits, self.h = bf(synth.hidden(wl, seed=seed).reshape(B, Sq, d))
        self.wdq_bits, self.wdq = bf(synth.w_dq(wl, q_lora, seed)) if q_lora else (None, None)
        self.g_bits, self.g = bf(synth.q_norm_gamma(q_lora, seed)) if (q_lora and gamma) else (None, None)
        self.wuq_bits, self.wuq = bf(synth.w_uq(wl, q_lora, seed))
        self.wqr_bits, self.wqr = bf(synth.w_qr(wl, q_lora, seed))
        cached = synth.cached_lengths(wl, seed) if start is None else np.asarray(start, np.int64)
        self.start = cached.astype(np.int32)

    def oracle(self, rows=None):
        wl = self.wl
        B, Sq = wl.batch, wl.q_len
        pos = (self.start[:, None] + np.arange(Sq)[None, :]).reshape(-1)
        h = self.h.reshape(B * Sq, -1)
        sel = np.arange(B * Sq) if rows is None else np.asarray(rows)
        qn, qp = oracle.query_rows(h[sel], self.wdq, self.g, casebuild.RMS_EPS, self.wuq, self.wqr,
                                   pos[sel], wl.n_heads, casebuild.ROPE_BASE)
        return qn, qp

    def run(self):
        from mla_latent_kv_06_amd import binding as b
        dims = b.Dims.from_workload(self.wl)
        opt = lambda x: None if x is None else dev_bf16(x)
        qn, qp = b.query_project(dims, dev_bf16(self.h_bits), opt(self.wdq_bits), opt(self.g_bits),
                                 dev_bf16(self.wuq_bits), dev_bf16(self.wqr_bits),
                                 torch.from_numpy(self.start).to(DEV),
                                 rms_eps=casebuild.RMS_EPS, rope_base=casebuild.ROPE_BASE)
        torch.cuda.synchronize()
        f = lambda t: t.float().cpu().numpy().astype(np.float64)
        T = self.wl.batch * self.wl.q_len
        return f(qn).reshape(T, self.wl.n_heads, -1), f(qp).reshape(T, self.wl.n_heads, -1)


def check(got, ref, tag):
    err = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    ratio = float(np.max(err / (2.0 ** -8 * np.abs(ref) + 2.0 ** -6 * rms)))
    _, rel = error_stats(got, ref)
    print(f"{tag}: max-abs {err.max():.3e} (rms {rms:.3f}) bound use {ratio:.2f} rel-L2 {rel:.3e}",
          flush=True)
    assert np.isfinite(got).all(), tag
    assert ratio <= 1.0, (tag, ratio)
    assert rel <= 5e-3, (tag, rel)


@pytest.mark.parametrize("gamma", [True, False])
def test_query_v3_batch64(gamma):
    """The headline batch: 64 rows at position 8191, d_q 1536."""
    announce("query v3 b64", "gamma", gamma)
    qc = QueryCase(V3, synth.Q_LORA_RANK_V3, gamma=gamma)
    qn, qp = qc.run()
    rn, rp = qc.oracle()
    check(qn, rn, f"q_nope gamma={gamma}")
    check(qp, rp, f"q_pe gamma={gamma}")


def test_query_v3_two_queries_batch128_sampled():
    """bs128 with two query rows per sequence (256 rows, ragged positions
    8k-32k), checked on a sample of rows spread over the token blocks."""
    wl = W["v3_b128_ctx8k32k_fp8_q2"]
    announce(wl.name, "query path")
    qc = QueryCase(wl, synth.Q_LORA_RANK_V3)
    qn, qp = qc.run()
    rows = np.array([0, 1, 31, 32, 63, 100, 127, 128, 200, 254, 255])
    rn, rp = qc.oracle(rows)
    check(qn[rows], rn, "q_nope bs128 q2")
    check(qp[rows], rp, "q_pe bs128 q2")


@pytest.mark.parametrize("batch,q_len", [(1, 1), (3, 1), (33, 1), (5, 2)])
def test_query_ragged_rows(batch, q_len):
    wl = V3.replace(batch=batch, q_len=q_len, ctx_lo=100, ctx_hi=131000)
    announce("query ragged", batch, q_len)
    qc = QueryCase(wl, synth.Q_LORA_RANK_V3)
    qn, qp = qc.run()
    rn, rp = qc.oracle()
    check(qn, rn, f"q_nope B={batch} Sq={q_len}")
    check(qp, rp, f"q_pe B={batch} Sq={q_len}")


def test_query_far_positions():
    """Positions near 2^17: the rotation angle needs more than fp32."""
    wl = V3.replace(batch=4, q_len=2)
    announce("query far positions")
    qc = QueryCase(wl, synth.Q_LORA_RANK_V3, start=[131070, 131000, 65537, 7])
    _, qp = qc.run()
    _, rp = qc.oracle()
    check(qp, rp, "q_pe far positions")


def test_query_full_rank():
    """d_q = 0: W_UQ and W_QR applied to h directly."""
    wl = V3.replace(batch=8, q_len=1)
    announce("query full rank")
    qc = QueryCase(wl, 0)
    qn, qp = qc.run()
    rn, rp = qc.oracle()
    check(qn, rn, "q_nope full rank")
    check(qp, rp, "q_pe full rank")


def test_query_small_head_shape():
    wl = V3.replace(n_heads=4, qk_nope_dim=16, qk_rope_dim=16, d_model=256, batch=6, q_len=2,
                    ctx_lo=0, ctx_hi=50)
    announce("query small heads")
    qc = QueryCase(wl, 64)
    qn, qp = qc.run()
    rn, rp = qc.oracle()
    check(qn, rn, "q_nope small heads")
    check(qp, rp, "q_pe small heads")


def test_query_path_then_decode():
    """Query path + decode on the GPU against query_rows + decode_naive: the
    rotary queries' positions meet the cache's rotated keys."""
    from mla_latent_kv_06_amd import binding as b
    from tests import gpu_util
    wl = W["v3_b64_ctx1k8k_paged_bf16"].replace(name="v3_qpath", batch=3, ctx_lo=40, ctx_hi=450,
                                                 q_len=2, append=False)
    announce("query path + decode")
    case = build_case(wl)
    qc = QueryCase(wl, synth.Q_LORA_RANK_V3, start=case.seq_lens - wl.q_len)
    qn, qp = qc.run()
    dc = gpu_util.DeviceCase(case)
    dc.q_nope = torch.from_numpy(qn.reshape(case.q_nope.shape).astype(np.float32)).to(torch.bfloat16).to(DEV)
    dc.q_pe = torch.from_numpy(qp.reshape(case.q_pe.shape).astype(np.float32)).to(torch.bfloat16).to(DEV)
    out, lse = dc.decode(num_splits=0)
    out, lse = gpu_util.to_np(out), gpu_util.to_np(lse)
    rn, rp = qc.oracle()
    rows_all = case.pool_rows_f64()
    rows = [oracle.gather_sequence(rows_all, case.block_table[i], int(case.seq_lens[i]), wl.block_size)
            for i in range(wl.batch)]
    B, Sq, H = wl.batch, wl.q_len, wl.n_heads
    ref, ref_lse = oracle.decode_naive(rn.reshape(B, Sq, H, -1), rp.reshape(B, Sq, H, -1),
                                       case.act_f64("w_uk"), case.act_f64("w_uv"), rows, Sq)
    max_abs, rel = error_stats(out, ref)
    d_lse = float(np.max(np.abs(lse - ref_lse)))
    print(f"query path + decode: max-abs {max_abs:.3e} rel-L2 {rel:.3e} lse {d_lse:.3e}", flush=True)
    assert max_abs <= 2e-2 and rel <= 5e-3 and d_lse <= 1e-2, (max_abs, rel, d_lse)


def test_query_whole_prompt_sampled():
    """Two 1024-token prompts at once (2048 rows): the projections' row passes
    spread over 22 workgroup rows with no depth split.  Sampled rows across
    the passes and both prompts."""
    wl = V3.replace(batch=2, q_len=1024, ctx_lo=0, ctx_hi=0)
    announce("query whole prompt", "2 x 1024")
    qc = QueryCase(wl, synth.Q_LORA_RANK_V3)
    qn, qp = qc.run()
    rows = np.array([0, 1, 95, 96, 191, 500, 1023, 1024, 1100, 1919, 2047])
    rn, rp = qc.oracle(rows)
    check(qn[rows], rn, "q_nope whole prompt")
    check(qp[rows], rp, "q_pe whole prompt")
