"""Chunked prefill through the library's calls, against the oracle alone.

A prompt of L tokens per sequence is processed in chunks: for each chunk of
C tokens, mla_cache_append writes their cache rows, mla_query_project forms
their queries from the same layer input h, and mla_decode_absorbed or
mla_prefill (q_len = C, causal inside the chunk) attends over everything
cached so far.  The
concatenated outputs must equal causal attention over the whole prompt:
``decode_naive`` with q_len = L on the oracle's own cache rows
(``append_rows``) and queries (``query_rows``), all from the same seeded
draws.  No expected value comes from the device.

Bars.  The cache holds bf16 rows, so the oracle attends over its own rows
rounded to bf16 (``round_to_bf16``), as the decode-only tests read back the
stored bf16 rows.  The scores then still carry three roundings the decode-only
tests do not (c_Q, q and q_lat), each moving a score by up to ~2^-9 of its
size, and the first rows of a prompt see one or two tokens, so nothing
averages out.  The bars are the decode's: output max-abs <= 2e-2, rel-L2 <=
5e-3, lse <= 1e-2.
"""

from __future__ import annotations

import time

import numpy as np
import pytest
import torch

import oracle
from mla_latent_kv_06_amd import synth
from tests import casebuild
from tests.casebuild import error_stats

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def announce(*what):
    print("[gpu-case]", *what, flush=True)


def bf(x):
    bits = casebuild.to_bf16_bits(x)
    return bits, oracle.bf16_bits_to_f64(bits)


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


@pytest.mark.parametrize("L,C,attn", [(300, 128, "decode"), (200, 64, "decode"),
                                      (300, 128, "prefill"), (300, 300, "prefill")])
def test_chunked_prefill(L, C, attn):
    from mla_latent_kv_06_amd import binding as b
    B = 2
    wl = synth.WORKLOADS["v3_b64_ctx1k8k_paged_bf16"].replace(
        name="v3_prefill", batch=B, q_len=L, ctx_lo=0, ctx_hi=0, append=True)
    ql = synth.Q_LORA_RANK_V3
    announce("chunked prefill", "L", L, "C", C, "attention", attn)
    dims = b.Dims.from_workload(wl)
    H, N, R, V, dc = wl.n_heads, wl.qk_nope_dim, wl.qk_rope_dim, wl.v_head_dim, wl.kv_lora_rank

    h_bits, h = bf(synth.hidden(wl, n_new=L))                         # [B, L, d]
    wkva_bits, wkva = bf(synth.w_kv_a(wl))
    g_kv = np.ones(dc)
    wdq_bits, wdq = bf(synth.w_dq(wl, ql))
    gq_bits, gq = bf(synth.q_norm_gamma(ql))
    wuq_bits, wuq = bf(synth.w_uq(wl, ql))
    wqr_bits, wqr = bf(synth.w_qr(wl, ql))
    wuk_bits, wuk = bf(synth.w_uk(wl))
    wuv_bits, wuv = bf(synth.w_uv(wl))

    # ---- device: chunk by chunk ------------------------------------------------
    seq = np.full(B, L, dtype=np.int64)
    table, nblk = synth.block_tables(seq, wl.block_size, True)
    pool = torch.zeros((nblk, wl.block_size, wl.row_width), dtype=torch.bfloat16, device=DEV)
    bt = torch.from_numpy(table).to(DEV)
    h_dev = dev_bf16(h_bits)
    wkva_d, wdq_d, gq_d = dev_bf16(wkva_bits), dev_bf16(wdq_bits), dev_bf16(gq_bits)
    wuq_d, wqr_d, wuk_d, wuv_d = dev_bf16(wuq_bits), dev_bf16(wqr_bits), dev_bf16(wuk_bits), dev_bf16(wuv_bits)
    gkv_d = torch.ones(dc, dtype=torch.bfloat16, device=DEV)
    outs, lses = [], []
    torch.cuda.synchronize()
    t0 = time.time()
    for s0 in range(0, L, C):
        c = min(C, L - s0)
        dchunk = b.Dims.from_workload(wl.replace(q_len=c))
        hc = h_dev[:, s0:s0 + c].contiguous()
        start = torch.full((B,), s0, dtype=torch.int32, device=DEV)
        b.append(dchunk, hc, wkva_d, gkv_d, bt, start, pool, None,
                 rms_eps=casebuild.RMS_EPS, rope_base=casebuild.ROPE_BASE)
        qn, qp = b.query_project(dchunk, hc, wdq_d, gq_d, wuq_d, wqr_d, start,
                                 rms_eps=casebuild.RMS_EPS, rope_base=casebuild.ROPE_BASE)
        lens = torch.full((B,), s0 + c, dtype=torch.int32, device=DEV)
        if attn == "decode":
            out, lse = b.decode(dchunk, qn, qp, wuk_d, wuv_d, pool, None, bt, lens, num_splits=0)
        else:
            out, lse = b.prefill(dchunk, qn, qp, wuk_d, wuv_d, pool, None, bt, lens)
        outs.append(out)
        lses.append(lse)
    torch.cuda.synchronize()
    dt = time.time() - t0
    out = torch.cat(outs, dim=1).float().cpu().numpy().astype(np.float64)      # [B, L, H, V]
    lse = torch.cat(lses, dim=1).float().cpu().numpy().astype(np.float64)
    print(f"chunked prefill B={B} L={L} C={C}: {dt * 1e3:.1f} ms wall for {B * L} tokens "
          f"(first call includes set-up)", flush=True)

    # ---- oracle: the whole prompt at once ----------------------------------------
    pos = np.arange(L)
    rows = [oracle.round_to_bf16(oracle.append_rows(h[i], wkva, g_kv, casebuild.RMS_EPS, pos, dc,
                                                    casebuild.ROPE_BASE))
            for i in range(B)]
    qn_r, qp_r = [], []
    for i in range(B):
        a, c_ = oracle.query_rows(h[i], wdq, gq, casebuild.RMS_EPS, wuq, wqr, pos, H, casebuild.ROPE_BASE)
        qn_r.append(a)
        qp_r.append(c_)
    ref, ref_lse = oracle.decode_naive(np.stack(qn_r), np.stack(qp_r), wuk, wuv, rows, L)
    max_abs, rel = error_stats(out, ref)
    d_lse = float(np.max(np.abs(lse - ref_lse)))
    print(f"chunked prefill L={L} C={C}: max-abs {max_abs:.3e} rel-L2 {rel:.3e} lse {d_lse:.3e}",
          flush=True)
    assert np.isfinite(out).all()
    assert max_abs <= 2e-2 and rel <= 5e-3 and d_lse <= 1e-2, (max_abs, rel, d_lse)
