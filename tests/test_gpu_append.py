"""GPU parity of mla_cache_append against the oracle.

* Slots: exactly the batch * n_new addressed rows change; every other byte of
  the pool (NaN-poisoned spare slots included) stays bit-identical.
* bf16 rows: max-abs <= 2e-2 and rel-L2 <= 5e-3 against the unrounded float64
  row of the oracle.
* fp8 rows: the scale matches amax / 448 (relative 1e-5) and each stored value
  is one of the two e4m3 grid points (times the scale) bracketing the exact
  value, so only the rounding direction at a tie-free boundary can differ.
Then decode parity on the pool the GPU actually holds after the append.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from mla_latent_kv_06_amd import layout, synth
from tests import casebuild
from tests.casebuild import build_case, error_stats

pytestmark = pytest.mark.gpu
W = synth.WORKLOADS


def announce(*what):
    print("[gpu-case]", *what, flush=True)


def G():
    from tests import gpu_util
    return gpu_util


def expected_rows(case):
    wl = case.wl
    h = case.act_f64("h").reshape(-1, wl.d_model)
    w = case.act_f64("w_kv_a")
    g = case.act_f64("gamma")
    pos = (case.cached[:, None] + np.arange(wl.q_len)[None, :]).reshape(-1)
    rows = oracle.append_rows(h, w, g, casebuild.RMS_EPS, pos, wl.kv_lora_rank, casebuild.ROPE_BASE)
    slots = np.array([oracle.slot_index(case.block_table, t // wl.q_len, int(pos[t]), wl.block_size)
                      for t in range(len(pos))])
    return rows, slots


def run_append(case):
    dc = G().DeviceCase(case)
    before = case.pool.copy()
    before_scale = None if case.scale is None else case.scale.copy()
    dc.append()
    after, after_scale = dc.pool_host()
    return dc, before, before_scale, after, after_scale


def check_untouched(before, after, slots, D):
    """Token rows of the pools (library layout: uint16 pools are bf16) equal
    except at ``slots``; returns the rows at ``slots`` after."""
    kind = "bf16" if before.dtype == np.uint16 else "token-major"
    b = layout.pool_rows(before, kind).reshape(-1, D)
    a = layout.pool_rows(after, kind).reshape(-1, D)
    mask = np.ones(len(b), dtype=bool)
    mask[slots] = False
    assert np.array_equal(a[mask].view(np.uint8), b[mask].view(np.uint8))
    return a[slots]


def _bf16_append(wl, tag):
    announce(tag)
    case = build_case(wl)
    dc, before, _, after, _ = run_append(case)
    rows, slots = expected_rows(case)
    assert len(np.unique(slots)) == len(slots)
    got = oracle.bf16_bits_to_f64(check_untouched(before, after, slots, wl.row_width))
    max_abs, rel = error_stats(got, rows)
    print(f"{tag} append: max-abs {max_abs:.3e} rel-L2 {rel:.3e}", flush=True)
    assert max_abs <= 2e-2 and rel <= 5e-3
    return case, dc, after


def test_append_then_decode_batch64_workload():
    """The batch-64 workload: one new token per sequence, then decode on the
    pool read back from the device."""
    wl = W["v3_b64_ctx1k8k_paged_bf16"]
    lens = synth.seq_lens(wl)
    seqs = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 7, 40})
    announce(wl.name, "fill", seqs)
    case = build_case(wl, fill=seqs)
    dc, before, _, after, _ = run_append(case)
    rows, slots = expected_rows(case)
    got = oracle.bf16_bits_to_f64(check_untouched(before, after, slots, wl.row_width))
    max_abs, rel = error_stats(got, rows)
    print(f"append: max-abs {max_abs:.3e} rel-L2 {rel:.3e}", flush=True)
    assert max_abs <= 2e-2 and rel <= 5e-3
    out, lse = dc.decode()
    out, lse = G().to_np(out), G().to_np(lse)
    heads = np.arange(3, 128, 17)
    ref, ref_lse = case.oracle_decode(seqs=seqs, heads=heads, pool=after)
    ma, rl = error_stats(out[seqs][:, :, heads], ref)
    print(f"decode after append: max-abs {ma:.3e} rel-L2 {rl:.3e}", flush=True)
    assert ma <= 2e-2 and rl <= 5e-3
    assert np.max(np.abs(lse[seqs][:, :, heads] - ref_lse)) <= 1e-2


@pytest.mark.parametrize("n_new", [1, 3])
def test_append_mid_bf16(n_new):
    wl = W["v3_b64_ctx1k8k_paged_bf16"].replace(name="v3_mid_append", batch=5, ctx_lo=60,
                                                ctx_hi=200, q_len=n_new)
    _bf16_append(wl, f"v3_mid_append n_new={n_new}")


def test_append_split_k_kernel():
    """d_model a multiple of 16 but not of 64: the split-K MFMA projection
    (other V3 appends use the weight-streaming GEMM)."""
    wl = W["v3_b64_ctx1k8k_paged_bf16"].replace(name="v3_append_d1040", batch=3, ctx_lo=60,
                                                ctx_hi=200, q_len=2, d_model=1040)
    _bf16_append(wl, "v3 append d_model=1040")


def test_append_long_positions():
    """Positions near 131072: the rotary angle needs double precision."""
    wl = W["v3_b64_ctx1k8k_paged_bf16"].replace(name="v3_far_append", batch=2, ctx_lo=131000,
                                                ctx_hi=131070)
    announce("v3_far_append")
    case = build_case(wl, fill=[])
    dc, before, _, after, _ = run_append(case)
    rows, slots = expected_rows(case)
    got = oracle.bf16_bits_to_f64(check_untouched(before, after, slots, wl.row_width))
    max_abs, rel = error_stats(got, rows)
    assert max_abs <= 2e-2 and rel <= 5e-3


def _bracket_check(codes, scale, rows):
    vals = oracle.e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))
    for t in range(len(rows)):
        x = rows[t] / scale[t]
        got = oracle.e4m3fn_decode(codes[t])
        mag = np.minimum(np.abs(x), 448.0)
        hi = vals[np.clip(np.searchsorted(vals, mag, side="left"), 0, 0x7E)]
        lo = vals[np.clip(np.searchsorted(vals, mag, side="right") - 1, 0, 0x7E)]
        ok = (np.abs(got) == hi) | (np.abs(got) == lo)
        ok &= (np.sign(got) == np.sign(x)) | (got == 0)
        assert ok.all(), (t, np.where(~ok)[0][:5])


@pytest.mark.parametrize("path", ["mfma", "portable"])
def test_append_fp8(path):
    if path == "mfma":
        wl = W["v3_b128_ctx8k32k_fp8_q2"].replace(name="v3_fp8_append", batch=4, ctx_lo=30,
                                                  ctx_hi=300, append=True)
    else:
        wl = synth.Workload("portable_fp8_append", 6, 48, 8, 24, 20, 40, 16, 3, 2, 5, 60, True,
                            "fp8", "f32", append=True)
    announce("fp8 append", path)
    case = build_case(wl)
    dc, before, before_scale, after, after_scale = run_append(case)
    rows, slots = expected_rows(case)
    codes = check_untouched(before, after, slots, wl.row_width)
    sc_before = before_scale.reshape(-1)
    sc_after = after_scale.reshape(-1)
    mask = np.ones(len(sc_before), dtype=bool)
    mask[slots] = False
    assert np.array_equal(sc_after[mask].view(np.uint32), sc_before[mask].view(np.uint32))
    scale = sc_after[slots].astype(np.float64)
    exp_scale = np.max(np.abs(rows), axis=1) / 448.0
    assert np.max(np.abs(scale / exp_scale - 1)) <= 1e-5
    _bracket_check(codes, scale, rows)
    # decode on what the device holds
    out, lse = dc.decode(num_splits=2)
    out = G().to_np(out)
    ref, _ = case.oracle_decode(pool=after, scale=after_scale)
    ma, _ = error_stats(out, ref)
    assert ma <= 6e-2


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_append_portable(act):
    wl = synth.Workload("portable_append", 6, 48, 8, 24, 20, 40, 16, 3, 2, 5, 60, True,
                        "bf16", act, append=True)
    _bf16_append(wl, f"portable append {act}")


def test_append_whole_prompt():
    """4400 new rows at once (two prompts of 2200 tokens after short prefixes):
    the projection's row passes spread over 46 workgroup rows with no depth
    split, the path a whole prompt takes."""
    wl = W["v3_b64_ctx1k8k_paged_bf16"].replace(name="v3_append_prompt", batch=2, ctx_lo=0,
                                                ctx_hi=100, q_len=2200)
    _bf16_append(wl, "v3 append of 2 x 2200 tokens")
