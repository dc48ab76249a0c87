"""Host-side assembly of seeded test cases (inputs + what the oracle needs).

Draws come from ``mla_latent_kv_06_amd.synth``; the cache rows a workload
holds are [RMSNorm(latent draw) ; RoPE(rotary draw, position)] computed with
the oracle's float64 functions, then stored in the cache dtype:

* bf16: round-to-nearest-even by torch's CPU cast,
* fp8:  the oracle's per-token e4m3 quantiser (scale = amax / 448),
* f32:  float32.

Unused pool slots and spare blocks are poisoned with NaN so a kernel that
reads outside the visible tokens shows it.  Pools are held in the library's
layout (``mla_latent_kv_06_amd.layout``: token-major blocks);
``Case.rows`` gives token rows.
"""

from __future__ import annotations

import concurrent.futures
import dataclasses

import numpy as np
import torch

import oracle
from mla_latent_kv_06_amd import layout, synth

RMS_EPS = 1e-6
ROPE_BASE = 10000.0

BF16_NAN = np.uint16(0x7FC0)
FP8_NAN = np.uint8(0x7F)


def to_bf16_bits(x) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32)))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def store_act(x, dtype: str) -> np.ndarray:
    """Activation / weight storage: bf16 bit patterns or float32."""
    if dtype == "bf16":
        return to_bf16_bits(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    raise ValueError(dtype)


def act_to_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return oracle.bf16_bits_to_f64(stored)
    return np.asarray(stored, dtype=np.float64)


def cache_rows_f64(wl: synth.Workload, b: int, length: int, seed: int = 0) -> np.ndarray:
    """Exact cache rows of sequence b (positions 0..length-1), float64."""
    raw = synth.cache_draws(wl, b, length, seed).astype(np.float64)
    lat = oracle.rmsnorm(raw[:, :wl.kv_lora_rank], None, RMS_EPS)
    kr = oracle.rope(raw[:, wl.kv_lora_rank:], np.arange(length), ROPE_BASE)
    return np.concatenate([lat, kr], axis=1)


@dataclasses.dataclass
class Case:
    wl: synth.Workload
    seed: int
    cached: np.ndarray          # [B] tokens in the cache before the step
    seq_lens: np.ndarray        # [B] int32 decode lengths (cached + q_len)
    block_table: np.ndarray     # [B, max_blocks] int32
    num_blocks: int
    pool: np.ndarray            # [num_blocks, bs, D] uint16 (bf16) | uint8 (fp8) | float32, library layout
    scale: np.ndarray | None    # [num_blocks, bs] float32 (fp8 only)
    q_nope: np.ndarray          # stored dtype
    q_pe: np.ndarray
    w_uk: np.ndarray
    w_uv: np.ndarray
    filled: list                # sequences whose rows were written
    h: np.ndarray | None = None
    w_kv_a: np.ndarray | None = None
    gamma: np.ndarray | None = None

    # ---- float64 views of what the device holds -------------------------
    def rows(self, pool=None) -> np.ndarray:
        """Token rows [num_blocks * bs, D] of a pool in the library layout."""
        return layout.pool_rows(self.pool if pool is None else pool, self.wl.cache_dtype)

    def pool_rows_f64(self, pool=None, scale=None) -> np.ndarray:
        scale = self.scale if scale is None else scale
        raw = self.rows(pool)
        if self.wl.cache_dtype == "bf16":
            return oracle.bf16_bits_to_f64(raw)
        if self.wl.cache_dtype == "fp8":
            return oracle.dequantize_rows_fp8(raw, scale.reshape(-1))
        return raw.astype(np.float64)

    def seq_rows(self, b: int, pool=None, scale=None, length=None) -> np.ndarray:
        rows = self.pool_rows_f64(pool, scale)
        L = int(self.seq_lens[b] if length is None else length)
        return oracle.gather_sequence(rows, self.block_table[b], L, self.wl.block_size)

    def act_f64(self, name: str) -> np.ndarray:
        return act_to_f64(getattr(self, name), self.wl.act_dtype)

    def oracle_decode(self, seqs=None, heads=None, pool=None, scale=None):
        """Oracle output for the listed sequences (all by default) and heads."""
        seqs = list(range(self.wl.batch)) if seqs is None else list(seqs)
        rows_all = self.pool_rows_f64(pool, scale)
        qn = self.act_f64("q_nope")[seqs]
        qp = self.act_f64("q_pe")[seqs]
        wuk = self.act_f64("w_uk")
        wuv = self.act_f64("w_uv")
        if heads is not None:
            qn, qp, wuk, wuv = qn[:, :, heads], qp[:, :, heads], wuk[heads], wuv[heads]
        rows = [oracle.gather_sequence(rows_all, self.block_table[b], int(self.seq_lens[b]),
                                       self.wl.block_size) for b in seqs]
        scale_ = oracle.default_softmax_scale(self.wl.qk_nope_dim, self.wl.qk_rope_dim)
        return oracle.decode_naive(qn, qp, wuk, wuv, rows, self.wl.q_len, scale_)


def build_case(wl: synth.Workload, seed: int = 0, fill=None, seq_lens_override=None) -> Case:
    """Assemble a case.  ``fill``: sequences whose cache rows are drawn exactly
    (default all); the other sequences' blocks stay NaN-poisoned, which is
    only valid when their outputs are not checked."""
    cached = synth.cached_lengths(wl, seed)
    if seq_lens_override is not None:
        cached = np.asarray(seq_lens_override, dtype=np.int64) - wl.q_len
    seq_lens = (cached + wl.q_len).astype(np.int32)
    table, num_blocks = synth.block_tables(seq_lens, wl.block_size, wl.paged, seed)
    D, bs = wl.row_width, wl.block_size
    if wl.cache_dtype == "bf16":
        pool = np.full((num_blocks, bs, D), BF16_NAN, dtype=np.uint16)
        scale = None
    elif wl.cache_dtype == "fp8":
        pool = np.full((num_blocks, bs, D), FP8_NAN, dtype=np.uint8)
        scale = np.full((num_blocks, bs), np.nan, dtype=np.float32)
    else:
        pool = np.full((num_blocks, bs, D), np.nan, dtype=np.float32)
        scale = None
    flat = pool.reshape(-1, D)
    flat_scale = None if scale is None else scale.reshape(-1)
    fill = list(range(wl.batch)) if fill is None else list(fill)
    def write(b):
        # rows the cache already holds before the step: all decode tokens for
        # decode-only workloads, the cached prefix when the append writes the rest
        n_rows = int(cached[b]) if wl.append else int(seq_lens[b])
        rows = cache_rows_f64(wl, b, n_rows, seed)
        j = np.arange(n_rows)
        phys = table[b, j // bs].astype(np.int64) * bs + j % bs
        if wl.cache_dtype == "bf16":
            flat[phys] = to_bf16_bits(rows)
        elif wl.cache_dtype == "fp8":
            codes, sc = oracle.quantize_rows_fp8(rows)
            flat[phys] = codes
            flat_scale[phys] = sc
        else:
            flat[phys] = rows.astype(np.float32)

    # sequences own disjoint slots, and numpy drops the GIL in the heavy steps
    with concurrent.futures.ThreadPoolExecutor(min(8, max(1, len(fill)))) as ex:
        list(ex.map(write, fill))
    pool = layout.rows_to_pool(flat, bs, wl.cache_dtype)      # token rows -> library layout
    case = Case(
        wl=wl, seed=seed, cached=cached, seq_lens=seq_lens, block_table=table,
        num_blocks=num_blocks, pool=pool, scale=scale,
        q_nope=store_act(synth.q_nope(wl, seed), wl.act_dtype),
        q_pe=store_act(synth.q_pe(wl, seed), wl.act_dtype),
        w_uk=store_act(synth.w_uk(wl, seed), wl.act_dtype),
        w_uv=store_act(synth.w_uv(wl, seed), wl.act_dtype),
        filled=fill,
    )
    if wl.append:
        case.h = store_act(synth.hidden(wl, seed=seed), wl.act_dtype)
        case.w_kv_a = store_act(synth.w_kv_a(wl, seed), wl.act_dtype)
        case.gamma = store_act(np.ones(wl.kv_lora_rank, dtype=np.float32), wl.act_dtype)
    return case


def error_stats(got: np.ndarray, ref: np.ndarray):
    """(max-abs, rel-L2) of got vs ref over the whole tensor."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    denom = float(np.linalg.norm(ref.ravel()))
    rel = float(np.linalg.norm(diff.ravel())) / denom if denom > 0 else float(np.linalg.norm(diff.ravel()))
    return max_abs, rel
