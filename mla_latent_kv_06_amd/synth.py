"""Seeded synthetic inputs for MLA decode and cache-append workloads.

This module holds the workload shapes and the random draws, and nothing of
the method's arithmetic: no projection, normalisation, rotation, softmax or
quantisation happens here.  Raw draws are float32 from
``numpy.random.default_rng``; each kind of input has its own stream keyed by
(seed, stream tag[, sequence index]) so any one sequence's cache can be drawn
without drawing the others.

Value distributions (all draws standard normal, then scaled by a constant):

* cache rows: N(0, 1) per channel.  A workload's cache holds
  [RMSNorm(latent draw) ; RoPE(rotary draw, position = token index)], which the
  caller computes from these draws.
* q_nope, q_pe, h: N(0, 1).
* W_UK [H, N, d_c], W_UV [H, V, d_c]: N(0, 1) / sqrt(d_c)  (std 1/sqrt(fan_in),
  fan_in = d_c, the up-projections' input width).
* W_kv,a [d_c + R, d]: N(0, 1) / sqrt(d).
* query path: W_DQ [d_q, d]: N(0, 1) / sqrt(d); W_UQ [H N, f] and W_QR [H R, f]:
  N(0, 1) / sqrt(f), f = d_q (or d for full-rank queries, d_q = 0); the query
  norm's gamma [d_q]: 1 + 0.1 N(0, 1).
* sequence lengths: uniform integers on the closed range.
* block tables: ceil(L/bs) blocks per sequence taken in order from one random
  permutation of a shared pool (or the identity for contiguous caches); the
  pool has 1% spare blocks (at least one) and table padding is -1.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

# stream tags
_LENGTHS, _BLOCKS, _CACHE, _QNOPE, _QPE, _WUK, _WUV, _H, _WKVA, _WDQ, _WUQ, _WQR, _QG, _WO = range(14)

# query compression width of the DeepSeek-V3 shape (0 = full-rank queries)
Q_LORA_RANK_V3 = 1536


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one decode (+ optional append) workload."""
    name: str
    n_heads: int
    kv_lora_rank: int
    qk_rope_dim: int
    qk_nope_dim: int
    v_head_dim: int
    d_model: int
    block_size: int
    batch: int
    q_len: int
    ctx_lo: int              # cached tokens before the new ones, inclusive range
    ctx_hi: int
    paged: bool              # randomly permuted block table (else identity)
    cache_dtype: str         # "f32" | "bf16" | "fp8"
    act_dtype: str           # "f32" | "bf16"
    num_splits: int = 0      # 0: library heuristic
    append: bool = False     # the new tokens are written by the append kernel

    @property
    def row_width(self) -> int:
        return self.kv_lora_rank + self.qk_rope_dim

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


_V3 = dict(n_heads=128, kv_lora_rank=512, qk_rope_dim=64, qk_nope_dim=128,
           v_head_dim=128, d_model=7168, block_size=64)

# The five graded workloads and the headline measurement point.  ctx_* count
# tokens cached before the step; the q_len new tokens come on top, so a
# sequence's decode length is L_old + q_len.
WORKLOADS = {
    # tiny fp32, 4 heads, 64-token contiguous cache
    "tiny_f32": Workload("tiny_f32", 4, 32, 16, 16, 16, 64, 64, 1, 1, 63, 63,
                         False, "f32", "f32"),
    # V3 single layer, batch 1, 4096-token contiguous cache
    "v3_b1_ctx4k_bf16": Workload("v3_b1_ctx4k_bf16", **_V3, batch=1, q_len=1,
                                 ctx_lo=4095, ctx_hi=4095, paged=False,
                                 cache_dtype="bf16", act_dtype="bf16"),
    # V3, batch 64, contexts U[1024, 8192], paged, plus a one-token append
    "v3_b64_ctx1k8k_paged_bf16": Workload("v3_b64_ctx1k8k_paged_bf16", **_V3, batch=64,
                                          q_len=1, ctx_lo=1024, ctx_hi=8192, paged=True,
                                          cache_dtype="bf16", act_dtype="bf16",
                                          append=True),
    # V3, batch 4, 131072-token contexts, 32 split-KV partitions
    "v3_b4_ctx128k_split32_bf16": Workload("v3_b4_ctx128k_split32_bf16", **_V3, batch=4,
                                           q_len=1, ctx_lo=131071, ctx_hi=131071,
                                           paged=True, cache_dtype="bf16",
                                           act_dtype="bf16", num_splits=32),
    # V3, fp8 cache, batch 128, contexts U[8192, 32768], two causal query tokens
    "v3_b128_ctx8k32k_fp8_q2": Workload("v3_b128_ctx8k32k_fp8_q2", **_V3, batch=128,
                                        q_len=2, ctx_lo=8190, ctx_hi=32766, paged=True,
                                        cache_dtype="fp8", act_dtype="bf16"),
    # headline point: batch 64, every context 8192 after a one-token append
    "v3_b64_ctx8k_paged_bf16": Workload("v3_b64_ctx8k_paged_bf16", **_V3, batch=64,
                                        q_len=1, ctx_lo=8191, ctx_hi=8191, paged=True,
                                        cache_dtype="bf16", act_dtype="bf16",
                                        append=True),
}

# Prefill measurement point: two fresh 8192-token prompts (nothing cached
# before them), paged, bf16; every query sees its causal prefix.
PREFILL_WORKLOADS = {
    "v3_prefill_b2_8k_bf16": Workload("v3_prefill_b2_8k_bf16", **_V3, batch=2, q_len=8192,
                                      ctx_lo=0, ctx_hi=0, paged=True, cache_dtype="bf16",
                                      act_dtype="bf16"),
    "v3_prefill_b2_8k_fp8": Workload("v3_prefill_b2_8k_fp8", **_V3, batch=2, q_len=8192,
                                     ctx_lo=0, ctx_hi=0, paged=True, cache_dtype="fp8",
                                     act_dtype="bf16"),
}


def _rng(seed: int, *tags: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), *[int(t) for t in tags]])


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def cached_lengths(wl: Workload, seed: int = 0) -> np.ndarray:
    """Tokens already cached per sequence (before the q_len new ones), int64 [B]."""
    if wl.ctx_lo == wl.ctx_hi:
        return np.full(wl.batch, wl.ctx_lo, dtype=np.int64)
    return _rng(seed, _LENGTHS).integers(wl.ctx_lo, wl.ctx_hi, size=wl.batch,
                                         endpoint=True).astype(np.int64)


def seq_lens(wl: Workload, seed: int = 0) -> np.ndarray:
    """Decode lengths (cached + new tokens), int32 [B]."""
    return (cached_lengths(wl, seed) + wl.q_len).astype(np.int32)


def block_tables(lengths, block_size: int, paged: bool, seed: int = 0,
                 spare_frac: float = 0.01):
    """Block table [B, max_blocks] int32 (-1 padded) and the pool's block count.

    Sequence b takes ceil(L_b / block_size) blocks, in order, from a random
    permutation of the pool (identity when ``paged`` is False)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    nb = (lengths + block_size - 1) // block_size
    total = int(nb.sum())
    spare = max(1, int(math.ceil(spare_frac * total))) if paged else 0
    num_blocks = total + spare
    ids = _rng(seed, _BLOCKS).permutation(num_blocks) if paged else np.arange(num_blocks)
    max_blocks = int(nb.max()) if len(nb) else 0
    table = np.full((len(lengths), max(max_blocks, 1)), -1, dtype=np.int32)
    at = 0
    for b, n in enumerate(nb):
        table[b, :n] = ids[at:at + n]
        at += n
    return table, num_blocks


def cache_draws(wl: Workload, b: int, length: int, seed: int = 0) -> np.ndarray:
    """Raw N(0,1) draws [length, d_c + R] for sequence b's cached rows."""
    return _normal(_rng(seed, _CACHE, b), (int(length), wl.row_width))


def q_nope(wl: Workload, seed: int = 0) -> np.ndarray:
    return _normal(_rng(seed, _QNOPE), (wl.batch, wl.q_len, wl.n_heads, wl.qk_nope_dim))


def q_pe(wl: Workload, seed: int = 0) -> np.ndarray:
    return _normal(_rng(seed, _QPE), (wl.batch, wl.q_len, wl.n_heads, wl.qk_rope_dim))


def w_uk(wl: Workload, seed: int = 0) -> np.ndarray:
    w = _normal(_rng(seed, _WUK), (wl.n_heads, wl.qk_nope_dim, wl.kv_lora_rank))
    return w * np.float32(1.0 / math.sqrt(wl.kv_lora_rank))


def w_uv(wl: Workload, seed: int = 0) -> np.ndarray:
    w = _normal(_rng(seed, _WUV), (wl.n_heads, wl.v_head_dim, wl.kv_lora_rank))
    return w * np.float32(1.0 / math.sqrt(wl.kv_lora_rank))


def hidden(wl: Workload, n_new: int | None = None, seed: int = 0) -> np.ndarray:
    """Append input h [B, n_new, d] (n_new defaults to q_len)."""
    n = wl.q_len if n_new is None else n_new
    return _normal(_rng(seed, _H), (wl.batch, n, wl.d_model))


def w_kv_a(wl: Workload, seed: int = 0) -> np.ndarray:
    w = _normal(_rng(seed, _WKVA), (wl.row_width, wl.d_model))
    return w * np.float32(1.0 / math.sqrt(wl.d_model))


def w_dq(wl: Workload, q_lora_rank: int, seed: int = 0) -> np.ndarray:
    """Query down-projection [d_q, d]."""
    w = _normal(_rng(seed, _WDQ), (q_lora_rank, wl.d_model))
    return w * np.float32(1.0 / math.sqrt(wl.d_model))


def _q_fan_in(wl: Workload, q_lora_rank: int) -> int:
    return q_lora_rank if q_lora_rank > 0 else wl.d_model


def w_uq(wl: Workload, q_lora_rank: int, seed: int = 0) -> np.ndarray:
    """Query content up-projection [H * N, d_q] (or [H * N, d] at d_q = 0)."""
    f = _q_fan_in(wl, q_lora_rank)
    w = _normal(_rng(seed, _WUQ), (wl.n_heads * wl.qk_nope_dim, f))
    return w * np.float32(1.0 / math.sqrt(f))


def w_qr(wl: Workload, q_lora_rank: int, seed: int = 0) -> np.ndarray:
    """Query rotary projection [H * R, d_q] (or [H * R, d] at d_q = 0)."""
    f = _q_fan_in(wl, q_lora_rank)
    w = _normal(_rng(seed, _WQR), (wl.n_heads * wl.qk_rope_dim, f))
    return w * np.float32(1.0 / math.sqrt(f))


def w_o(wl: Workload, seed: int = 0) -> np.ndarray:
    """Output projection [d, H * V]: column block h * V .. +V acts on head h."""
    f = wl.n_heads * wl.v_head_dim
    w = _normal(_rng(seed, _WO), (wl.d_model, f))
    return w * np.float32(1.0 / math.sqrt(f))


def q_norm_gamma(q_lora_rank: int, seed: int = 0) -> np.ndarray:
    """Query-latent norm weights [d_q]: 1 + 0.1 N(0, 1)."""
    return np.float32(1.0) + np.float32(0.1) * _normal(_rng(seed, _QG), (q_lora_rank,))
