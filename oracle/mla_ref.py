"""Naive float64 reference for MLA decode and the latent-cache append.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
HIP library or its binding.

Sources, by page title and section:

* "DeepSeek-V2: MLA Explained" (mibrahim.dev), "MLA Full Formulas":
  section 2 (key-value joint compression: per-head content keys and values are
  up-projections of one shared latent; the rotary key is shared by all heads
  and concatenated to every head's content key) and section 3 (attention:
  per-head softmax over cached tokens 1..t of q.k / sqrt(d_h + d_h^R),
  weighting the per-head values).
* "KV Compression -- DeepSeek-V3" (AI Engineer Exhaustive), "How it works":
  one linear map emits 512 latent channels followed by the 64-channel rotary
  key before rotation; the latent is RMS-normalised before it is cached.
* "DeepSeek-V2: MLA Explained", "MLA Full Formulas", section 3 (last
  equation): the heads' outputs, concatenated head after head, go through
  one output projection W_O.
* "HuggingFace version does NOT use efficient MLA caching" (DeepSeek-R1
  discussion), list item 2: cache the latent and the rotary key, rebuild full
  per-head keys and values at every step.  That "decompress" form is what
  ``decode_naive`` computes; it never uses the weight-absorbed shortcut.

Readings where the pages are silent (the plainest reading the rest supports):

* RMSNorm is y = x / sqrt(mean(x^2) + eps) * gamma (the pages name it only).
* RoPE rotates interleaved pairs (x[2k], x[2k+1]) by angle
  pos * base^(-2k/R); base 10000, position = token index.
* Query row s of a sequence holding L tokens (the q_len new ones included)
  sees tokens 0 .. L - q_len + s (causal, bottom-right aligned).
* A row that sees no token outputs zeros and lse = -inf.
"""

from __future__ import annotations

import math

import numpy as np



def default_softmax_scale(qk_nope_dim: int, qk_rope_dim: int) -> float:
    """1 / sqrt(d_h + d_h^R): the score divisor of "DeepSeek-V2: MLA
    Explained", section 3, with d_h read as the per-head content (nope) width."""
    return 1.0 / math.sqrt(qk_nope_dim + qk_rope_dim)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode raw bfloat16 bit patterns (uint16) to float64.

    bfloat16 is the upper half of an IEEE binary32, so widening the pattern by
    16 zero bits gives the exact binary32 value."""
    bits = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even), as
    float64.  bfloat16 keeps 8 significant bits and binary32's exponent range;
    below 2^-126 the spacing stays 2^-133 (subnormals).  Overflow is not
    handled (the values rounded here are far below 2^127)."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                       # x = m 2^e, 0.5 <= |m| < 1
    q = np.maximum(e, -125) - 8              # exponent of the last kept bit
    return np.ldexp(np.rint(np.ldexp(x, -q)), q)   # rint: ties to even


def rmsnorm(x: np.ndarray, gamma: np.ndarray | None = None, eps: float = 0.0) -> np.ndarray:
    """Root-mean-square normalisation over the last axis, in float64.

    The latent RMSNorm of "KV Compression -- DeepSeek-V3", "How it works"
    (the formula itself is not printed; this is the standard definition)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    y = x / np.sqrt(ms + eps)
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)
    return y


def rope(x: np.ndarray, positions, base: float = 10000.0) -> np.ndarray:
    """Rotary position embedding on the last axis (width R, even), float64.

    The decoupled rotary key of "DeepSeek-V2: MLA Explained", section 2
    (k^R_t = RoPE(W^KR h_t)).  Pair k = (x[2k], x[2k+1]) is rotated by the
    angle pos * base^(-2k/R), k = 0 .. R/2 - 1."""
    x = np.asarray(x, dtype=np.float64)
    r = x.shape[-1]
    if r % 2:
        raise ValueError("rope width must be even")
    pos = np.asarray(positions, dtype=np.float64)
    k = np.arange(r // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * k / r)                      # [R/2]
    ang = pos[..., None] * inv_freq                        # [..., R/2]
    c, s = np.cos(ang), np.sin(ang)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def append_rows(h, w_kv_a, gamma, eps, positions, kv_lora_rank, rope_base=10000.0):
    """The cache rows one new token adds: [RMSNorm(c_t) ; RoPE(k~_t)].

    "KV Compression -- DeepSeek-V3", "How it works": one map W_kv,a (rows
    0..d_c-1 are W^DKV, rows d_c.. are W^KR) sends h_t to
    [c_t ; k~_t] (equation (1) widened by the rotary rows); the latent part is
    RMS-normalised and the rotary part rotated by the token's position.

    h: [T, d] ; w_kv_a: [d_c + R, d] ; gamma: [d_c] ; positions: [T].
    Returns float64 rows [T, d_c + R], not rounded to any storage type."""
    h = np.asarray(h, dtype=np.float64)
    w = np.asarray(w_kv_a, dtype=np.float64)
    x = h @ w.T                                            # [T, d_c + R]
    lat = rmsnorm(x[:, :kv_lora_rank], gamma, eps)
    kr = rope(x[:, kv_lora_rank:], positions, rope_base)
    return np.concatenate([lat, kr], axis=1)


def query_rows(h, w_dq, q_gamma, eps, w_uq, w_qr, positions, n_heads, rope_base=10000.0):
    """Query path of "DeepSeek-V2: MLA Explained", "MLA Full Formulas", step 1
    (query compression), in float64:

      c_Q   = W_DQ h                         (h itself when w_dq is None:
                                              full-rank queries, q_lora_rank 0)
      c_Q   = RMSNorm(c_Q) * gamma           when q_gamma is given (the V3
                                              reading: "KV Compression --
                                              DeepSeek-V3" notes RMSNorm after
                                              the compressed latent vectors)
      q^C   = W_UQ c_Q,  split into n_heads blocks [q^C_1; ...; q^C_H]
      q^R   = RoPE(W_QR c_Q), per head block, at the token's position

    h [T, d]; w_dq [d_q, d]; w_uq [H * N, d_q]; w_qr [H * R, d_q];
    positions [T].  Returns (q_nope [T, H, N], q_pe [T, H, R])."""
    h = np.asarray(h, dtype=np.float64)
    c = h if w_dq is None else h @ np.asarray(w_dq, dtype=np.float64).T
    if q_gamma is not None:
        c = rmsnorm(c, q_gamma, eps)
    T = c.shape[0]
    q_nope = (c @ np.asarray(w_uq, dtype=np.float64).T).reshape(T, n_heads, -1)
    qr = (c @ np.asarray(w_qr, dtype=np.float64).T).reshape(T, n_heads, -1)
    pos = np.asarray(positions, dtype=np.float64)
    q_pe = np.stack([rope(qr[:, i, :], pos, rope_base) for i in range(n_heads)], axis=1)
    return q_nope, q_pe


def slot_index(block_table: np.ndarray, b: int, pos: int, block_size: int) -> int:
    """Physical row (block * block_size + offset) that token ``pos`` of
    sequence ``b`` occupies in the paged pool."""
    return int(block_table[b, pos // block_size]) * block_size + pos % block_size


def gather_sequence(pool_rows: np.ndarray, block_table_row: np.ndarray, length: int,
                    block_size: int) -> np.ndarray:
    """Rows 0..length-1 of one sequence, read through its block-table row.

    pool_rows: [num_blocks * block_size, D] (any dtype; returned as given)."""
    j = np.arange(length)
    phys = np.asarray(block_table_row, dtype=np.int64)[j // block_size] * block_size + j % block_size
    return pool_rows[phys]


def decode_naive(q_nope, q_pe, w_uk, w_uv, seq_rows, q_len, softmax_scale=None):
    """Naive MLA decode in float64 ("decompress" form).

    For every sequence b, query row s and head i, following "DeepSeek-V2: MLA
    Explained", sections 2 and 3:

      K_{j,i} = [W_UK[i] c_j ; k^R_j]          (content key ; shared rotary key)
      V_{j,i} =  W_UV[i] c_j
      q_i     = [q^C_i ; q^R_i]
      o_i     = sum_j softmax_j(q_i . K_{j,i} * scale) V_{j,i}

    over the tokens row s may see (0 .. L_b - q_len + s).

    q_nope [B, Sq, H, N], q_pe [B, Sq, H, R], w_uk [H, N, d_c], w_uv [H, V, d_c];
    seq_rows: list of B float arrays [L_b, d_c + R] (latent then rotary key).
    Returns (out [B, Sq, H, V], lse [B, Sq, H]) in float64; lse is the natural
    log of the softmax denominator of the scaled scores.
    """
    q_nope = np.asarray(q_nope, dtype=np.float64)
    q_pe = np.asarray(q_pe, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    B, Sq, H, N = q_nope.shape
    R = q_pe.shape[-1]
    d_c = w_uk.shape[-1]
    V = w_uv.shape[1]
    if Sq != q_len:
        raise ValueError("q_len does not match q_nope")
    scale = default_softmax_scale(N, R) if softmax_scale is None else float(softmax_scale)
    out = np.zeros((B, Sq, H, V))
    lse = np.full((B, Sq, H), -np.inf)
    for b in range(B):
        rows = np.asarray(seq_rows[b], dtype=np.float64)
        L = rows.shape[0]
        c = rows[:, :d_c]
        kr = rows[:, d_c:]
        for i in range(H):
            k_full = np.concatenate([c @ w_uk[i].T, kr], axis=1)   # [L, N + R]
            v_full = c @ w_uv[i].T                                  # [L, V]
            for s in range(Sq):
                n_vis = L - Sq + s + 1
                if n_vis <= 0:
                    continue
                q = np.concatenate([q_nope[b, s, i], q_pe[b, s, i]])
                sc = (k_full[:n_vis] @ q) * scale
                m = sc.max()
                e = np.exp(sc - m)
                tot = e.sum()
                out[b, s, i] = (e / tot) @ v_full[:n_vis]
                lse[b, s, i] = m + math.log(tot)
    return out, lse


def decode_absorbed(q_nope, q_pe, w_uk, w_uv, seq_rows, q_len, softmax_scale=None):
    """MLA decode in the weight-absorbed form, float64.

    "DeepSeek-V2: MLA Explained", "Optimization Note": W_UK moves onto the
    query side and W_UV onto the output by associativity, so per sequence b,
    query row s and head i

      q_lat_i = W_UK[i]^T q^C_i                       (d_c values)
      s_j     = (q_lat_i . c_j + q^R_i . k^R_j) * scale
      o_lat_i = sum_j softmax_j(s) c_j
      o_i     = W_UV[i] o_lat_i

    over the tokens row s may see.  Equal to ``decode_naive`` up to rounding
    (matrix associativity); it costs 2 (d_c + R + d_c) flops per visible
    token and head instead of the naive form's decompression, which makes
    whole-workload checks of the large configurations affordable.
    Arguments and results as ``decode_naive``."""
    q_nope = np.asarray(q_nope, dtype=np.float64)
    q_pe = np.asarray(q_pe, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    B, Sq, H, N = q_nope.shape
    R = q_pe.shape[-1]
    d_c = w_uk.shape[-1]
    V = w_uv.shape[1]
    if Sq != q_len:
        raise ValueError("q_len does not match q_nope")
    scale = default_softmax_scale(N, R) if softmax_scale is None else float(softmax_scale)
    out = np.zeros((B, Sq, H, V))
    lse = np.full((B, Sq, H), -np.inf)
    for b in range(B):
        rows = np.asarray(seq_rows[b], dtype=np.float64)
        L = rows.shape[0]
        c = rows[:, :d_c]
        kr = rows[:, d_c:]
        for s in range(Sq):
            n_vis = L - Sq + s + 1
            if n_vis <= 0:
                continue
            q_lat = np.stack([w_uk[i].T @ q_nope[b, s, i] for i in range(H)])   # [H, d_c]
            sc = (q_lat @ c[:n_vis].T + q_pe[b, s] @ kr[:n_vis].T) * scale       # [H, n_vis]
            m = sc.max(axis=1)
            e = np.exp(sc - m[:, None])
            tot = e.sum(axis=1)
            o_lat = (e / tot[:, None]) @ c[:n_vis]                               # [H, d_c]
            out[b, s] = np.stack([w_uv[i] @ o_lat[i] for i in range(H)])
            lse[b, s] = m + np.log(tot)
    return out, lse



def output_rows(o, w_o):
    """Output projection in float64: u = W_O [o_1; ...; o_H].

    "DeepSeek-V2: MLA Explained", "MLA Full Formulas", section 3: per query
    row, the H heads' outputs are concatenated head after head (a vector of
    H * V values) and multiplied by W_O.

    o [B, Sq, H, V] (a decode's output), w_o [d_model, H * V] whose columns
    h * V .. (h + 1) * V act on head h.  Returns u [B, Sq, d_model]."""
    o = np.asarray(o, dtype=np.float64)
    w_o = np.asarray(w_o, dtype=np.float64)
    B, Sq, H, V = o.shape
    if w_o.ndim != 2 or w_o.shape[1] != H * V:
        raise ValueError("w_o must be [d_model, H * V]")
    concat = o.reshape(B, Sq, H * V)            # [o_1; ...; o_H] for every row
    return concat @ w_o.T
