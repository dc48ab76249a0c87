"""Closed-form cache sizes, for pinning the cache layout.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* MLA caches the d_c-wide latent plus the R-wide rotary key per token per
  layer ("KV Compression -- DeepSeek-V3", "How it works"; "DeepSeek-V2: MLA
  Explained", "Caching Strategy").
* Standard multi-head attention caches one key and one value of width d_h per
  KV head ("KV Compression -- DeepSeek-V3", "Overview").
"""

from __future__ import annotations


def mla_elems_per_token_layer(kv_lora_rank: int, qk_rope_dim: int) -> int:
    return kv_lora_rank + qk_rope_dim


def mla_bytes_per_token(n_layers: int, kv_lora_rank: int, qk_rope_dim: int,
                        elem_bytes: int, scale_bytes: int = 0) -> int:
    """All layers' cache bytes for one token (scale_bytes: per-token scale)."""
    return n_layers * (mla_elems_per_token_layer(kv_lora_rank, qk_rope_dim) * elem_bytes + scale_bytes)


def mha_elems_per_token_layer(n_kv_heads: int, head_dim: int) -> int:
    return 2 * n_kv_heads * head_dim


def mha_bytes_per_token(n_layers: int, n_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return n_layers * mha_elems_per_token_layer(n_kv_heads, head_dim) * elem_bytes


def pool_bytes(num_blocks: int, block_size: int, kv_lora_rank: int, qk_rope_dim: int,
               elem_bytes: int) -> int:
    """Bytes of a paged pool of ``num_blocks`` blocks of ``block_size`` rows."""
    return num_blocks * block_size * mla_elems_per_token_layer(kv_lora_rank, qk_rope_dim) * elem_bytes
