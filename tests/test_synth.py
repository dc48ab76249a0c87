"""The seeded input generator: determinism, shapes, distributions."""

import numpy as np

from mla_latent_kv_06_amd import synth


def test_same_seed_same_bytes():
    wl = synth.WORKLOADS["v3_b64_ctx1k8k_paged_bf16"]
    for f in (synth.cached_lengths, synth.q_nope, synth.q_pe):
        assert np.array_equal(f(wl, 0), f(wl, 0))
    assert not np.array_equal(synth.q_nope(wl, 0), synth.q_nope(wl, 1))
    a = synth.cache_draws(wl, 3, 100)
    b = synth.cache_draws(wl, 3, 100)
    assert a.dtype == np.float32 and np.array_equal(a, b)
    # a sequence's rows do not depend on how many were drawn
    assert np.array_equal(synth.cache_draws(wl, 3, 40), a[:40])
    t1, n1 = synth.block_tables(synth.seq_lens(wl), 64, True, 0)
    t2, n2 = synth.block_tables(synth.seq_lens(wl), 64, True, 0)
    assert n1 == n2 and np.array_equal(t1, t2)


def test_workload_shapes_and_ranges():
    w = synth.WORKLOADS
    assert synth.seq_lens(w["tiny_f32"]).tolist() == [64]
    assert synth.seq_lens(w["v3_b1_ctx4k_bf16"]).tolist() == [4096]
    L2 = synth.seq_lens(w["v3_b64_ctx1k8k_paged_bf16"])
    assert len(L2) == 64 and L2.min() >= 1025 and L2.max() <= 8193
    assert synth.seq_lens(w["v3_b4_ctx128k_split32_bf16"]).tolist() == [131072] * 4
    L4 = synth.seq_lens(w["v3_b128_ctx8k32k_fp8_q2"])
    assert len(L4) == 128 and L4.min() >= 8192 and L4.max() <= 32768
    assert synth.seq_lens(w["v3_b64_ctx8k_paged_bf16"]).tolist() == [8192] * 64


def test_weight_scales():
    wl = synth.WORKLOADS["v3_b1_ctx4k_bf16"]
    assert abs(synth.w_uk(wl).std() * np.sqrt(512) - 1) < 0.01
    assert abs(synth.w_uv(wl).std() * np.sqrt(512) - 1) < 0.01
    assert abs(synth.w_kv_a(wl).std() * np.sqrt(7168) - 1) < 0.01


def test_prefill_workloads():
    for wl in synth.PREFILL_WORKLOADS.values():
        assert synth.seq_lens(wl).tolist() == [8192, 8192]        # fresh prompts
        assert wl.n_heads == 128 and wl.kv_lora_rank == 512 and wl.block_size == 64
