"""Benchmark: absorbed-MLA decode tokens/s + latent-cache HBM GB/s on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--layers NL] [--splits S] [--no-cpu-baseline] [--cpu-tokens N]
                    [--query-path] [--report FILE]
    python bench.py --prefill v3_prefill_b2_8k_bf16 [--steps K] [--warmup W]

One step = the whole hot path for one layer over one batch: the cache append
of the new tokens (wkv_a projection, RMSNorm, RoPE, paged write; workloads
that define one) followed by the absorbed decode (q absorption, split-KV
attention over the paged latent cache, log-sum-exp combine, W_UV) -- one
mla_decode_step call when the workload appends, called stage by stage so
that HIP events bracket the split-KV launch.  Steps rotate over NL
independent layer copies (own pool, weights, queries) so the working set is
far larger than the 256 MB last-level cache; inputs are resident in HBM before
timing starts.  Prints ONE JSON line on stdout; details go to stderr.

Default workload: DeepSeek-V3 head shape (128 heads, latent 512, rotary 64),
bf16, batch 64, every sequence 8192 tokens after the append, paged blocks of 64
with a randomly permuted block table.

--prefill WORKLOAD times the prefill instead: one step = mla_prefill over every
prompt token of the batch for one layer (gather, K/V rebuild, causal
attention); its JSON line reports prompt tokens/s and the attention kernel
against the bf16 MFMA peak.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

METRIC = "MLA decode tokens/s + latent-cache HBM GB/s (% of peak) at bs64, ctx 8k"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
EVENT_STRIDE = 3               # timed steps per kernel-event sample
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ("decode_mfma.hip", "common.hpp", "internal.hpp")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "split_kv_ring_kernel_v3_b64_ctx8k_bf16_hbm_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class KernelEvent:
    """A HIP event for timing kernels inside the timed loop, created with
    hipEventDisableSystemFence: recording it does not write back and
    invalidate the caches.  (A default event's system-scope release flushes
    the L2's dirty lines when it is recorded: after a kernel that wrote tens
    of MB, such as the split-KV partials, that puts several microseconds
    between the kernel and the next one.)  Elapsed times are read after a
    device synchronisation, as with any event."""

    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        if KernelEvent._hip is None:
            # the HIP runtime torch has already loaded (same soname)
            KernelEvent._hip = ctypes.CDLL("libamdhip64.so.7")
        self._ct = ctypes
        self.ev = ctypes.c_void_p()
        self._check(KernelEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.ev),
                                                             ctypes.c_uint(self.DISABLE_SYSTEM_FENCE)))

    @staticmethod
    def _check(err):
        if err != 0:
            raise RuntimeError(f"HIP event call failed with error {err}")

    def record(self, stream):
        self._check(KernelEvent._hip.hipEventRecord(self.ev, self._ct.c_void_p(stream.cuda_stream)))

    def elapsed_time(self, end):
        ms = self._ct.c_float()
        self._check(KernelEvent._hip.hipEventElapsedTime(self._ct.byref(ms), self.ev, end.ev))
        return ms.value

    def __del__(self):
        if self._hip is not None and self.ev:
            self._hip.hipEventDestroy(self.ev)


def kernel_source_digest():
    """First 16 hex digits of sha256 over the split-KV kernel's source files."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "mla_latent_kv_06_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


PREFILL_SOURCES = ("prefill.hip", "prefill.hpp", "common.hpp", "internal.hpp")
PREFILL_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "prefill_attn_kernel_v3_b2_8k_bf16_hbm_traffic.txt")


def prefill_traffic(workload):
    """HBM bytes per prefill attention launch from the committed counter
    summary, or None when it was taken on other sources or another workload."""
    import hashlib
    import re
    if workload != "v3_prefill_b2_8k_bf16" or not os.path.exists(PREFILL_TRAFFIC_PROFILE):
        return None
    h = hashlib.sha256()
    for f in PREFILL_SOURCES:
        with open(os.path.join(ROOT, "mla_latent_kv_06_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    text = open(PREFILL_TRAFFIC_PROFILE).read()
    d = re.search(r"first 16 hex\):\s*([0-9a-f]{16})", text)
    t = re.search(r"total HBM traffic per launch\s*=\s*([0-9,]+) B", text)
    if not d or not t or d.group(1) != h.hexdigest()[:16]:
        return None
    return int(t.group(1).replace(",", ""))


def profiled_traffic(workload):
    """HBM bytes per split-KV launch from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE, copy-calibrated), or None when that summary
    was taken on other kernel sources or another workload."""
    import re
    if workload != "v3_b64_ctx8k_paged_bf16" or not os.path.exists(TRAFFIC_PROFILE):
        return None
    text = open(TRAFFIC_PROFILE).read()
    d = re.search(r"first 16 hex\):\s*([0-9a-f]{16})", text)
    t = re.search(r"total HBM traffic per launch\s*=\s*([0-9,]+) B", text)
    if not d or not t or d.group(1) != kernel_source_digest():
        return None
    return int(t.group(1).replace(",", ""))


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="v3_b64_ctx8k_paged_bf16")
    p.add_argument("--layers", type=int, default=8)
    p.add_argument("--splits", type=int, default=None,
                   help="split-KV partitions per query row (default: the workload's own; "
                        "0 = the library's balanced schedule)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--query-path", action="store_true",
                   help="add the query path (W_DQ, norm, W_UQ / W_QR, RoPE) to each step")
    p.add_argument("--prefill", default=None, metavar="WORKLOAD",
                   help="time the prefill (gather, K/V rebuild, causal attention) on a "
                        "prefill workload, e.g. v3_prefill_b2_8k_bf16, instead of the decode step")
    p.add_argument("--cpu-tokens", type=int, default=262144,
                   help="CPU-baseline sample: first sequences of layer 0 up to this many cached tokens")
    p.add_argument("--output-study", action="store_true",
                   help="instead: time the output side of the layer at the workload's rows: "
                        "u = W_O o (W_O [d_model, H V]) against the merged-weight form "
                        "u = (W_O W_UV) o_lat ([d_model, H d_c]), and the decode through W_O")
    p.add_argument("--report", default=None)
    p.add_argument("--copy-bytes", type=int, default=0,
                   help="instead: copy a buffer of this many bytes 5 times (calibrates "
                        "hardware byte counters against a kernel of known traffic)")
    return p.parse_args()


class Layer:
    """One layer's device tensors."""

    def __init__(self, wl, li, dims, dev, torch, synth, b, query_path=False):
        seed = 1000 + li
        B, H = wl.batch, wl.n_heads
        bf = torch.bfloat16

        def up(x):
            return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev).to(bf)

        self.q_nope = up(synth.q_nope(wl, seed))
        self.q_pe = up(synth.q_pe(wl, seed))
        self.w_uk = up(synth.w_uk(wl, seed))
        self.w_uv = up(synth.w_uv(wl, seed))
        self.w_kv_a = up(synth.w_kv_a(wl, seed))
        self.gamma = torch.ones(wl.kv_lora_rank, dtype=bf, device=dev)
        self.h = up(synth.hidden(wl, seed=seed))
        if query_path:                   # query compression weights (d_q = 1536)
            ql = synth.Q_LORA_RANK_V3
            self.w_dq = up(synth.w_dq(wl, ql, seed))
            self.q_gamma = up(synth.q_norm_gamma(ql, seed))
            self.w_uq = up(synth.w_uq(wl, ql, seed))
            self.w_qr = up(synth.w_qr(wl, ql, seed))
        cached = synth.cached_lengths(wl, seed)
        seq_lens = (cached + wl.q_len).astype(np.int32)
        table, nblk = synth.block_tables(seq_lens, wl.block_size, wl.paged, seed)
        self.seq_lens_host = seq_lens
        self.table_host = table
        self.block_table = torch.from_numpy(table).to(dev)
        self.seq_lens = torch.from_numpy(seq_lens).to(dev)
        self.start_pos = torch.from_numpy(cached.astype(np.int32)).to(dev)
        # cache rows: N(0,1) drawn on the device (unit RMS in expectation);
        # decode time does not depend on the values.  fp8: e4m3 codes of the
        # draw times 64 (inside the +-448 range) with a per-token scale of 1/64.
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        fp8 = wl.cache_dtype == "fp8"
        self.pool = torch.empty((nblk, wl.block_size, wl.row_width),
                                dtype=torch.uint8 if fp8 else bf, device=dev)
        flat = self.pool.view(-1, wl.row_width)
        step = 1 << 16
        for i in range(0, flat.shape[0], step):
            x = torch.randn(flat[i:i + step].shape, generator=g, device=dev, dtype=torch.float32)
            if fp8:
                flat[i:i + step] = (x * 64.0).to(torch.float8_e4m3fn).view(torch.uint8)
            else:
                flat[i:i + step] = x.to(bf)
        self.scale = (torch.full((nblk, wl.block_size), 1.0 / 64.0, dtype=torch.float32, device=dev)
                      if fp8 else None)
        self.out = torch.empty((B, wl.q_len, H, wl.v_head_dim), dtype=bf, device=dev)
        self.lse = torch.empty((B, wl.q_len, H), dtype=torch.float32, device=dev)


def graph_step_ms(torch, dev, stream, step, layers, K):
    """The step captured once per layer into a HIP graph (every library call
    only enqueues kernels), then K replays timed with events; ms per step."""
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step(layers[0])                      # an eager run on the capturing stream
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for L in layers:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            step(L)
        graphs.append(g)
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for i in range(K):
        graphs[i % len(graphs)].replay()
    g1.record(stream)
    torch.cuda.synchronize()
    return g0.elapsed_time(g1) / K


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library runs the decode of one GPU's share; it has no cross-GPU path)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from mla_latent_kv_06_amd import synth
    from mla_latent_kv_06_amd import binding as b

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_bytes:
        n = args.copy_bytes // 16 * 16
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {n} bytes 5 times")
        return
    if args.prefill:
        prefill_main(args, torch, synth, b, dev)
        return
    if args.output_study:
        output_study(args, torch, synth, b, dev)
        return
    wl = synth.WORKLOADS[args.workload]
    if wl.act_dtype != "bf16" or wl.cache_dtype not in ("bf16", "fp8"):
        raise SystemExit("bench.py times the bf16-activation workloads (bf16 or fp8 cache)")
    dims = b.Dims.from_workload(wl)
    B, Sq, H = wl.batch, wl.q_len, wl.n_heads
    splits = wl.num_splits if args.splits is None else args.splits

    t_setup = time.time()
    layers = [Layer(wl, li, dims, dev, torch, synth, b, args.query_path) for li in range(args.layers)]
    ql = synth.Q_LORA_RANK_V3 if args.query_path else 0
    ws_q = (torch.empty(max(1, b.query_workspace_size(dims, B, Sq, wl.d_model, ql)), dtype=torch.uint8,
                        device=dev) if args.query_path else None)
    ws_dec = torch.empty(b.decode_workspace_size(dims, B, Sq, splits), dtype=torch.uint8, device=dev)
    ws_step = (torch.empty(b.step_workspace_size(dims, B, Sq, wl.d_model, splits), dtype=torch.uint8,
                           device=dev) if wl.append else None)
    torch.cuda.synchronize()
    log(f"setup {time.time() - t_setup:.1f}s: {args.layers} layers, "
        f"pool {layers[0].pool.numel() * layers[0].pool.element_size() / 1e6:.1f} MB each, "
        f"splits {splits if splits else 'balanced'}")

    stream = torch.cuda.current_stream(dev)

    def step(L, ev=None, qev=None):
        if args.query_path:              # the decode's queries from the layer input
            if qev is not None:
                qev[0].record(stream)
            b.query_project(dims, L.h, L.w_dq, L.q_gamma, L.w_uq, L.w_qr, L.start_pos,
                            rms_eps=1e-6, rope_base=10000.0, q_nope=L.q_nope, q_pe=L.q_pe,
                            workspace=ws_q)
            if qev is not None:
                qev[1].record(stream)
        common = (dims, L.q_nope, L.q_pe, L.w_uk, L.w_uv, L.pool, L.scale, L.block_table,
                  L.seq_lens)
        if wl.append:
            # mla_decode_step: the append of the step's tokens and the decode,
            # its stages called in turn so that events bracket the split-KV pass
            def stp(stages):
                b.decode_step(dims, L.h, L.w_kv_a, L.gamma, L.start_pos, L.q_nope, L.q_pe, L.w_uk,
                              L.w_uv, L.pool, L.scale, L.block_table, L.seq_lens, num_splits=splits,
                              rms_eps=1e-6, rope_base=10000.0, out=L.out, lse=L.lse,
                              workspace=ws_step, stages=stages)
            stp(b.STEP_PROJECT | b.STEP_FINALIZE_ABSORB)
            if ev is not None:
                ev[0].record(stream)
            stp(b.STEP_SPLIT_KV)
            if ev is not None:
                ev[1].record(stream)
            stp(b.STEP_COMBINE)
            return
        b.decode(*common, num_splits=splits, out=L.out, lse=L.lse, workspace=ws_dec,
                 stages=b.STAGE_ABSORB_Q)
        if ev is not None:
            ev[0].record(stream)
        b.decode(*common, num_splits=splits, out=L.out, lse=L.lse, workspace=ws_dec,
                 stages=b.STAGE_SPLIT_KV)
        if ev is not None:
            ev[1].record(stream)
        b.decode(*common, num_splits=splits, out=L.out, lse=L.lse, workspace=ws_dec,
                 stages=b.STAGE_COMBINE)

    for i in range(args.warmup):
        step(layers[i % len(layers)])
    torch.cuda.synchronize()

    K = args.steps
    # Kernel events on every EVENT_STRIDE-th step of the timed region: a
    # recorded event is a queue packet of its own that holds the next kernel
    # back by about 5 us on this GPU, so instrumenting every step would add
    # ~10 us to each; the sampled steps are spread over the whole region.
    sampled = [i % EVENT_STRIDE == 0 for i in range(K)]
    qevs = [(KernelEvent(), KernelEvent()) if sampled[i] else None for i in range(K)] if args.query_path else []
    evs = [(KernelEvent(), KernelEvent()) if sampled[i] else None for i in range(K)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    if torch.distributed.is_available() and torch.distributed.is_initialized():
        torch.distributed.barrier()
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(K):
        step(layers[i % len(layers)], evs[i], qevs[i] if args.query_path else None)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / K
    k_ms = np.array([e[0].elapsed_time(e[1]) for e in evs if e is not None])
    q_ms = np.array([e[0].elapsed_time(e[1]) for e in qevs if e is not None]) if args.query_path else None
    k_avg_s = float(k_ms.mean()) / 1e3

    # Reference for the roofline on this GPU: libmla_probe's streaming read
    # (16-byte loads, 512 workgroups, each over one contiguous range) of a
    # 1 GiB buffer (four times the 256 MB last-level cache, whatever the
    # workload's pool size); median of 12 reads after 2 warm-ups, outside the
    # timed region.
    # (A failure here costs only this reference: stream_read_gbs is then null.)
    stream_gbs = None
    try:
        probe_buf = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        sink = b.probe_read(probe_buf)
        s_ms = []
        for i in range(14):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            b.probe_read(probe_buf, sink)
            e1.record(stream)
            torch.cuda.synchronize()
            s_ms.append(e0.elapsed_time(e1))
        del probe_buf
        probe_bytes = 1 << 30
        stream_gbs = probe_bytes / (float(np.median(s_ms[2:])) / 1e3) / 1e9
    except (ImportError, OSError, RuntimeError) as exc:
        log(f"streaming-read probe unavailable: {exc}")

    # The same step replayed from HIP graphs (one per layer, captured after
    # the timed region; every library call only enqueues kernels): one graph
    # launch per step instead of one host call per stage, timed over K
    # replays.  Reported beside `value`, which stays the eager step's.
    graph_ms = None
    try:
        graph_ms = graph_step_ms(torch, dev, stream, step, layers, K) if not args.query_path else None
    except RuntimeError as exc:       # reported as missing, never fatal to the bench line
        log(f"graph replay unavailable: {exc}")

    tokens_per_step = B * Sq
    value = tokens_per_step / (ms_step / 1e3)
    # algorithmic work of the split-KV kernel: every cache token's 576-element
    # row (plus its fp8 scale) is read once; 2*H*(576+512) flops per visible
    # token and query row
    seq_lens = layers[0].seq_lens_host.astype(np.int64)
    row_bytes = wl.row_width * (1 if wl.cache_dtype == "fp8" else 2) + (4 if wl.cache_dtype == "fp8" else 0)
    cache_bytes = int(seq_lens.sum()) * row_bytes
    flops = sum(int(L - Sq + s + 1) for L in seq_lens for s in range(Sq)) * 2 * H * (wl.row_width + wl.kv_lora_rank)
    achieved = cache_bytes / k_avg_s / 1e9
    tflops = flops / k_avg_s / 1e12
    # matrix-core peak: both products run on the bf16 matrix cores
    mfma_peak = BF16_PEAK_TFLOPS
    mfma_bound = flops / cache_bytes > mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    step_gbs = cache_bytes / (ms_step / 1e3) / 1e9
    log(f"step {ms_step * 1e3:.1f} us  ({value:.4g} tok/s)  split-KV kernel {k_avg_s * 1e6:.1f} us "
        f"(p10 {np.percentile(k_ms, 10) * 1e3:.1f} / p90 {np.percentile(k_ms, 90) * 1e3:.1f})")
    log(f"cache {cache_bytes / 1e6:.1f} MB: kernel {achieved:.0f} GB/s ({achieved / HBM_PEAK_GBS:.1%} of 8 TB/s), "
        f"step {step_gbs:.0f} GB/s; kernel {flops / k_avg_s / 1e12:.0f} TFLOP/s "
        f"({flops / k_avg_s / 1e12 / mfma_peak:.1%} of the {mfma_peak:.0f} TFLOP/s MFMA peak)")
    if graph_ms is not None:
        log(f"step replayed from a HIP graph: {graph_ms * 1e3:.1f} us ({tokens_per_step / (graph_ms / 1e3):.4g} tok/s)")
    if stream_gbs is not None:
        log(f"streaming read of 1 GiB (libmla_probe) on this GPU: {stream_gbs:.0f} GB/s; the split-KV kernel "
            f"reaches {achieved / stream_gbs:.1%} of it")

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "batch": B, "ctx": int(seq_lens.max()), "q_len": Sq,
            "heads": H, "kv_lora_rank": wl.kv_lora_rank, "rope_dim": wl.qk_rope_dim,
            "block_size": wl.block_size, "paged": wl.paged,
            "num_splits": splits if splits else "balanced",
            "layers_rotated": args.layers,
            "cache_dtype": wl.cache_dtype,
            "step": (("cache append of %d token(s)/seq + " % Sq if wl.append else "")
                     + ("query path + " if args.query_path else "") + "absorbed decode, one layer"),
            "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "bound": "mfma" if mfma_bound else "hbm",
            "kernel": "split_kv_ring_kernel" if wl.cache_dtype == "bf16" else "split_kv_kernel<fp8>",
            "achieved": round(tflops if mfma_bound else achieved, 1),
            "peak": round(mfma_peak, 1) if mfma_bound else HBM_PEAK_GBS,
            "unit": "TFLOP/s" if mfma_bound else "GB/s",
            "frac": round(tflops / mfma_peak if mfma_bound else achieved / HBM_PEAK_GBS, 4),
            "hbm_gbs": round(achieved, 1),
            "traffic": profiled_traffic(wl.name), "traffic_unit": "bytes per launch",
            "algorithmic_bytes": cache_bytes,
            "avg_launch_us": round(k_avg_s * 1e6, 2),
            "launches_timed": int(len(k_ms)),
            "mfma_tflops": round(flops / k_avg_s / 1e12, 1),
            "mfma_frac": round(flops / k_avg_s / 1e12 / mfma_peak, 4),
            "stream_read_gbs": None if stream_gbs is None else round(stream_gbs, 1),
            "frac_of_stream_read": None if stream_gbs is None else round(achieved / stream_gbs, 4),
        },
        "cpu_baseline": None,
    }
    if graph_ms is not None:
        result["graph"] = {"ms_per_step": round(graph_ms, 5),
                           "tokens_per_s": round(tokens_per_step / (graph_ms / 1e3), 1),
                           "replays": K, "note": "the same step replayed from one HIP graph per layer"}
    if args.query_path:
        # algorithmic bytes: the three weights, gamma, h and the two outputs
        ql, d = synth.Q_LORA_RANK_V3, wl.d_model
        hq = H * (wl.qk_nope_dim + wl.qk_rope_dim)
        q_bytes = 2 * (ql * d + ql + hq * ql + B * Sq * d + B * Sq * hq)
        q_s = float(q_ms.mean()) / 1e3
        result["config"]["q_lora_rank"] = ql
        result["query_path"] = {
            "avg_us": round(q_s * 1e6, 2), "algorithmic_bytes": q_bytes,
            "gbs": round(q_bytes / q_s / 1e9, 1), "frac": round(q_bytes / q_s / 1e9 / HBM_PEAK_GBS, 4),
        }
        log(f"query path {q_s * 1e6:.1f} us: {q_bytes / 1e6:.1f} MB -> {q_bytes / q_s / 1e9:.0f} GB/s "
            f"({q_bytes / q_s / 1e9 / HBM_PEAK_GBS:.1%} of 8 TB/s)")

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, wl, layers[0], torch)

    print(json.dumps(result), flush=True)
    if args.report:
        with open(args.report, "w") as f:
            json.dump(result, f, indent=1)


def output_study(args, torch, synth, b, dev):
    """The layer's output side at the workload's rows R = batch * q_len:
      factored  u = W_O o,           W_O   [d_model, H V]   (mla_output_project)
      merged    u = (W_O W_UV) o_lat, W_OV [d_model, H d_c] (the same GEMM, K = H d_c)
    and one decode through W_O (mla_decode_output) against the decode alone.
    Weights are random bf16 (timing does not depend on values); two W_O
    copies alternate so that the 235 MB weight does not stay in the 256 MB
    last-level cache.  One JSON line."""
    wl = synth.WORKLOADS[args.workload]
    R, H, V, dc, d = wl.batch * wl.q_len, wl.n_heads, wl.v_head_dim, wl.kv_lora_rank, wl.d_model
    bf = torch.bfloat16
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    rnd = lambda *shape: (torch.randn(*shape, generator=g, device=dev, dtype=torch.float32) * 0.01).to(bf)
    w_o = [rnd(d, H * V) for _ in range(2)]
    w_ov = rnd(d, H * dc)
    o = rnd(R, H * V)
    lat = rnd(R, H * dc)
    stream = torch.cuda.current_stream(dev)

    def timed(fn, K):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for i in range(K):
            fn(i)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / K / 1e3

    K = max(4, args.steps)
    ws = torch.empty(max(b.output_workspace_size(R, H * dc, d), b.output_workspace_size(R, H * V, d)),
                     dtype=torch.uint8, device=dev)
    outb = torch.empty(R, d, dtype=bf, device=dev)
    fact_s = timed(lambda i: b.output_project(o, w_o[i & 1], out=outb, workspace=ws), K)
    merged_s = timed(lambda i: b.output_project(lat, w_ov, out=outb, workspace=ws), max(4, K // 4))
    fact_bytes = d * H * V * 2 + R * H * V * 2 + R * d * 2
    merged_bytes = d * H * dc * 2 + R * H * dc * 2 + R * d * 2
    # the decode alone against the decode through W_O, on one layer
    layer = Layer(wl, 0, b.Dims.from_workload(wl), dev, torch, synth, b)
    dims = b.Dims.from_workload(wl)
    common = (dims, layer.q_nope, layer.q_pe, layer.w_uk, layer.w_uv, layer.pool, layer.scale,
              layer.block_table, layer.seq_lens)
    ws_d = torch.empty(b.decode_output_workspace_size(dims, wl.batch, wl.q_len, 0, d), dtype=torch.uint8,
                       device=dev)
    u = torch.empty(wl.batch, wl.q_len, d, dtype=bf, device=dev)
    dec_s = timed(lambda i: b.decode(*common, out=layer.out, lse=layer.lse, workspace=ws_d), K)
    dec_out_s = timed(lambda i: b.decode_output(*common, w_o[i & 1], u=u, lse=layer.lse, workspace=ws_d), K)
    res = {
        "study": "output side", "workload": wl.name, "rows": R, "d_model": d,
        "factored_w_o": {"k": H * V, "bytes": fact_bytes, "us": round(fact_s * 1e6, 2),
                         "gbs": round(fact_bytes / fact_s / 1e9, 1)},
        "merged_w_ov": {"k": H * dc, "bytes": merged_bytes, "us": round(merged_s * 1e6, 2),
                        "gbs": round(merged_bytes / merged_s / 1e9, 1)},
        "decode_us": round(dec_s * 1e6, 2), "decode_through_w_o_us": round(dec_out_s * 1e6, 2),
    }
    log(f"W_O GEMM {fact_s * 1e6:.1f} us ({fact_bytes / 1e6:.0f} MB, {fact_bytes / fact_s / 1e9:.0f} GB/s); "
        f"merged W_OV GEMM {merged_s * 1e6:.1f} us ({merged_bytes / 1e6:.0f} MB, "
        f"{merged_bytes / merged_s / 1e9:.0f} GB/s); decode {dec_s * 1e6:.1f} us, "
        f"decode through W_O {dec_out_s * 1e6:.1f} us")
    print(json.dumps(res), flush=True)


class PrefillLayer:
    """One layer's prefill inputs: queries of every prompt token, the absorbed
    weights, and a paged pool holding the prompt's cache rows."""

    def __init__(self, wl, li, dev, torch, synth):
        seed = 2000 + li
        bf = torch.bfloat16

        def up(x):
            return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev).to(bf)

        self.q_nope = up(synth.q_nope(wl, seed))
        self.q_pe = up(synth.q_pe(wl, seed))
        self.w_uk = up(synth.w_uk(wl, seed))
        self.w_uv = up(synth.w_uv(wl, seed))
        seq_lens = synth.seq_lens(wl, seed)
        table, nblk = synth.block_tables(seq_lens, wl.block_size, wl.paged, seed)
        self.seq_lens_host = seq_lens
        self.table_host = table
        self.block_table = torch.from_numpy(table).to(dev)
        self.seq_lens = torch.from_numpy(seq_lens).to(dev)
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        fp8 = wl.cache_dtype == "fp8"
        x = torch.randn((nblk, wl.block_size, wl.row_width), generator=g, device=dev)
        self.pool = (x * 64.0).to(torch.float8_e4m3fn).view(torch.uint8) if fp8 else x.to(bf)
        self.scale = (torch.full((nblk, wl.block_size), 1.0 / 64.0, dtype=torch.float32, device=dev)
                      if fp8 else None)
        self.out = torch.empty((wl.batch, wl.q_len, wl.n_heads, wl.v_head_dim), dtype=bf, device=dev)
        self.lse = torch.empty((wl.batch, wl.q_len, wl.n_heads), dtype=torch.float32, device=dev)


def prefill_main(args, torch, synth, b, dev):
    """One step = mla_prefill over every prompt of the batch for one layer
    (gather, K/V rebuild, causal attention), inputs resident in HBM; layers
    rotate as for the decode.  Roofline: the attention kernel against the
    bf16 MFMA peak, 2 H (N + R + V) flops per visible (query, key) pair."""
    wl = synth.PREFILL_WORKLOADS[args.prefill]
    dims = b.Dims.from_workload(wl)
    B, Sq, H = wl.batch, wl.q_len, wl.n_heads
    n_layers = min(args.layers, 2)
    t_setup = time.time()
    layers = [PrefillLayer(wl, li, dev, torch, synth) for li in range(n_layers)]
    ws = torch.empty(b.prefill_workspace_size(dims, B, Sq, layers[0].table_host.shape[1]),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"setup {time.time() - t_setup:.1f}s: {n_layers} layers, workspace {ws.numel() / 1e9:.2f} GB")
    stream = torch.cuda.current_stream(dev)

    def step(L, ev=None):
        common = (dims, L.q_nope, L.q_pe, L.w_uk, L.w_uv, L.pool, L.scale, L.block_table, L.seq_lens)
        kw = dict(out=L.out, lse=L.lse, workspace=ws)
        if ev is not None:
            ev[0].record(stream)
        b.prefill(*common, stages=b.PREFILL_GATHER, **kw)
        if ev is not None:
            ev[1].record(stream)
        b.prefill(*common, stages=b.PREFILL_DECOMPRESS, **kw)
        if ev is not None:
            ev[2].record(stream)
        b.prefill(*common, stages=b.PREFILL_ATTEND, **kw)
        if ev is not None:
            ev[3].record(stream)

    for i in range(args.warmup):
        step(layers[i % n_layers])
    torch.cuda.synchronize()
    K = args.steps
    evs = [[KernelEvent() for _ in range(4)] for _ in range(K)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(K):
        step(layers[i % n_layers], evs[i])
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / K
    span = lambda j: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) / 1e3
    g_s, d_s, a_s = span(0), span(1), span(2)

    seq_lens = layers[0].seq_lens_host.astype(np.int64)
    pairs = sum(int(min(L, L - Sq + s + 1)) for L in seq_lens for s in range(Sq) if L - Sq + s + 1 > 0)
    attn_flops = pairs * 2 * H * (wl.qk_nope_dim + wl.qk_rope_dim + wl.v_head_dim)
    dec_flops = int(seq_lens.sum()) * 2 * H * (wl.qk_nope_dim + wl.v_head_dim) * wl.kv_lora_rank
    tokens = B * Sq
    value = tokens / (ms_step / 1e3)
    a_tf, d_tf = attn_flops / a_s / 1e12, dec_flops / d_s / 1e12
    log(f"step {ms_step:.3f} ms ({value:.4g} prompt tok/s): gather {g_s * 1e6:.0f} us, "
        f"rebuild {d_s * 1e6:.0f} us ({d_tf:.0f} TFLOP/s), attention {a_s * 1e6:.0f} us "
        f"({a_tf:.0f} TFLOP/s, {a_tf / BF16_PEAK_TFLOPS:.1%} of {BF16_PEAK_TFLOPS:.0f})")
    result = {
        "metric": "MLA prefill tokens/s (decompressed form, causal, one layer)",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "batch": B, "prompt": Sq, "ctx": int(seq_lens.max()),
            "heads": H, "kv_lora_rank": wl.kv_lora_rank, "rope_dim": wl.qk_rope_dim,
            "block_size": wl.block_size, "paged": wl.paged, "cache_dtype": wl.cache_dtype,
            "layers_rotated": n_layers,
            "step": "prefill of every prompt token (gather, K/V rebuild, causal attention), one layer",
            "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "bound": "mfma", "kernel": "prefill_attn_kernel",
            "achieved": round(a_tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(a_tf / BF16_PEAK_TFLOPS, 4), "traffic": prefill_traffic(wl.name),
            "traffic_unit": "bytes per launch",
            "algorithmic_flops": attn_flops, "avg_launch_us": round(a_s * 1e6, 2),
        },
        "rebuild": {"kernel": "prefill_decompress_kernel", "avg_us": round(d_s * 1e6, 2),
                    "algorithmic_flops": dec_flops, "tflops": round(d_tf, 1),
                    "frac": round(d_tf / BF16_PEAK_TFLOPS, 4)},
        "gather_us": round(g_s * 1e6, 2),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = prefill_cpu_baseline(wl, layers[0], torch)
    print(json.dumps(result), flush=True)
    if args.report:
        with open(args.report, "w") as f:
            json.dump(result, f, indent=1)


def prefill_cpu_baseline(wl, L, torch, n_q=8192, heads=tuple(range(16))):
    """The CPU oracle (naive float64 attention) on a bounded sample: the first
    n_q queries of prompt 0 (all of it at 8192) for 16 of the 128 heads, each
    query seeing its causal prefix; the rate is scaled to whole prompt tokens
    (all heads).  Also checks the GPU output on that sample."""
    import oracle
    from mla_latent_kv_06_amd import layout
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    torch.cuda.synchronize()
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    nb = (n_q + wl.block_size - 1) // wl.block_size
    ids = torch.from_numpy(L.table_host[0, :nb].astype(np.int64)).to(L.pool.device)
    blocks = layout.pool_rows(L.pool.index_select(0, ids), wl.cache_dtype)     # token rows
    if wl.cache_dtype == "fp8":
        rows64 = oracle.dequantize_rows_fp8(blocks.cpu().numpy(),
                                            L.scale.index_select(0, ids).reshape(-1).cpu().numpy())
    else:
        rows64 = f64(blocks)
    rows = oracle.gather_sequence(rows64, np.arange(nb), n_q, wl.block_size)
    hs = list(heads)
    qn = f64(L.q_nope[:1, :n_q])[:, :, hs]
    qp = f64(L.q_pe[:1, :n_q])[:, :, hs]
    wuk, wuv = f64(L.w_uk)[hs], f64(L.w_uv)[hs]
    t = time.time()
    ref, _ = oracle.decode_naive(qn, qp, wuk, wuv, [rows], n_q)
    dt = time.time() - t
    got = f64(L.out[:1, :n_q])[:, :, hs]
    err = float(np.max(np.abs(got - ref)))
    log(f"cpu oracle: {n_q} queries x {len(hs)} heads in {dt:.1f}s on {threads} threads; "
        f"GPU vs oracle max-abs {err:.2e}")
    return {"value": round(n_q * len(hs) / wl.n_heads / dt, 4), "unit": "tokens/s", "cores": threads,
            "host_cpus": os.cpu_count(),
            "kind": "oracle",
            "sample": f"first {n_q} of {wl.q_len} queries of prompt 0, heads {hs[0]}-{hs[-1]} of "
                      f"{wl.n_heads}, naive float64 attention, {dt:.1f}s; rate scaled to all heads",
            "gpu_vs_oracle_max_abs": err}


def cpu_baseline(args, wl, L, torch):
    """The CPU oracle (naive float64 decode) on a bounded sample of the same
    workload: the first sequences of layer 0 up to --cpu-tokens cached tokens, all heads, read back
    from the device.  Also checks the GPU output for those sequences."""
    import oracle
    from mla_latent_kv_06_amd import layout
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    n, tot = 0, 0
    while n < wl.batch and (n == 0 or tot + int(L.seq_lens_host[n]) <= args.cpu_tokens):
        tot += int(L.seq_lens_host[n])
        n += 1
    D = wl.row_width
    torch.cuda.synchronize()

    def f64(t):
        return t.float().cpu().numpy().astype(np.float64)

    def seq_rows(i):
        # this sequence's blocks only (gathered on the device), then the
        # oracle's own gather over a compact table
        nb = (int(L.seq_lens_host[i]) + wl.block_size - 1) // wl.block_size
        ids = torch.from_numpy(L.table_host[i, :nb].astype(np.int64)).to(L.pool.device)
        blocks = layout.pool_rows(L.pool.index_select(0, ids), wl.cache_dtype)  # token rows
        if wl.cache_dtype == "fp8":
            codes = blocks.cpu().numpy()
            sc = L.scale.index_select(0, ids).reshape(-1).cpu().numpy()
            rows64 = oracle.dequantize_rows_fp8(codes, sc)
        else:
            rows64 = f64(blocks)
        return oracle.gather_sequence(rows64, np.arange(nb), int(L.seq_lens_host[i]), wl.block_size)

    rows = [seq_rows(i) for i in range(n)]
    qn, qp = f64(L.q_nope[:n]), f64(L.q_pe[:n])
    wuk, wuv = f64(L.w_uk), f64(L.w_uv)
    t = time.time()
    ref, _ = oracle.decode_naive(qn, qp, wuk, wuv, rows, wl.q_len)
    dt = time.time() - t
    got = f64(L.out[:n])
    err = float(np.max(np.abs(got - ref)))
    log(f"cpu oracle: {n} sequences in {dt:.1f}s on {threads} threads; GPU vs oracle max-abs {err:.2e}")
    return {"value": round(n * wl.q_len / dt, 4), "unit": "tokens/s", "cores": threads,
            "host_cpus": os.cpu_count(), "kind": "oracle",
            "sample": f"{n} of {wl.batch} sequences ({tot} cached tokens, {wl.q_len} query "
                      f"row(s) each, all {wl.n_heads} heads), naive float64 decode, {dt:.1f}s",
            "gpu_vs_oracle_max_abs": err}


if __name__ == "__main__":
    main()
