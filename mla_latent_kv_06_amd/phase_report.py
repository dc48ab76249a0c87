"""Where the bf16 split-KV kernel's cycles go, per phase.

    python -m mla_latent_kv_06_amd.phase_report [--batch 64] [--ctx 8192] [--runs 6] [--json]

Runs the decode's split-KV pass (absorbed queries first, outside the timed
launches) on a synthetic uniform batch -- V3 head shape, bf16 paged cache of
`ctx` tokens per sequence, contiguous block tables -- with libmla_phases.so,
the instrumented build of the library (include/mla_debug.h), and prints each
wave's lap timers averaged over the working waves and launches: schedule walk,
first landing, first half-tile, the steady-state half-tiles split into barrier
wait / score chain / value chain, the last half-tiles, the vote and the
epilogue.  The instrumented kernel runs slightly slower than libmla.so's.

The library is chosen when the binding is imported, so this runs as its own
process (MLA_LIBRARY is set here before the import).
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
PHASES_LIB = os.path.join(PKG, "libmla_phases.so")
PHASE_WORDS = 16384
LAPS = [(8, "schedule walk"), (9, "first landing"), (10, "first half-tile"),
        (0, "steady: barrier wait"), (1, "steady: score chain"), (2, "steady: value chain"),
        (12, "last half-tiles"), (13, "vote"), (14, "epilogue")]


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--batch", type=int, default=64)
    ap.add_argument("--ctx", type=int, default=8192)
    ap.add_argument("--runs", type=int, default=6, help="timed split-KV launches (after 2 warm-ups)")
    ap.add_argument("--json", action="store_true", help="also print one JSON line")
    args = ap.parse_args(argv)
    if not os.path.exists(PHASES_LIB):
        raise SystemExit(f"{PHASES_LIB} not built; run `python -m mla_latent_kv_06_amd.build`")
    os.environ["MLA_LIBRARY"] = PHASES_LIB
    import torch
    if "mla_latent_kv_06_amd.binding" in sys.modules:
        raise SystemExit("the binding is already loaded in this process; run phase_report on its own")
    from mla_latent_kv_06_amd import binding as b
    if not torch.cuda.is_available():
        raise SystemExit("phase_report needs a GPU")
    lib = b.lib()
    lib.mla_debug_phase_stamps.restype = ctypes.c_int
    lib.mla_debug_phase_stamps.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    host = np.zeros(PHASE_WORDS, dtype=np.uint32)

    def read_stamps():
        st = lib.mla_debug_phase_stamps(host.ctypes.data, host.nbytes)
        if st != 0:
            raise RuntimeError(f"mla_debug_phase_stamps: status {st}")
        return host.reshape(256, 4, 16).astype(np.int64).copy()

    B, L, H = args.batch, args.ctx, 128
    if L % 64 or B < 1 or L < 64:
        raise SystemExit("ctx must be a positive multiple of 64")
    dev = torch.device("cuda:0")
    dims = b.Dims.make(H, 512, 64, 128, 128, 64, "bf16", "bf16")
    g = torch.Generator(device=dev).manual_seed(1)
    nblk = B * L // 64
    pool = (torch.randn((nblk, 64, 576), generator=g, device=dev) * 0.5).to(torch.bfloat16)
    bt = torch.arange(nblk, dtype=torch.int32, device=dev).reshape(B, L // 64)
    sl = torch.full((B,), L, dtype=torch.int32, device=dev)
    qn = torch.randn((B, 1, H, 128), generator=g, device=dev).to(torch.bfloat16)
    qp = torch.randn((B, 1, H, 64), generator=g, device=dev).to(torch.bfloat16)
    wuk = (torch.randn((H, 128, 512), generator=g, device=dev) * 0.05).to(torch.bfloat16)
    wuv = (torch.randn((H, 128, 512), generator=g, device=dev) * 0.05).to(torch.bfloat16)
    ws = torch.empty(b.decode_workspace_size(dims, B, 1, 0), dtype=torch.uint8, device=dev)
    common = (dims, qn, qp, wuk, wuv, pool, None, bt, sl)
    b.decode(*common, workspace=ws, stages=b.STAGE_ABSORB_Q)
    ms, acc = [], None
    for i in range(args.runs + 2):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.decode(*common, workspace=ws, stages=b.STAGE_SPLIT_KV)
        e1.record()
        torch.cuda.synchronize()
        d = read_stamps()
        if i < 2:
            continue
        ms.append(e0.elapsed_time(e1))
        live = d[:, :, 5] > 0                 # waves that processed a piece
        if acc is None:
            acc = {"waves": [], "span_us": []}
        w = d[live]
        acc["waves"].append(w)
        rt0, rt1 = w[:, 6], w[:, 7]
        base = rt0.min()
        acc["span_us"].append(float(((rt1 - base) % (1 << 32)).max()) * 0.01)
    waves = np.concatenate(acc["waves"])
    total = waves[:, 4].astype(np.float64)
    wave_us = ((waves[:, 7] - waves[:, 6]) % (1 << 32)) * 0.01
    clock = float((total / np.maximum(wave_us, 1e-9)).mean()) / 1e3
    n_half = waves[:, 3].astype(np.float64)
    lap_sum = waves[:, [0, 1, 2, 8, 9, 10, 12, 13, 14]].sum(1)
    assert np.all(lap_sum == waves[:, 4]), "laps do not add up to the wave's cycles"
    out = {"workload": f"bf16 batch {B} x {L} tokens, 128 heads, balanced schedule",
           "launches": len(ms), "event_us": float(np.median(ms)) * 1e3,
           "body_span_us": float(np.median(acc["span_us"])), "clock_ghz": clock,
           "wave_cycles": float(total.mean()), "steady_half_tiles_per_wave": float(n_half.mean()),
           "laps": {}}
    print(f"{out['workload']}: {len(ms)} split-KV launches, median {out['event_us']:.1f} us between "
          f"events, kernel body {out['body_span_us']:.1f} us (first wave start to last wave end), "
          f"shader clock {clock:.2f} GHz")
    print(f"per wave: {total.mean():.0f} cycles, {n_half.mean():.0f} steady-state half-tiles")
    print(f"{'phase':26s} {'cycles/wave':>12s} {'share':>7s} {'per half-tile':>14s}")
    for k, name in LAPS:
        c = waves[:, k].astype(np.float64)
        per = (c / np.maximum(n_half, 1)).mean() if k in (0, 1, 2) else float("nan")
        out["laps"][name] = {"cycles": float(c.mean()), "share": float(c.mean() / total.mean()),
                             "per_half_tile": None if k not in (0, 1, 2) else float(per)}
        per_s = f"{per:14.0f}" if k in (0, 1, 2) else " " * 14
        print(f"{name:26s} {c.mean():12.0f} {c.mean() / total.mean():7.3f} {per_s}")
    if args.json:
        print(json.dumps(out))
    return out


if __name__ == "__main__":
    main()
