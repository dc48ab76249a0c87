"""Build libmla.so (gfx950) in-tree with hipcc.

    python -m mla_latent_kv_06_amd.build [--verbose]

Every .hip file under csrc/ is compiled to an object in _build/, then linked
into mla_latent_kv_06_amd/libmla.so.  The streaming-read probe (probe/, a
measurement yardstick, not part of the attention path) becomes
mla_latent_kv_06_amd/libmla_probe.so.  The same sources compiled with
-DMLA_PHASE_STAMPS (the split-KV kernel's phase timers, include/mla_debug.h)
become mla_latent_kv_06_amd/libmla_phases.so.  Always rebuilds (no staleness
check).
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmla.so")
PROBE_SRC = os.path.join(PKG, "probe", "read_probe.hip")
PROBE_LIB = os.path.join(PKG, "libmla_probe.so")
PHASES_LIB = os.path.join(PKG, "libmla_phases.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr)
    # the host pass does not know the gfx feature above; drop that one warning
    out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer for the C ABI's
# validation code (device code is built as usual: each sanitizer flag is
# restricted to the host pass).  The result loads only with clang's ASan
# runtime preloaded (see tests/test_abi_sanitized.py).
SAN_FLAGS = ["-g", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
SAN_LIB = os.path.join(BUILD, "san", "libmla_san.so")


def build_sanitized(verbose: bool = False) -> str:
    d = os.path.join(BUILD, "san")
    os.makedirs(d, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = [os.path.join(d, f[:-4] + ".o") for f in srcs]
    cmds = [[HIPCC, *FLAGS, *SAN_FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(srcs, objs)]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-shared-libsan", *objs, "-o", SAN_LIB], verbose)
    return SAN_LIB


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = [os.path.join(BUILD, f[:-4] + ".o") for f in srcs]
    cmds = [[HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(srcs, objs)]
    pdir = os.path.join(BUILD, "phases")
    os.makedirs(pdir, exist_ok=True)
    pobjs = [os.path.join(pdir, f[:-4] + ".o") for f in srcs]
    cmds += [[HIPCC, *FLAGS, "-DMLA_PHASE_STAMPS", "-c", os.path.join(CSRC, s), "-o", o]
             for s, o in zip(srcs, pobjs)]
    probe_tmp = PROBE_LIB + ".tmp"
    cmds.append([HIPCC, *FLAGS, "-shared", PROBE_SRC, "-o", probe_tmp])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    os.replace(probe_tmp, PROBE_LIB)
    for lib, ob in ((PHASES_LIB, pobjs), (LIB, objs)):
        tmp = lib + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *ob, "-o", tmp], verbose)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
