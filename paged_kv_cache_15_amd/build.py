"""Builds libpagedkv.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_15_amd.build [--verbose]

Every HIP source is compiled with packed-fp32 instructions disabled
(``-target-feature -packed-fp32-ops``): float code must not be turned into
v_pk_{add,mul,fma}_f32.
"""
import os
import subprocess
import sys
import time
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpagedkv.so")
SOURCES = ["allocator.cpp", "sha256.cpp", "device_info.cpp", "cache_ops.hip", "bandwidth_probe.hip", "decode_attention.hip",
           "decode_attention_streamk.hip", "decode_attention_shared.hip",
           "prefill_attention.hip"]
ARCH = os.environ.get("PAGED_KV_ARCH", "gfx950")


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose=False):
    objs = []
    flags = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-result",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    t0 = time.time()
    cmds = []
    for src in SOURCES:
        obj = os.path.join(CSRC, src.rsplit(".", 1)[0] + ".o")
        cmds.append([hipcc(), *flags, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    # the translation units are independent: compile them side by side
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", "8"))))
    with ThreadPoolExecutor(jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s")
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd))
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    # hipcc's host pass does not know the packed-fp32 feature and says so; harmless
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln
             and "is not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv or "-v" in sys.argv)
