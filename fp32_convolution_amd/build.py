"""Builds libfconv.so (HIP, gfx950) in-tree with hipcc.

Usage: python fp32_convolution_amd/build.py [-v]   (run by path: importing the
package would load the library being rebuilt)

Flags: -O3 for gfx950 only; -munsafe-fp-atomics so float atomicAdd is the
native global_atomic_add_f32; packed-FP32 VALU instructions disabled
(-packed-fp32-ops) so the compiler never emits v_pk_{add,mul,fma}_f32.
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfconv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["fconv_api.hip", "conv2d_pool.hip", "conv2d_pool_ex.hip", "dwsep_conv1d.hip"]

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


# Per-file additions.  The generalised-pool kernels take maxima of conv
# outputs; with NaNs left out of the contract (a window holding a NaN has an
# unspecified maximum) v_max_f32 needs no quieting copy of each operand, which
# removes a third of those kernels' epilogue instructions.
FILE_FLAGS = {"conv2d_pool_ex.hip": ["-fno-honor-nans"]}


def _compile(src: str, verbose: bool, build_dir: str = BUILD, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *HIP_FLAGS, *FILE_FLAGS.get(src, []), *[f"-D{d}" for d in defines], "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, flush=True)
    return obj


PROBE_SOURCES = ["ceiling_probe.hip"]
PROBE_LIB = os.path.join(HERE, "libfconv_probe.so")


def _link(objs, out: str, verbose: bool) -> None:
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)


def build(verbose: bool = False, out: str = LIB, build_dir: str = BUILD, defines=()) -> str:
    """Compiles every source and links `out` (libfconv.so), then the
    benchmark's ceiling probes (libfconv_probe.so, default build only).
    `defines` (NAME=VALUE strings) override compile-time tiling macros for a
    variant build."""
    os.makedirs(build_dir, exist_ok=True)
    probes = out == LIB and not defines
    srcs = SOURCES + (PROBE_SOURCES if probes else [])
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, defines), srcs))
    _link(objs[:len(SOURCES)], out, verbose)
    if probes:
        _link(objs[len(SOURCES):], PROBE_LIB, verbose)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
