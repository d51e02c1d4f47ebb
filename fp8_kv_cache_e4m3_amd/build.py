"""Build libfp8attn.so in-tree with hipcc for gfx950.

    python fp8_kv_cache_e4m3_amd/build.py             # runs without importing (and loading) the package
    python fp8_kv_cache_e4m3_amd/build.py --timeline  # libfp8attn_timeline.so: the same library with the
                                                      # decode kernel's phase stamps (bench.py --timeline)

Every source is compiled on each call (no stale objects); objects go to ``_build/``
(``_build_timeline/``) next to this file and the shared library lands in this package directory.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfp8attn.so")
TIMELINE_LIB = os.path.join(PKG, "libfp8attn_timeline.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/lib/llvm/bin/clang++"


def _torch_lib_dir():
    try:
        import torch
    except Exception:
        return None
    d = os.path.join(os.path.dirname(torch.__file__), "lib")
    return d if os.path.exists(os.path.join(d, "libamdhip64.so")) else None

SOURCES = ["api.cpp", "quantize.hip", "decode.hip", "combine.hip", "prefill.hip", "prefill_wide.hip",
           "verify.hip", "cache_write.hip"]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops (v_pk_*_f32).
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I" + os.path.join(os.path.dirname(PKG), "include")]


def _compile(src: str, build_dir: str = BUILD, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    extra = os.environ.get("EXTRA_HIPCC_FLAGS", "").split()   # e.g. -D tuning switches for experiments
    cmd = [HIPCC] + COMMON + list(defines) + extra + lang + ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l and "(ignoring feature)" not in l)
    if msg.strip():
        print(f"[build] {src}:\n{msg}", file=sys.stderr)
    return obj


def build(verbose: bool = True, timeline: bool = False) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    build_dir = BUILD + "_timeline" if timeline else BUILD
    lib = TIMELINE_LIB if timeline else LIB
    defines = ["-DFP8ATTN_TIMELINE"] if timeline else []
    os.makedirs(build_dir, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, defines), srcs))
    tmp = lib + ".tmp"
    # One HIP runtime per process: torch ships its own libamdhip64.so without a SONAME and its
    # libraries load it by the unversioned name.  Linking against that file records the same
    # unversioned name here, so in a process that already imported torch the loader reuses
    # torch's runtime and stream handles stay valid across the two libraries.  Without torch,
    # the rpath finds the system runtime under /opt/rocm/lib.
    rt_dir = _torch_lib_dir()
    cmd = [CLANGXX, "-shared", "-fPIC", "-o", tmp] + objs
    if rt_dir:
        cmd += ["-L" + rt_dir, "-lamdhip64", "-Wl,-rpath," + rt_dir + ":/opt/rocm/lib"]
    else:
        cmd += ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # A kernel whose host stub is missing links fine but fails at load time: catch it here.
    r = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l.split()[-1] for l in r.stdout.splitlines() if "__device_stub__" in l]
    if missing:
        raise RuntimeError("kernel host stubs are undefined in the linked library: " + ", ".join(missing))
    shutil.move(tmp, lib)
    if verbose:
        print(f"[build] {lib}")
    return lib


if __name__ == "__main__":
    build(timeline="--timeline" in sys.argv[1:])
