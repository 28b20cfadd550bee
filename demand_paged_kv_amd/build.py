"""Build libgrowpage.so (HIP, gfx950) in-tree with hipcc.

    python -m demand_paged_kv_amd.build                    # compile every source, link the library
    python -m demand_paged_kv_amd.build --host-sanitizers  # also a host-instrumented variant

The library lands next to this file (demand_paged_kv_amd/libgrowpage.so), which is
where the binding looks for it.  The host-sanitizer variant (_build/san/libgrowpage_san.so)
instruments the host code only, with AddressSanitizer and UndefinedBehaviorSanitizer; its
device code is the ordinary build's at -O1.  It is for host-side checks of the argument
validation on a machine without a GPU: load it with the ASan runtime preloaded
(asan_runtime() names the file), ASAN_OPTIONS=detect_leaks=0 for the Python process.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libgrowpage.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["api.hip", "ema.hip", "scan.hip", "finish.hip", "decide.hip", "compact.hip", "attn.hip",
           "pool_alloc.hip", "static_scratch.hip"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    "-ffp-contract=off",                       # no silent multiply-add contraction
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",  # no packed FP32 math
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: libgrowpage needs ROCm's hipcc to build")


SAN_DIR = os.path.join(BUILD_DIR, "san")
SAN_OUT = os.path.join(SAN_DIR, "libgrowpage_san.so")
# each sanitizer flag right after its -Xarch_host: the device code is never instrumented
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    """Path of the shared ASan runtime of ROCm's clang (to preload)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    res = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the ASan runtime of ROCm's clang was not found")
    return path


def _compile(src: str, flags=None, out_dir: str = BUILD_DIR) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *(HIPCC_FLAGS if flags is None else flags), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


def build_host_sanitized(verbose: bool = True) -> str:
    """The host-instrumented variant (see the module docstring); returns its path."""
    os.makedirs(SAN_DIR, exist_ok=True)
    flags = [f for f in HIPCC_FLAGS if f != "-O3"] + ["-O1"] + SAN_FLAGS
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda src: _compile(src, flags, SAN_DIR), SOURCES))
    tmp = SAN_OUT + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", *SAN_FLAGS, "-shared-libasan", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, SAN_OUT)
    if verbose:
        print(f"built {SAN_OUT}")
    return SAN_OUT


if __name__ == "__main__":
    build()
    if "--host-sanitizers" in sys.argv[1:]:
        build_host_sanitized()
    sys.exit(0)
