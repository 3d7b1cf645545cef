"""Build libmi_attn.so (HIP for gfx950) in the package directory.

Every call recompiles all sources: ``python -m masked_flashattention_forward_amd.build``.

``python -m masked_flashattention_forward_amd.build --host-asan DIR`` builds a copy with
AddressSanitizer on the host code only (argument validation, planning, launch set-up;
device code is built as usual) into DIR/libmi_attn.so, for running the CPU tests under
ASan with the sanitizer runtime preloaded. It never replaces the in-tree library.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmi_attn.so")
ARCH = os.environ.get("MI_ATTN_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # no packed fp32 arithmetic in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# host-side AddressSanitizer (each -fsanitize applies to the host compilation only)
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, host_asan_dir: str | None = None) -> str:
    build_dir = BUILD if host_asan_dir is None else os.path.join(host_asan_dir, "_obj")
    lib = LIB if host_asan_dir is None else os.path.join(host_asan_dir, "libmi_attn.so")
    extra = () if host_asan_dir is None else HOST_ASAN
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda f: _compile(f, build_dir, extra), srcs))
    tmp = lib + ".tmp"
    link_extra = [] if host_asan_dir is None else ["-Xarch_host", "-fsanitize=address"]
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources", file=sys.stderr)
    return lib


if __name__ == "__main__":
    if len(sys.argv) == 3 and sys.argv[1] == "--host-asan":
        build(verbose=True, host_asan_dir=os.path.abspath(sys.argv[2]))
    else:
        build(verbose=True)
