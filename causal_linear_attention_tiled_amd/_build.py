"""Build liblinattn.so for gfx950 with hipcc (in-tree, no JIT cache)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "liblinattn.so")
OUT_SAN = os.path.join(PKG, "liblinattn_san.so")
BUILD_DIR = os.path.join(ROOT, "_build")
# host code only (device code is unchanged): AddressSanitizer and UBSan
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # Keep the compiler from forming packed fp32 VALU ops (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, sanitize: bool = False) -> str:
    sub = os.path.join(BUILD_DIR, "san") if sanitize else BUILD_DIR
    os.makedirs(sub, exist_ok=True)
    obj = os.path.join(sub, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *(SAN_FLAGS if sanitize else []), "-x", "hip", "-c", src, "-o", obj,
           f"-I{os.path.join(ROOT, 'include')}"]
    subprocess.run(cmd, check=True)
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every source under csrc/ and link liblinattn.so (always rebuilds).  With
    sanitize, liblinattn_san.so: the host code built with AddressSanitizer and UBSan (the
    process must preload the sanitizer runtime)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), srcs))
    out = OUT_SAN if sanitize else OUT
    tmp = out + ".tmp"
    link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if sanitize:
        link[1:1] = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                     "-Xarch_host", "-shared-libsan"]
    subprocess.run(link, check=True)
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
