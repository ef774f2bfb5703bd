"""Builds libl3.so (gfx950) in-tree with hipcc: one object per source, then a shared link."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libl3.so")
SOURCES = ["route.hip", "attn.hip", "gemm.hip", "gemm_skinny.hip", "stage.hip", "backward.hip", "alloc.hip", "l3_api.hip"]
HEADERS = ["cdna4.h", "l3_internal.h"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # no packed fp32 instructions (v_pk_*_f32) anywhere in this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("packed-fp32-ops", "not a recognized feature", "remark:")
    err = "\n".join(l for l in r.stderr.splitlines() if not any(s in l for s in noise))
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)


def build(jobs: int = 4) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in SOURCES]
    cmds = [[HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


# Host-side checking build: the sources whose host code handles caller input (plan and
# argument validation, workspace sizing, the prefetch's distinct-ID remap, the LZW
# allocation trie) are compiled again with AddressSanitizer and UndefinedBehaviorSanitizer
# on their host code only, and linked with the regular objects of the other sources.
# The result is loaded by a process with the clang ASan runtime preloaded.
SANITIZED = ["l3_api.hip", "alloc.hip"]
HOST_SAN_LIB = os.path.join(BUILD, "libl3_hostsan.so")
HOST_SAN_FLAGS = ["-g", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined"]


def build_host_sanitized(jobs: int = 4) -> str:
    objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in SOURCES]
    if not all(os.path.exists(o) for o in objs):
        build(jobs)
    san = {s: os.path.join(BUILD, "hostsan_" + s.replace(".hip", ".o")) for s in SANITIZED}
    cmds = [[HIPCC, *FLAGS, *HOST_SAN_FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in san.items()]
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(_run, cmds))
    link = [san.get(s, o) for s, o in zip(SOURCES, objs)]
    tmp = HOST_SAN_LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link, "-o", tmp])
    os.replace(tmp, HOST_SAN_LIB)
    return HOST_SAN_LIB


if __name__ == "__main__":
    print(build())
