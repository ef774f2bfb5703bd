"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU, no GPU).

The fp64 oracle (plain C) is rebuilt with gcc -fsanitize=address,undefined and runs
every forward and backward pin; the library's host code that handles caller input
(plan and argument validation, workspace sizing, the LZW allocation trie) is rebuilt
with the sanitizers on its host side only (static_token_routed_amd/build.py,
build_host_sanitized) and driven through its C ABI.  Each runs in a child process
with the matching sanitizer runtime preloaded (the Python interpreter itself is not
instrumented); any report fails the test."""
import importlib.util
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
DRIVER = os.path.join(HERE, "sanitizer_driver.py")
SAN_OPTS = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
            "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run(kind, lib, preload):
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_OPTS)
    r = subprocess.run([sys.executable, DRIVER, kind, lib], env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "SANITIZER_DRIVER_OK" in r.stdout, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return r.stdout


def _gcc_lib(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip(f"gcc has no {name}")
    return p


def test_oracle_under_sanitizers(tmp_path):
    so = oracle.build(out=str(tmp_path / "liboracle_san.so"),
                      extra=("-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                             "-fno-sanitize-recover=undefined"))
    out = _run("oracle", so, f"{_gcc_lib('libasan.so')} {_gcc_lib('libubsan.so')}")
    print(out[-500:])


def test_library_host_code_under_sanitizers():
    spec = importlib.util.spec_from_file_location("_l3_build", os.path.join(ROOT, "static_token_routed_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    try:
        so = b.build_host_sanitized()
    except (FileNotFoundError, RuntimeError) as e:  # no hipcc in this environment
        pytest.skip(f"cannot build: {e}")
    rt = subprocess.run([b.HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    if not os.path.exists(rt):
        import glob
        found = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        if not found:
            pytest.skip("no clang ASan runtime")
        rt = found[0]
    out = _run("library", so, rt)
    print(out[-500:])
