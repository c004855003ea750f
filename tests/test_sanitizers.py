"""CPU sanitizer runs (no GPU): AddressSanitizer and UndefinedBehaviorSanitizer over

- the CPU oracle, built from oracle/sv_oracle.cpp with g++ -fsanitize=address,undefined, with every pin of
  tests/test_oracle_pins.py run against it in a child process (the sanitizer runtime preloaded);
- the library's host code (argument checks, workspace planning, launch set-up), built with hipcc and the
  sanitizers on the host side only, with every test of tests/test_abi_cpu.py run against it.

Any sanitizer report aborts the child (halt on error), which fails the test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lossless_draft_verification_04_amd", "csrc")
SOURCES = ["sv_api.hip", "sv_chain.hip", "sv_chain_small.hip", "sv_greedy.hip", "sv_tree.hip", "sv_fanout.hip", "sv_cache.hip",
           "sv_presto.hip", "sv_branch.hip", "sv_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = dict(ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")

pytestmark = pytest.mark.slow


def _child(args, preload, extra_env):
    env = dict(os.environ, **SAN_ENV, **extra_env, LD_PRELOAD=preload)
    return subprocess.run(args, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    so = str(tmp_path / "libsv_oracle_san.so")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                    os.path.join(ROOT, "oracle", "sv_oracle.cpp"), "-o", so], check=True)
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    res = _child([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                  "tests/test_oracle_pins.py"], asan, {"SV_ORACLE_LIB": so})
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0, tail
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, tail


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    so = str(tmp_path / "libspecverify_san.so")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             # sanitizers on the host side only: each -fsanitize is passed to the host compilation
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined"]
    subprocess.run([HIPCC, *flags, "-I" + os.path.join(ROOT, "include"), *[os.path.join(CSRC, f) for f in SOURCES],
                    "-o", so], check=True, capture_output=True)
    rt = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True,
                        check=True).stdout.strip()
    if not os.path.exists(rt):
        rt = os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "lib", "llvm", "lib", "clang")
        cands = [os.path.join(d, f) for d, _, fs in os.walk(rt) for f in fs if f == "libclang_rt.asan-x86_64.so"]
        assert cands, "clang ASan runtime not found"
        rt = cands[0]
    script = (
        "import ctypes, sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "from lossless_draft_verification_04_amd import specverify as svx\n"
        f"L = ctypes.CDLL({so!r})\n"
        "for name, (args, res) in svx._SIGS.items():\n"
        "    fn = getattr(L, name); fn.argtypes = args; fn.restype = res\n"
        "svx._lib = L\n"
        "import tests.test_abi_cpu as T\n"
        "names = [k for k in dir(T) if k.startswith('test_')]\n"
        "for k in names:\n"
        "    getattr(T, k)()\n"
        "print('ran', len(names))\n")
    res = _child([sys.executable, "-c", script], rt, {})
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0, tail
    assert "ran " in res.stdout and "runtime error" not in res.stderr, tail
