"""AddressSanitizer builds of the CPU oracle and of the C-ABI library's host
side, run on the CPU.

The oracle (`oracle/engram_oracle.c`) is compiled with AddressSanitizer and
UndefinedBehaviorSanitizer into a driver that calls every one of its entry
points on small inputs whose buffers are exactly the documented sizes
(`tests/native/asan_oracle_check.c`).  The library's sources are compiled with
the sanitizer on their host code only (device code is built as usual) and
linked into a driver that creates and destroys plans and calls every entry
point with arguments that host-side validation rejects before any device
work (`tests/native/asan_host_check.cpp`).  Either driver exits non-zero on a
sanitizer report or an unexpected status.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")


def _run(cmd, env_extra=None, timeout=300):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, env=env)


def test_oracle_under_asan_and_ubsan(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path / "asan_oracle")
    r = _run(["gcc", "-std=gnu11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
              "-fsanitize=address,undefined", os.path.join(NATIVE, "asan_oracle_check.c"),
              os.path.join(ROOT, "oracle", "engram_oracle.c"), "-lm", "-o", exe])
    assert r.returncode == 0, r.stderr
    r = _run([exe], {"ASAN_OPTIONS": "detect_leaks=1", "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr[-4000:]


def test_library_host_side_under_asan(tmp_path):
    from hashed_gram_embedding_vocab_amd import build as b
    clang = "/opt/rocm/llvm/bin/clang++"
    if not (os.path.exists(b.HIPCC) and os.path.exists(clang)):
        pytest.skip("hipcc / clang++ not available")
    # the sanitizer on host code only; device code is built as for the library
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]

    def comp(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [b.HIPCC] + b.COMMON + (b.DEVICE if src.endswith(".hip") else []) + san + ["-c", src, "-o", obj]
        r = _run(cmd)
        assert r.returncode == 0, r.stderr[-4000:]
        return obj

    srcs = b.sources() + [os.path.join(NATIVE, "asan_host_check.cpp")]
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(comp, srcs))
    exe = str(tmp_path / "asan_host")
    r = _run([clang, "-fsanitize=address", "-o", exe] + objs + ["-L/opt/rocm/lib", "-lamdhip64",
                                                                  "-Wl,-rpath,/opt/rocm/lib"])
    assert r.returncode == 0, r.stderr[-4000:]
    # leak checking off: the HIP runtime keeps process-lifetime allocations
    r = _run([exe], {"ASAN_OPTIONS": "detect_leaks=0"})
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr[-4000:]
