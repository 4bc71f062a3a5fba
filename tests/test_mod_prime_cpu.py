"""The kernels' table-slot reduction, run on the CPU.

The hash reduces a mixed 64-bit value modulo each table's prime with a
multiply-high estimate and conditional subtractions (hash_math.h, shared by
the kernels and the plan's host code).  Here that same header is compiled
for the host and checked against the exact remainder `%`, for every prime of
every workload, at the edges of the 64-bit range, at and around multiples of
the prime, and on 10^9 values spread over the range in total.
"""

import os
import shutil
import subprocess

import pytest

from synthetic import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "mod_prime_check.cpp")
CSRC = os.path.join(ROOT, "hashed_gram_embedding_vocab_amd", "csrc")


def _hipcc():
    return os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if not os.path.exists(_hipcc()):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("modprime") / "mod_prime_check")
    subprocess.check_call([_hipcc(), "-O2", "-std=c++17", "-I" + CSRC, "-I" + os.path.join(ROOT, "include"),
                           SRC, "-o", exe])
    return exe


def _primes():
    ps = set()
    for wl in W.WORKLOADS.values():
        ps.update(wl.primes())
    # the smallest tables and the largest row count a plan accepts (< 2^31)
    ps.update([2, 3, 5, 7, 13, 2147483647])
    return sorted(ps)


def test_mod_prime_equals_exact_remainder(checker):
    primes = _primes()
    assert len(primes) > 60
    per_prime = 10**9 // len(primes)
    r = subprocess.run([checker, str(per_prime)] + [str(p) for p in primes], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert int(r.stdout.split()[-1]) >= 10**9 * 0.99


def test_mod_prime_checker_detects_a_wrong_reduction(checker, tmp_path):
    """The checker itself fails on a reduction that skips the corrections."""
    text = open(os.path.join(CSRC, "hash_math.h")).read()
    broken = text.replace("    if (r >= p) r -= p;\n", "")
    assert broken != text
    (tmp_path / "hash_math.h").write_text(broken)
    exe = str(tmp_path / "broken_check")
    subprocess.check_call([_hipcc(), "-O2", "-std=c++17", "-I" + str(tmp_path), SRC, "-o", exe])
    r = subprocess.run([exe, "1000", "500009", "78124999"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "MISMATCH" in r.stdout
