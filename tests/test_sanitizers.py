"""Memory and undefined-behaviour checks on the host (no GPU): the oracle's C functions and the
library's host-side validation, each built with AddressSanitizer and UndefinedBehaviorSanitizer
and run on small inputs (tests/sanitize/).  The library is built as for the product with the
sanitizers on its host code only; the validation calls fail before anything would be enqueued,
so no kernel runs (and no GPU is needed)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "ssm_sequence_mixer_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "oracle_checks"
    subprocess.check_call(["gcc", "-std=c99"] + SAN + [
        os.path.join(HERE, "oracle_checks.c"), os.path.join(ROOT, "oracle", "ia_oracle.c"),
        "-lm", "-o", str(exe)])
    r = subprocess.run([str(exe)], env=ENV, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")


def test_host_validation_under_address_and_ub_sanitizers(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    srcs = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC))
            if f.endswith((".cpp", ".hip"))] + [os.path.join(HERE, "abi_checks.cpp")]
    host = []
    for flag in SAN:
        host += ["-Xarch_host", flag]
    objs = []
    procs = []
    for src in srcs:
        obj = tmp_path / (os.path.basename(src) + ".o")
        objs.append(str(obj))
        procs.append(subprocess.Popen(
            [hipcc, "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-Xclang",
             "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
             "-I", CSRC] + host + ["-c", src, "-o", str(obj)],
            stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out, _ = p.communicate(timeout=600)
        assert p.returncode == 0, out
    exe = tmp_path / "abi_checks"
    subprocess.check_call([hipcc, "--offload-arch=gfx950"] + host + objs + ["-o", str(exe)])
    r = subprocess.run([str(exe)], env=ENV, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("(0 failure(s))")
