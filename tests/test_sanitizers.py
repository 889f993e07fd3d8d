"""CPU sanitizer pass: the oracle built with AddressSanitizer and
UndefinedBehaviorSanitizer (gcc, -fno-sanitize-recover, so any report fails
the run) under the oracle's own pin and property tests, in a child process
with the sanitizer runtime preloaded into the interpreter. The HIP library's
host-side argument checks get the same pass where the toolchain's host
sanitizer runtime can be preloaded (its device code is untouched: the
sanitizers apply to the host compile only)."""
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer", "-g"]
# The oracle's pins and property tests (the planted-mistake tests build their
# own unsanitized copies, so they are left out).
ORACLE_TESTS = ["test_oracle_pins.py", "test_oracle_properties.py", "test_oracle_lowrank.py",
                "test_oracle_tree.py", "test_oracle_tree_sample.py", "test_oracle_outcomes.py",
                "test_bandit_oracle.py", "test_match_rules.py", "test_oracle_stats.py"]


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run_child(tests, env_extra, timeout):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=99"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=98"
    cmd = [sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           *[os.path.join(HERE, t) for t in tests]]
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)


def test_oracle_under_asan_and_ubsan():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    with tempfile.TemporaryDirectory(prefix="oracle_san_") as d:
        lib = oracle.build(out=os.path.join(d, "liboracle_san.so"), extra_flags=SAN_FLAGS)
        r = _run_child(ORACLE_TESTS, {"ORACLE_LIB": lib, "LD_PRELOAD": asan}, timeout=900)
    text = r.stdout + r.stderr
    assert "AddressSanitizer" not in text and "runtime error" not in text, text[-4000:]
    assert r.returncode == 0, text[-4000:]
    assert " passed" in r.stdout


def test_the_sanitized_run_catches_a_planted_overflow():
    """The same pass on a copy of the oracle with a one-past-the-end read planted
    in the residual draw fails with an AddressSanitizer report."""
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    src = os.path.join(os.path.dirname(oracle.__file__), "spec_oracle.c")
    text = open(src).read()
    anchor = "    int j = oracle_inverse_cdf_alt(r, V, u, margin, alt);\n"
    assert anchor in text
    planted = text.replace(anchor, anchor + "    if (V > 0 && r[V] == 12345.0)\n        j = -1;\n", 1)
    with tempfile.TemporaryDirectory(prefix="oracle_san_bad_") as d:
        bad = os.path.join(d, "spec_oracle.c")
        with open(bad, "w") as f:
            f.write(planted)
        lib = os.path.join(d, "liboracle_bad.so")
        srcs = [bad, os.path.join(os.path.dirname(src), "bandit_oracle.c")]
        subprocess.run(["gcc", "-std=c99", "-O1", "-fPIC", "-shared", *SAN_FLAGS, "-o", lib, *srcs,
                        "-lm"], check=True)
        r = _run_child(["test_oracle_pins.py"], {"ORACLE_LIB": lib, "LD_PRELOAD": asan}, timeout=600)
    assert r.returncode == 99  # the AddressSanitizer exit code set above
    assert "heap-buffer-overflow" in r.stdout + r.stderr


def _clang_asan_runtime():
    import glob
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_host_code_of_the_hip_library_under_asan_and_ubsan():
    """The library rebuilt with AddressSanitizer and UndefinedBehaviorSanitizer
    on its host compile (each -fsanitize flag behind -Xarch_host: device code is
    built as usual), under the ABI tests' host-side argument checks."""
    from device_draft_verification_amd import build as hipbuild
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("the ROCm clang AddressSanitizer runtime is not installed")
    flags = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer"):
        flags += ["-Xarch_host", f]
    with tempfile.TemporaryDirectory(prefix="hip_host_san_") as d:
        lib = hipbuild.build(out=os.path.join(d, "libspecverify_san.so"), jobs=8,
                             extra_flags=flags)
        assert b"__asan_report" in open(lib, "rb").read()
        r = _run_child(["test_abi.py"], {"SPEC_VERIFY_LIB": lib, "LD_PRELOAD": rt}, timeout=600)
    text = r.stdout + r.stderr
    assert "AddressSanitizer" not in text and "runtime error" not in text, text[-4000:]
    assert r.returncode == 0, text[-4000:]
    assert " passed" in r.stdout
