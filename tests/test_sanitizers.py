"""CPU sanitizer tier: AddressSanitizer and UndefinedBehaviorSanitizer over
the host code.

- The fp64 oracle (oracle/ssm_oracle.c) is rebuilt with gcc's sanitizers and
  driven by tests/sanitize/oracle_driver.c through every function, at ragged
  sizes, GQA ratios, padded and out-of-range slots and its own rejections.
- The library's argument-validation unit (csrc/ssmd_api.hip) is rebuilt with
  the sanitizers on its host side only (each -fsanitize= after -Xarch_host;
  the device code is built as usual and never runs), linked with the other
  library objects, and driven by tests/sanitize/abi_host_driver.cpp with calls
  that every entry point must refuse before touching a GPU. That driver hides
  every GPU from itself before its first HIP call.

Both runs must exit 0 with no sanitizer report."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ORACLE_SRC = os.path.join(ROOT, "oracle", "ssm_oracle.c")
PKG = os.path.join(ROOT, "ssm_recurrent_decode_gated_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = dict(ASAN_OPTIONS="abort_on_error=0:halt_on_error=1:detect_stack_use_after_return=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
REPORT_MARKS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer", "SUMMARY: ")


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, env=env)
    return r.returncode, r.stdout + r.stderr


def _assert_clean(rc, text, ok_line, what):
    reports = [l for l in text.splitlines() if any(m in l for m in REPORT_MARKS)]
    assert rc == 0 and ok_line in text and not reports, f"{what}: rc={rc}\n{text[-4000:]}"


def test_oracle_under_asan_ubsan(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_driver")
    rc, text = _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
                     "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fopenmp",
                     os.path.join(SAN, "oracle_driver.c"), ORACLE_SRC, "-lm", "-o", exe])
    assert rc == 0, text
    rc, text = _run([exe], env=dict(os.environ, **SAN_ENV))
    _assert_clean(rc, text, "ORACLE_DRIVER_OK", "oracle driver")


def test_abi_host_validation_under_asan_ubsan(tmp_path):
    if not os.access(HIPCC, os.X_OK):
        pytest.skip("hipcc not available")
    objs = sorted(o for o in glob.glob(os.path.join(PKG, "_build", "*.o")) if "ssmd_api" not in os.path.basename(o))
    if not objs:
        pytest.skip("library objects not built (run __graft_entry__.build())")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    api_o, drv_o, exe = (str(tmp_path / n) for n in ("api_san.o", "drv.o", "abi_driver"))
    rc, text = _run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-fno-omit-frame-pointer",
                     "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san, *inc, "-c",
                     os.path.join(PKG, "csrc", "ssmd_api.hip"), "-o", api_o])
    assert rc == 0, text
    rc, text = _run([HIPCC, "-O1", "-g", "-std=c++17", *host_san, *inc, "-c",
                     os.path.join(SAN, "abi_host_driver.cpp"), "-o", drv_o])
    assert rc == 0, text
    rc, text = _run([HIPCC, "-g", "--offload-arch=gfx950", *host_san, drv_o, api_o, *objs, "-o", exe])
    assert rc == 0, text
    # the HIP runtime keeps allocations for the life of the process; leaks are
    # not what this run looks for
    env = dict(os.environ, **SAN_ENV)
    env["ASAN_OPTIONS"] += ":detect_leaks=0"
    rc, text = _run([exe], env=env)
    _assert_clean(rc, text, "ABI_HOST_DRIVER_OK", "ABI host driver")
