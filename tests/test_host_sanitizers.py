"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The C-ABI's argument checks (kda_abi.cpp: size and overlap arithmetic,
workspace layouts; its kernel launchers replaced by the failing stand-ins in
sanitize/launch_stubs.cpp) and the C oracle (oracle/kda_oracle.c) are built
with gcc's -fsanitize=address,undefined, and the ABI-validation, binding and
oracle-pin tests are run against those builds in a child process with the
sanitizer runtimes preloaded.  Any sanitizer report ends the child with an
error and fails this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-g", "-O1", "-fPIC", "-shared", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]
SUITES = ["test_abi.py", "test_binding_validation.py", "test_oracle_pins.py", "test_oracle_pins_bwd.py",
          "test_oracle_pins_dplr.py", "test_oracle_pins_gdn.py", "test_oracle_pins_layer.py"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    d = tmp_path_factory.mktemp("san")
    abi, orc = str(d / "libkda.so"), str(d / "libkda_oracle.so")
    subprocess.check_call(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                           os.path.join(ROOT, "gated_delta_rule_55_amd", "csrc", "kda_abi.cpp"),
                           os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"), "-o", abi])
    subprocess.check_call(["gcc", "-std=c11", *SAN, "-fno-fast-math", os.path.join(ROOT, "oracle", "kda_oracle.c"),
                           "-lm", "-lpthread", "-o", orc])
    return abi, orc


def test_abi_checks_and_oracle_under_asan_ubsan(sanitized):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc's sanitizer runtimes are not installed")
    abi, orc = sanitized
    env = dict(os.environ)
    # the sanitizer runtimes go first; whatever else is preloaded stays after them
    env["LD_PRELOAD"] = ":".join([asan, ubsan] + ([env["LD_PRELOAD"]] if env.get("LD_PRELOAD") else []))
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["KDA_LIBRARY"], env["KDA_ORACLE_LIBRARY"] = abi, orc
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           *(os.path.join(ROOT, "tests", s) for s in SUITES)]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
