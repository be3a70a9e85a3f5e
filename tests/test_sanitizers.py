"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Two sanitized builds, each driven by existing CPU tests in a child process that preloads the
sanitizer runtime:

* libkla with ASan + UBSan on its host pass (gated_delta_rule_kla_amd.build), loaded through
  KLA_LIBRARY: tests/test_abi.py runs every argument check and error path of the C ABI and
  the workspace formulas (no GPU call is reached);
* the fp64 C oracle (oracle.build_sanitized, gcc), loaded through KLA_ORACLE_LIBRARY: the
  oracle's pins run against it.

Any sanitizer report fails the child (UBSan halts on the first error) and so the test.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:alloc_dealloc_mismatch=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1", "OMP_NUM_THREADS": "4"}


def _child(env_extra, argv, timeout):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(env_extra)
    r = subprocess.run([sys.executable, *argv], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=timeout)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    return r.stdout


def test_c_abi_checks_under_asan_ubsan(tmp_path):
    from gated_delta_rule_kla_amd import build
    lib = build.build_host_sanitized(str(tmp_path / "kla"))
    env = {"KLA_LIBRARY": lib, "LD_PRELOAD": build.sanitizer_runtime()}
    loaded = _child(env, ["-c", "import gated_delta_rule_kla_amd as k; k.load_library(); "
                                "print(k.library_path())"], 300)
    assert loaded.strip().endswith(lib)
    _child(env, ["-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
                 "tests/test_abi.py"], 600)


def test_oracle_under_asan_ubsan(tmp_path):
    import oracle
    lib = oracle.build_sanitized(str(tmp_path / "libkla_oracle_san.so"))
    pre = ":".join(subprocess.check_output(["gcc", f"-print-file-name={n}"], text=True).strip()
                   for n in ("libasan.so", "libubsan.so"))
    env = {"KLA_ORACLE_LIBRARY": lib, "LD_PRELOAD": pre}
    loaded = _child(env, ["-c", "import oracle; oracle._load(); print(oracle._LIB)"], 300)
    assert loaded.strip() == lib
    _child(env, ["-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
                 "tests/test_oracle_pins.py", "tests/test_oracle_variants.py",
                 "tests/test_oracle_diag.py"], 900)
