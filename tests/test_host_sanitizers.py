"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only): the library's host side (argument validation, plans, the C ABI in
dry-run) built with hipcc's host sanitizers, and the oracle built with gcc's,
each exercised by the CPU tests in a child process that preloads the matching
sanitizer runtime. Any report aborts the child (no recovery), so a passing
child means a clean run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(cmd):
    try:
        path = subprocess.run(cmd, capture_output=True, text=True, timeout=60).stdout.strip()
    except (OSError, subprocess.TimeoutExpired):
        return None
    return path if path and os.path.isabs(path) and os.path.exists(path) else None


def _load(name, rel):
    import importlib.util
    spec = importlib.util.spec_from_file_location(name, os.path.join(ROOT, rel))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _child(env_extra, tests):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", **env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", *tests, "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    tail = "\n".join((r.stdout + r.stderr).splitlines()[-30:])
    assert r.returncode == 0, f"sanitized run failed:\n{tail}"
    assert " passed" in r.stdout, tail
    return r.stdout


def test_library_host_code_under_sanitizers(tmp_path):
    rt = _runtime(["/opt/rocm/llvm/bin/clang", "-print-file-name=libclang_rt.asan-x86_64.so"])
    if rt is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    build = _load("_gqa_build_san", "decoder_attention_rope_amd/build.py")
    lib = build.build(out=str(tmp_path / "libgqa.so"), host_sanitize=True)
    _child({"LD_PRELOAD": rt, "GQA_LIBRARY": lib}, ["tests/test_abi.py"])


def test_oracle_under_sanitizers(tmp_path):
    asan = _runtime(["gcc", "-print-file-name=libasan.so"])
    ubsan = _runtime(["gcc", "-print-file-name=libubsan.so"])
    if asan is None or ubsan is None:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    obuild = _load("_oracle_build_san", "oracle/build.py")
    lib = obuild.build(str(tmp_path / "liboracle.so"), sanitize=True)
    # The pins on the sanitized oracle, and every planted mistake rebuilt with
    # the sanitizers too (ORACLE_SANITIZE).
    _child({"LD_PRELOAD": f"{asan} {ubsan}", "ORACLE_LIBRARY": lib, "ORACLE_SANITIZE": "1"},
           ["tests/test_oracle_pins.py", "tests/test_oracle_mutations.py"])
