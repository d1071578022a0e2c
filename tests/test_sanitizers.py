"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The fp64 oracle, built with gcc -fsanitize=address,undefined (errors fatal),
  runs the whole pin suite (tests/test_oracle_pins.py) in a child process with
  the sanitizer runtime preloaded: every oracle function on every pin's inputs
  without an out-of-bounds access or undefined behaviour.
* The C-ABI library with its host code (argument validation, geometry,
  workspace sizing) instrumented and its device code uninstrumented (kernels
  are never launched here) runs the ABI suite (tests/test_abi_host.py) the
  same way.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")


def _runtime(cmd):
    out = subprocess.run(cmd, capture_output=True, text=True).stdout.strip()
    return out if out and os.path.isabs(out) and os.path.exists(out) else None


def _run_suite(test_file, env_extra, preload, logdir):
    """Run one test file in a child with the sanitizer runtime preloaded; the
    sanitizers' reports go to files under logdir (the child's own output capture
    would hide them), and any report fails the test with its text."""
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = f"detect_leaks=0:halt_on_error=1:log_path={logdir}/asan"
    env["UBSAN_OPTIONS"] = f"halt_on_error=1:print_stacktrace=1:log_path={logdir}/ubsan"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(TESTS, test_file)],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    text = r.stdout + r.stderr
    reports = "".join(open(os.path.join(logdir, f)).read() for f in sorted(os.listdir(logdir))
                      if f.startswith(("asan", "ubsan")))
    assert reports == "", reports[-4000:]
    assert r.returncode == 0, text[-4000:]
    return text


def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan = _runtime(["gcc", "-print-file-name=libasan.so"])
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    from oracle import oracle as oracle_mod
    lib = str(tmp_path / "liboracle_san.so")
    oracle_mod.compile_oracle(out=lib, extra=("-g", "-fno-omit-frame-pointer",
                                              "-fsanitize=address,undefined",
                                              "-fno-sanitize-recover=all"))
    text = _run_suite("test_oracle_pins.py", {"ETA_ORACLE_LIB": lib}, asan, str(tmp_path))
    assert " passed" in text


def test_abi_host_code_under_asan_ubsan(tmp_path):
    import glob
    rt = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    hipcc = "/opt/rocm/bin/hipcc"
    if not rt or not os.path.exists(hipcc):
        pytest.skip("hipcc or the clang AddressSanitizer runtime is not installed")
    pkg = os.path.join(ROOT, "long_context_decode_predict_amd")
    srcs = sorted(glob.glob(os.path.join(pkg, "csrc", "*.hip")))
    lib = str(tmp_path / "libeta_hostsan.so")
    # host code instrumented; the device code is built (at -O1) but never launched here
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-shared-libsan",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(pkg, "csrc"), *srcs,
           "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    text = _run_suite("test_abi_host.py", {"ETA_LIB_PATH": lib}, rt[0], str(tmp_path))
    assert " passed" in text
