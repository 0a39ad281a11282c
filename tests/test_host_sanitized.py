"""The host layer (argument validation and workspace arithmetic of the C ABI)
built with AddressSanitizer and UndefinedBehaviorSanitizer, running the
whole ABI suite (tests/test_abi.py: every validation path, every status
code, the KV-bytes closed forms with their int64 overflow guard) with no
GPU.  Any out-of-bounds access, use-after-free or undefined arithmetic in
the host code aborts the child run.  The device code of the library is
built as usual; only the host side is instrumented."""
import os
import subprocess
import sys
import tempfile

import pytest

from conftest import ROOT

ASAN_RT = "/opt/rocm/llvm/lib/clang/22/lib/linux/libclang_rt.asan-x86_64.so"


def _runtime():
    try:
        out = subprocess.run(["/opt/rocm/llvm/bin/clang", "-print-file-name=libclang_rt.asan-x86_64.so"],
                             capture_output=True, text=True, timeout=30).stdout.strip()
        if out and os.path.exists(out):
            return out
    except (OSError, subprocess.SubprocessError):
        pass
    return ASAN_RT if os.path.exists(ASAN_RT) else None


@pytest.mark.timeout(600)
def test_abi_suite_under_asan_and_ubsan():
    rt = _runtime()
    if rt is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_gqa_build", os.path.join(ROOT, "mqa_kv_cache_amd", "build.py"))
    bld = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bld)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    with tempfile.TemporaryDirectory() as tmp:
        lib = bld.build(out_path=os.path.join(tmp, "libgqa_attn.so"), extra_flags=san,
                        link_flags=["-fsanitize=address,undefined", "-shared-libsan"])
        env = dict(os.environ)
        env["MQA_KV_CACHE_AMD_LIB"] = lib
        env["LD_PRELOAD"] = rt
        # python itself is not instrumented: its allocations are not leaks of ours
        env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
        env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_abi.py")],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=500)
        tail = (r.stdout + r.stderr)[-3000:]
        assert r.returncode == 0, tail
        assert "passed" in r.stdout and "failed" not in r.stdout, tail
        assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, tail
