"""The host side of the library (argument validation, the balanced-cut plan,
tree masks, slot ranges, tiering endpoints, the streaming bookkeeping) under
AddressSanitizer: the host-instrumented build (build.py --asan) runs the
C-ABI CPU tests in a child process with the ASan runtime preloaded. Any
out-of-bounds or use-after-free in host code aborts that process."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc")
def test_abi_cpu_tests_under_host_asan():
    sys.path.insert(0, ROOT)
    from long_context_speculative_amd import build
    lib = build.build(asan=True)
    runtime = build.asan_runtime()
    assert os.path.exists(runtime), runtime
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               SS_VERIFY_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
    assert "passed" in r.stdout
    # the library such a child loads is the instrumented build, next to the runtime
    probe = ("from long_context_speculative_amd import ssverify as ss; ss.lib(); "
             "maps = open('/proc/self/maps').read(); "
             "print(ss.LIB_PATH in maps, 'libclang_rt.asan' in maps)")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r.stdout.split() == ["True", "True"], r.stdout + r.stderr[-2000:]
