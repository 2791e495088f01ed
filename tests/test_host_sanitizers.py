"""The C ABI's host-side paths under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU needed).

The library sources are compiled with the sanitizers on their host code only
(each -fsanitize= behind -Xarch_host; the device code is built as usual),
linked with tests/host_checks.cpp into one instrumented executable, and run:
every call it makes must be answered or rejected on the host, and neither
sanitizer may report anything (shape fields at their extremes, lengths past
the limits, NULL, misaligned and too-small arguments).
"""
import concurrent.futures
import os
import shutil
import subprocess

import pytest

from long_context_attention_lightning_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


@pytest.mark.skipif(shutil.which("/opt/rocm/bin/hipcc") is None, reason="hipcc not installed")
def test_host_paths_clean_under_asan_and_ubsan(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc"
    clangxx = "/opt/rocm/llvm/bin/clang++"
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(B.PKG, "csrc")]
    srcs = B.sources()
    objs = [str(tmp_path / (os.path.basename(s)[:-4] + ".o")) for s in srcs]

    def compile_one(so):
        s, o = so
        r = subprocess.run([hipcc, *B.HIPCC_FLAGS, *HOST_SAN, *inc, "-c", s, "-o", o], capture_output=True, text=True)
        return r.returncode, r.stderr[-2000:]

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        for rc, err in ex.map(compile_one, zip(srcs, objs)):
            assert rc == 0, err
    main_o = str(tmp_path / "host_checks.o")
    exe = str(tmp_path / "host_checks")
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-g"]
    r = subprocess.run([clangxx, "-std=c++17", *san, "-I", os.path.join(ROOT, "include"), "-c",
                        os.path.join(ROOT, "tests", "host_checks.cpp"), "-o", main_o], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([clangxx, *san, main_o, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
                        "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=0")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    print(out[-4000:])
    assert "runtime error" not in out, out[-4000:]
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0 and "host checks passed" in out, out[-4000:]
