"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): every library source is compiled with the sanitizers on its host
part (the gfx950 device code is built as usual and never runs here), linked
with tests/abi_check.cpp, and run; the checker exercises the argument
validation of every entry point, the size queries and the launch-free trace
calls, and must exit 0 with no sanitizer report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc():
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        pytest.skip("hipcc not available")
    return p


def test_abi_host_code_under_sanitizers(tmp_path):
    from gated_mla_latent_amd import build as B
    hipcc = _hipcc()
    # sanitizers on the host compilation only (each -fsanitize after -Xarch_host)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
    flags = [f"--offload-arch={B.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    procs, objs = [], []
    for src in B.sources():
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([hipcc, *flags, *san, "-c", src, "-o", obj], stdout=subprocess.PIPE,
                                      stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out = p.communicate(timeout=600)[0]
        assert p.returncode == 0, out
    main_obj = str(tmp_path / "abi_check.o")
    r = subprocess.run([hipcc, *flags, *san, "-x", "c++", "-I", os.path.join(ROOT, "include"), "-c",
                        os.path.join(ROOT, "tests", "abi_check.cpp"), "-o", main_obj],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    exe = str(tmp_path / "abi_check")
    r = subprocess.run([hipcc, f"--offload-arch={B.ARCH}", "-fno-gpu-sanitize", "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", main_obj, *objs, "-o", exe],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and "abi_check: ok" in r.stdout, r.stdout + r.stderr
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
