"""The library's host code (argument validation, split planning, workspace
sizes, status strings) built with AddressSanitizer and
UndefinedBehaviorSanitizer and driven on the CPU.

The library is compiled from the same sources with the sanitizers on the host
side only (`-Xarch_host`; device code unchanged) into a temporary folder, and
`tests/host_sanitize.cpp` calls the size queries over thousands of random
configurations and every compute entry point with arguments the validation
must reject, so no kernel is launched and no GPU is needed.  Any
out-of-bounds access, use of freed memory, signed overflow, misaligned or
NULL dereference in that code aborts the driver.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SANITIZE = ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
            "-fno-omit-frame-pointer", "-g")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is not available")
def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    from head_latent_attention_11_amd import build as B
    lib = B.build(out_dir=str(tmp_path), host_flags=SANITIZE)
    assert os.path.exists(lib)
    exe = str(tmp_path / "host_sanitize")
    host = [a for f in SANITIZE for a in ("-Xarch_host", f)]
    cmd = [HIPCC, "--cuda-host-only", "-O1", "-std=c++17", *host,
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "host_sanitize.cpp"),
           "-L", str(tmp_path), "-lmla", f"-Wl,-rpath,{tmp_path}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ)
    # leaks of the HIP runtime's own start-up are not this library's
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "host_sanitize OK" in r.stdout, out
    assert "AddressSanitizer" not in out and "runtime error" not in out, out
