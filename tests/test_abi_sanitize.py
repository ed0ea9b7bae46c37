"""The C ABI's host logic under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU): api.cpp and codebook.cpp are rebuilt with both sanitizers on the host
side and linked with the library's kernel objects into tests/native/
abi_sanitize.cpp, which walks status strings, level tables, workspace sizes,
argument validation, and valid calls whose first kernel launch fails because
no device is visible (each must return QLORA_ERR_HIP). The driver is run with
every device hidden and skips the launch part itself if one is visible."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_nf4_quantized_18_amd", "csrc")
BUILD = os.path.join(ROOT, "bit_nf4_quantized_18_amd", "_build")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


def test_abi_host_logic_under_asan_ubsan(tmp_path):
    kernels = [os.path.join(BUILD, f) for f in sorted(os.listdir(BUILD))] if os.path.isdir(BUILD) else []
    kernels = [f for f in kernels if f.endswith(".o") and os.path.basename(f) not in ("api.o", "codebook.o")]
    if not kernels or not os.path.exists(HIPCC):
        pytest.skip("the library's kernel objects are not built (python -m bit_nf4_quantized_18_amd.build)")
    flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-std=c++17", f"-I{ROOT}/include", f"-I{CSRC}"]
    objs = []
    for src in (os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "codebook.cpp"),
                os.path.join(ROOT, "tests", "native", "abi_sanitize.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        p = subprocess.run([HIPCC] + flags + SAN + ["-c", src, "-o", obj], capture_output=True, text=True)
        assert p.returncode == 0, p.stdout + p.stderr
        objs.append(obj)
    exe = str(tmp_path / "abi_sanitize")
    p = subprocess.run([HIPCC] + SAN + ["-o", exe] + objs + kernels, capture_output=True, text=True)
    assert p.returncode == 0, p.stdout + p.stderr
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    p = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "all checks passed" in p.stdout
