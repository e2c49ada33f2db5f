"""The C ABI's host code (argument validation, workspace sizing and carving) under
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

msa_api.hip is compiled with the sanitizers on its host side only, linked with the
kernel objects of the normal build and with tests/abi_sanitize_driver.cpp, and run.
The driver calls every entry point only with arguments that validation rejects, so
no kernel is launched, and sweeps the workspace queries over shapes up to the
largest the ABI accepts (and past them). Any sanitizer report or failed check fails
the test."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OBJ_DIR = os.path.join(ROOT, "_build", "libmsa")
API_SRC = os.path.join(ROOT, "block_sparse_attention_head_amd", "csrc", "msa_api.hip")
DRIVER = os.path.join(ROOT, "tests", "abi_sanitize_driver.cpp")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"

# host-side sanitizer flags: -Xarch_host keeps them off the device code
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _kernel_objects():
    return sorted(o for o in glob.glob(os.path.join(OBJ_DIR, "*.o")) if os.path.basename(o) != "msa_api.o")


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not found")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    objs = _kernel_objects()
    if not objs:
        pytest.skip("kernel objects not built (run the package build first)")
    api_o, drv_o, exe = tmp_path / "msa_api_san.o", tmp_path / "driver.o", tmp_path / "abi_driver"
    run = lambda cmd: subprocess.run(cmd, capture_output=True, text=True, timeout=600)  # noqa: E731
    r = run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", f"-I{ROOT}/include", *HOST_SAN, "-c", API_SRC, "-o", str(api_o)])
    assert r.returncode == 0, r.stderr[-3000:]
    r = run([CLANG, "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include", "-I/opt/rocm/include",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-c", DRIVER, "-o", str(drv_o)])
    assert r.returncode == 0, r.stderr[-3000:]
    r = run([CLANG, "-fsanitize=address,undefined", str(drv_o), str(api_o), *objs, "-L/opt/rocm/lib", "-lamdhip64",
             "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)])
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600, env=env)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "0 failures" in out, out[-2000:]
    shutil.rmtree(tmp_path, ignore_errors=True)
