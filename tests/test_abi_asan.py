"""The library's host code under AddressSanitizer, on the CPU (no GPU).

The host side of the C ABI (argument validation, error messages, the repack
cache and workspace bookkeeping, the size checks of the allocation-free entry
point) lives in api.hip.  This test compiles that file again with the host
pass instrumented by ASan, links it with the library's other objects (the
kernels are unchanged) into a separate shared library, builds the C++ driver
abi_asan_driver.cpp against it, and runs the driver: every call is rejected by
validation or fails at its first HIP call, from several threads, and ASan
reports any out-of-bounds access, use after free or double free on the way.
Needs the objects of a normal build (__graft_entry__.build())."""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build")
CSRC = os.path.join(ROOT, "quantized_decode_ggml_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm toolchain missing")
def test_host_code_under_address_sanitizer(tmp_path):
    objs = sorted(glob.glob(os.path.join(BUILD, "*.o")))
    if not any(o.endswith("api.o") for o in objs):
        pytest.skip("no library objects: run __graft_entry__.build() first")
    others = [o for o in objs if not o.endswith(os.sep + "api.o")]
    api_o = str(tmp_path / "api_asan.o")
    lib = str(tmp_path / "libqdec_asan.so")
    drv = str(tmp_path / "abi_asan_driver")
    # host pass instrumented, device pass untouched
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-fvisibility=hidden",
          "-DQDEC_BUILDING", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, "api.hip"), "-o", api_o])
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libasan", "-Xarch_host", "-fsanitize=address",
          "-o", lib, api_o, *others])
    # the driver is host-only C++ (no .hip source); the ASan runtime is a
    # shared library of the compiler, found through an rpath
    rt = _run([CLANGXX, "-print-file-name=libclang_rt.asan-x86_64.so"]).stdout.strip()
    _run([CLANGXX, "-std=c++17", "-O1", "-g", "-fsanitize=address", "-shared-libasan", "-fno-omit-frame-pointer",
          "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
          os.path.join(ROOT, "tests", "abi_asan_driver.cpp"), "-o", drv, lib, "-L/opt/rocm/lib", "-lamdhip64",
          f"-Wl,-rpath,{tmp_path}", "-Wl,-rpath,/opt/rocm/lib", f"-Wl,-rpath,{os.path.dirname(rt)}", "-lpthread"])
    env = dict(os.environ)
    # leaks at exit belong to the HIP runtime; other preloaded libraries may
    # come before the ASan runtime in the load order
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1:verify_asan_link_order=0"
    r = subprocess.run([drv], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "abi_asan_driver: 0 failures" in r.stdout, out[-4000:]
