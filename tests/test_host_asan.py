"""The C ABI layer's host code under AddressSanitizer (no GPU).

csrc/lowram_api.hip (the entry points: argument checks, plans, workspace
layout) is compiled with AddressSanitizer on its host pass and linked with g++,
together with the library's other objects as the regular build leaves them in
_build/obj, into tests/host_asan/abi_host_check.cpp.  The program calls the
sizing queries, the kernel choice and the argument checks of the entry points
on valid and on malformed dims; no call reaches the GPU.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_compressed_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ROCM_LIB = "/opt/rocm/lib"


@pytest.mark.skipif(not os.path.exists(HIPCC) or shutil.which("g++") is None, reason="needs hipcc and g++")
def test_abi_host_code_under_address_sanitizer():
    built = os.path.join(ROOT, "_build", "obj")
    others = [os.path.join(built, os.path.basename(s) + ".o") for s in sorted(glob.glob(os.path.join(CSRC, "*.hip")))
              if os.path.basename(s) != "lowram_api.hip"]
    if not all(os.path.exists(o) for o in others):
        pytest.skip("the library is not built (python -c 'import __graft_entry__ as g; g.build()')")
    out = os.path.join(ROOT, "_build", "host_asan")
    os.makedirs(out, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    api = os.path.join(out, "lowram_api.hip.o")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
                        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *inc,
                        "-c", os.path.join(CSRC, "lowram_api.hip"), "-o", api],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    objs = [api, *others]
    drv = os.path.join(out, "abi_host_check.o")
    r = subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer",
                        "-D__HIP_PLATFORM_AMD__", *inc, "-c", os.path.join(ROOT, "tests", "host_asan", "abi_host_check.cpp"),
                        "-o", drv], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    exe = os.path.join(out, "abi_host_check")
    r = subprocess.run(["g++", "-fsanitize=address", drv, *objs, "-L" + ROCM_LIB, "-Wl,-rpath," + ROCM_LIB,
                        "-lamdhip64", "-o", exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.stdout[-2000:], r.stderr[-4000:])
