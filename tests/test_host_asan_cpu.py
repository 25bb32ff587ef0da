"""The host layer of the C ABI (argument validation, workspace layout, error reporting) built
with AddressSanitizer and driven by the ABI tests, without a GPU.

moe_api.hip is compiled with the sanitizer on its host code only (the device code is built as
usual), linked with the library's other objects from the last build, and the ABI tests of
test_abi_cpu.py run in a child process with the sanitizer runtime preloaded and the binding
pointed at that library.  Any heap, stack or global overflow or use after free in the host
layer ends the child with a sanitizer report."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_moe_layer_bailingmoev3_amd")
BUILD = os.path.join(ROOT, "_build")


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_host_layer_under_address_sanitizer(tmp_path):
    hipcc, rt = _hipcc(), _asan_runtime()
    others = [o for o in glob.glob(os.path.join(BUILD, "*.hip.o")) if not o.endswith("moe_api.hip.o")]
    if not hipcc or not rt or not others:
        pytest.skip("needs hipcc, the clang sanitizer runtime and a previous build of the library")
    obj, lib = str(tmp_path / "moe_api_asan.o"), str(tmp_path / "libmoe_asan.so")
    inc = [f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(PKG, 'csrc')}"]
    compile_cmd = [hipcc, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
                   "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                   "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *inc,
                   "-c", os.path.join(PKG, "csrc", "moe_api.hip"), "-o", obj]
    link_cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                "-shared-libsan", "-o", lib, obj, *others]
    for cmd in (compile_cmd, link_cmd):
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
    plugin = tmp_path / "asan_library.py"
    plugin.write_text("import sparse_moe_layer_bailingmoev3_amd as m\n"
                      f"m.lib_path = lambda: {lib!r}\n")
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:halt_on_error=1",
               PYTHONPATH=os.pathsep.join([str(tmp_path), ROOT, os.environ.get("PYTHONPATH", "")]))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "asan_library", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out and "skipped" not in out.splitlines()[-1], out[-1000:]
