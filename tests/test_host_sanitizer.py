"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The C-ABI's argument checks (api.cpp) and the prefix-snapshot reader and
writer (prefix.cpp) are built host-only with both sanitizers, against the
stand-in device layer in host_stub.cpp, and driven on the CPU by
host_san_driver.py: a save/load round trip, every truncation of the header,
every header byte damaged, damaged body sections, trailing bytes, capacities,
key widths and argument errors, and the workspace checks of decode_step.  Any
out-of-bounds access, use after free or undefined behaviour aborts the child.
"""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "long_context_compressed_compress_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"


def _asan_runtime():
    base = "/opt/rocm/llvm/lib/clang"
    if not os.path.isdir(base):
        return None
    for ver in sorted(os.listdir(base), reverse=True):
        p = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


def test_driver_mirrors_the_cache_struct():
    """The driver's copy of csa_decode_cache is the binding's, field for field."""
    from long_context_compressed_compress_amd import libcsa
    src = open(os.path.join(HERE, "host_san_driver.py")).read()
    ns = {}
    start = src.index("FIELDS = [")
    end = src.index("\n\n", start)
    exec("import ctypes\n_i32, _i64, _f32, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p\n"
         + src[start:end], ns)
    assert [(n, t) for n, t in ns["FIELDS"]] == list(libcsa._DecodeCacheC._fields_)


@pytest.mark.timeout(600)
def test_host_code_under_sanitizers(tmp_path):
    rt = _asan_runtime()
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG) and rt):
        pytest.skip("hipcc, clang++ or the AddressSanitizer runtime is not installed")
    objs = []
    for src in (os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "prefix.cpp"), os.path.join(HERE, "host_stub.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [HIPCC, "--offload-host-only", "-x", "hip", "-std=c++17", "-O1", "-g", "-fPIC",
               "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=undefined", "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        objs.append(obj)
    so = str(tmp_path / "libcsa_hostsan.so")
    r = subprocess.run([CLANG, "-shared", "-fsanitize=address,undefined", "-Wl,-Bsymbolic", "-o", so, *objs],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    work = tmp_path / "files"
    work.mkdir()
    r = subprocess.run([sys.executable, os.path.join(HERE, "host_san_driver.py"), so, str(work)],
                       capture_output=True, text=True, env=env, timeout=500)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "host sanitizer driver: ok" in out, out[-6000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]
    shutil.rmtree(work, ignore_errors=True)
