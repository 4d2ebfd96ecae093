"""AddressSanitizer and UndefinedBehaviorSanitizer runs on the CPU.

- The oracle (oracle/kvq_oracle.c) built with gcc and the sanitizers, driven
  through every entry point on small ragged cases (tests/sanitize/oracle_driver.c).
- The library's host code -- argument validation, overlap checks, the
  planner, the static scratch limit -- built for the host only (no device
  code) with hipcc's clang and the sanitizers on the host side, linked with
  the HIP runtime and driven through the C ABI with invalid arguments and
  planning-only calls (tests/sanitize/abi_driver.cpp); nothing reaches a
  kernel launch, and the device addresses are never dereferenced.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "bit_kv_cache_03_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
           HIP_VISIBLE_DEVICES="-1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"])
    r = _run([exe], env=ENV, timeout=120)
    assert "oracle sanitizer run: ok" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm compilers not installed")
def test_host_code_under_sanitizers(tmp_path):
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    flags = ["--offload-arch=gfx950", "--cuda-host-only", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        lang = [] if src.endswith(".hip") else ["-x", "hip"]
        _run([HIPCC, *flags, *lang, "-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    # the device code is not built: each object's reference to its embedded
    # device binary gets an empty blob (the runtime loads device code lazily,
    # on a launch or a symbol lookup, and the driver makes neither)
    nm = _run(["nm", "-u", *objs]).stdout
    blobs = sorted({w for w in nm.split() if w.startswith("__hip_fatbin_")})
    stub = tmp_path / "device_blobs.c"
    stub.write_text("".join(f"const char {b}[64] __attribute__((aligned(4096))) = {{0}};\n" for b in blobs))
    _run([CLANGXX.replace("clang++", "clang"), "-c", str(stub), "-o", str(tmp_path / "device_blobs.o")])
    objs.append(str(tmp_path / "device_blobs.o"))
    drv = str(tmp_path / "abi_driver.o")
    _run([CLANGXX, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-I", os.path.join(ROOT, "include"), "-c", os.path.join(HERE, "abi_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_driver")
    _run([CLANGXX, "-fsanitize=address,undefined", drv, *objs, "-o", exe, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib"])
    r = _run([exe], env=ENV, timeout=300)
    assert "host sanitizer run: ok" in r.stdout
