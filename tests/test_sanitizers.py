"""The oracle and the host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

* tests/host/oracle_sanitize.c drives every oracle entry point over the edge cases the suite feeds
  it, in buffers of exactly the size each call may touch; built with gcc's sanitizers.
* tests/host/abi_validation.c calls every C entry point with arguments the host checks reject (and
  with "nothing to do" arguments), from four threads, against the library's own sources compiled
  with the sanitizers on the host pass only (device code is built as usual and never launched: no
  call here reaches the GPU).

Both programs print "ok" and exit 0 when every check holds; a sanitizer report ends them at once.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
CSRC = os.path.join(ROOT, "canvas_rope_rotary_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")

# sanitizers on the host pass only: device code is compiled as usual
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    noise = "is not a recognized feature for this target"
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    assert r.returncode == 0, f"{cmd[0]} exited {r.returncode}:\n{out[-4000:]}"
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = tmp_path / "oracle_sanitize"
    _run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-ffp-contract=off", "-Wall", "-Wextra", "-Werror", "-o", str(exe),
          os.path.join(HOST, "oracle_sanitize.c"), os.path.join(ROOT, "oracle", "mrope_oracle.c"), "-lm"])
    out = _run([str(exe)], env=ENV, timeout=120)
    assert out.strip().splitlines()[-1] == "ok"


def test_abi_host_paths_under_sanitizers(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("hipcc / clang not found")
    objs = []
    procs = []
    for src in ("mrope_kernels.hip", "mrope_abi.hip"):
        obj = tmp_path / (src + ".o")
        objs.append(str(obj))
        procs.append(subprocess.Popen(
            [HIPCC, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fPIC", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN, "-I", INCLUDE, "-I", CSRC,
             "-c", os.path.join(CSRC, src), "-o", str(obj)],
            stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    drv = tmp_path / "abi_validation.o"
    _run([CLANG, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall",
          "-Werror", "-I", INCLUDE, "-c", os.path.join(HOST, "abi_validation.c"), "-o", str(drv)])
    for p in procs:
        out, _ = p.communicate(timeout=600)
        assert p.returncode == 0, out[-4000:]
    exe = tmp_path / "abi_validation"
    _run([CLANG + "++", "-fsanitize=address,undefined", "-pthread", str(drv), *objs, "-L", os.path.join(ROCM, "lib"),
          "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", str(exe)])
    out = _run([str(exe)], env=ENV, timeout=120)
    assert out.strip().splitlines()[-1] == "ok"
