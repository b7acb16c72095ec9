"""Host AddressSanitizer + UndefinedBehaviorSanitizer builds of the CPU oracle
and of the C-ABI layer (argument validation and dispatch), with the oracle
pins and the ABI tests run under them in child processes (no GPU).

The oracle is rebuilt with gcc and its runtime; the library's host code
(api.cpp) with hipcc, the sanitizer flags applied to the host pass only, and
linked with the device objects of the regular build.  Each child preloads
the matching sanitizer runtime (the Python interpreter itself is not
instrumented) and fails on the first report."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mxfp8_block_scaled_05_amd", "csrc")
BUILD = os.path.join(ROOT, "mxfp8_block_scaled_05_amd", "_build")
HIPCC = "/opt/rocm/bin/hipcc"
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:detect_odr_violation=0:alloc_dealloc_mismatch=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-2000:], r.stderr[-4000:])


def _child(preload, code, tmp):
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV)
    env["UBSAN_OPTIONS"] += ":log_path=%s" % os.path.join(tmp, "ubsan")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    reports = "".join(open(f).read() for f in glob.glob(os.path.join(tmp, "ubsan*")))
    assert r.returncode == 0 and not reports, (r.returncode, r.stdout[-3000:], r.stderr[-3000:], reports[:3000])
    return r.stdout


def test_oracle_pins_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    libasan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(libasan):
        pytest.skip("gcc's libasan not available")
    so = str(tmp_path / "liboracle_san.so")
    _run([gcc, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-fopenmp", "-shared", "-fPIC",
          os.path.join(ROOT, "oracle", "mxfp8_oracle.c"), "-o", so, "-lm"])
    code = (
        "import sys; sys.path[:0] = ['tests', '.']\n"
        "import oracle\n"
        "oracle._LIB_PATH = %r\n"
        "oracle._SRC = oracle._LIB_PATH\n"
        "import pytest\n"
        "rc = pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu', 'tests/test_oracle_codec.py',\n"
        "                  'tests/test_oracle_quantize.py', 'tests/test_oracle_gemm.py', 'tests/test_oracle_regroup.py'])\n"
        "assert oracle._load()._name == oracle._LIB_PATH\n"
        "print('RC', int(rc), flush=True)\n"
        "sys.exit(int(rc))\n") % so
    out = _child(libasan, code, str(tmp_path))
    assert "RC 0" in out


def test_abi_under_asan_ubsan(tmp_path):
    rts = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    objs = [os.path.join(BUILD, n + ".o") for n in ("quantize", "dequantize", "repack", "gemm", "selfcheck")]
    if not os.path.exists(HIPCC) or not rts or not all(os.path.exists(o) for o in objs):
        pytest.skip("hipcc, the clang sanitizer runtime or the built device objects are missing")
    api_o = str(tmp_path / "api_san.o")
    so = str(tmp_path / "libmxfp8_san.so")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    _run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer", *san,
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, "api.cpp"), "-o", api_o])
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *san, *objs, api_o, "-o", so])
    code = (
        "import sys; sys.path[:0] = ['tests', '.']\n"
        "import mxfp8_block_scaled_05_amd as m\n"
        "m.LIB_PATH = %r\n"
        "import pytest\n"
        "rc = pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu', 'tests/test_abi.py'])\n"
        "assert m.lib()._name == m.LIB_PATH\n"
        "print('RC', int(rc), flush=True)\n"
        "sys.exit(int(rc))\n") % so
    out = _child(rts[-1], code, str(tmp_path))
    assert "RC 0" in out
