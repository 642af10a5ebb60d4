"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* The oracle, built by gcc with both sanitizers, runs its pins
  (tests/test_oracle_*.py) in a process with gcc's sanitizer runtimes
  preloaded.
* The library, built by hipcc with both sanitizers on the host pass only
  (device code as usual, never run here), runs the ABI tests
  (tests/test_abi.py: exports, and every host-side argument, shape,
  alignment and workspace rule, each of which returns before any HIP call)
  in a process with clang's runtime preloaded.

Any sanitizer report aborts its process, so the run fails."""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _pytest(files, env):
    e = {**os.environ, **SAN_ENV, **env}
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *files], cwd=ROOT, env=e, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-4000:] + r.stderr[-4000:])
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, r.stderr[-4000:]
    return r


def test_oracle_pins_under_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    import oracle
    lib = str(tmp_path / "liboracle_san.so")
    oracle.build(lib, extra_flags=("-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                                   "-fno-sanitize-recover=all"))
    rts = [subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True, text=True).stdout.strip()
           for n in ("libasan.so", "libubsan.so")]
    if not all(os.path.exists(p) for p in rts):
        pytest.skip("gcc's sanitizer runtimes are not installed")
    pins = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    _pytest(pins, {"LD_PRELOAD": " ".join(rts), "ORACLE_TEST_LIBRARY": lib})


def test_abi_host_code_under_sanitizers(tmp_path):
    rt = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt or not os.path.exists(HIPCC):
        pytest.skip("hipcc or clang's sanitizer runtime is not installed")
    srcs = sorted(glob.glob(os.path.join(ROOT, "top_reduction_amd", "csrc", "*.hip")))
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src)[:-4] + ".o"))
        r = subprocess.run([HIPCC, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = str(tmp_path / "liblmhead_san.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", lib],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    _pytest([os.path.join(ROOT, "tests", "test_abi.py")], {"LD_PRELOAD": rt[-1], "LMH_TEST_LIBRARY": lib})
