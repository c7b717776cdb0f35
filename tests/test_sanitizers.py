"""CPU sanitizer builds (AddressSanitizer + UndefinedBehaviorSanitizer, any
report fatal) of the two host-side layers:

- the oracle (oracle.c built by gcc with the sanitizers), running the whole
  CPU oracle suite (formats, GEMM, grouped GEMM, quantizers, epilogue,
  tolerance checker) in a child process with the sanitizer runtime
  preloaded;
- the library's host code (every .hip source compiled host-only by hipcc
  with the sanitizers on the host side, no device code), driven through the
  C ABI by tests/sanitize/abi_driver.c with the argument-check cases of
  test_abi.py (validation, size queries, status strings, and every entry
  point's rejection of bad arguments before any device work).

No GPU is needed or touched: no call reaches a kernel launch.
"""
import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from tests import test_abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_scaled_precision_03_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
FATAL = ("AddressSanitizer", "runtime error", "LeakSanitizer", "UndefinedBehaviorSanitizer")


def _check_clean(proc, what):
    out = proc.stdout + proc.stderr
    for marker in FATAL:
        assert marker not in out, "%s: sanitizer report\n%s" % (what, out[-6000:])
    assert proc.returncode == 0, "%s: exit %d\n%s" % (what, proc.returncode, out[-6000:])
    return out


def _gcc_asan_runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_suite_under_asan_ubsan(tmp_path):
    from oracle import build as oracle_build
    rt = _gcc_asan_runtime()
    if rt is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = oracle_build.build_sanitized(str(tmp_path / "liboracle_san.so"))
    env = dict(os.environ)
    env.update({
        "ORACLE_LIB": lib,
        "LD_PRELOAD": rt,
        # the interpreter's own allocations are not this test's subject
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "OMP_NUM_THREADS": "4",
    })
    files = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    proc = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider"]
                          + files, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = _check_clean(proc, "oracle suite")
    assert " passed" in out and " failed" not in out


def _driver_lines():
    lines = []
    for args, expect in test_abi.VALIDATE_CASES:
        lines.append(("mxgemm_validate", args, expect))
        lines.append(("mxgemm_run", args, expect if expect != 0 else None))
    for args, expect in test_abi.FUSED_CASES:
        a = list(args[:11]) + [args[11] or 0, args[12]]
        lines.append(("mxgemm_validate_fused", a, expect))
        lines.append(("mxgemm_run_fused", a, expect if expect != 0 else None))
    for args, expect in test_abi.GROUPED_CASES:
        lines.append(("grouped_fp8_gemm_validate", args, expect))
        lines.append(("grouped_fp8_gemm_run", args, expect if expect != 0 else None))
    for args, expect in test_abi.BF16_CASES:
        lines.append(("grouped_bf16_gemm_validate", args, expect))
        lines.append(("grouped_bf16_gemm_run", args, expect if expect != 0 else None))
    for fn, args, expect in test_abi.REJECT_CALLS:
        lines.append((fn, args, expect))
    for rows, K in ((4096, 4096), (300, 512), (11008, 11008), (-1, 128), (128, 100)):
        for fmt in (0, 4, 16, 7):
            lines.append(("mxgemm_preshuffle_b_bytes", (fmt, rows, K), None))
        lines.append(("mxgemm_preshuffle_scales_bytes", (rows, K), None))
    for s in (0, -1, -2, -3, -4, -99, 12345):
        lines.append(("mxgemm_status_string", (s,), 0))
    # calls whose success would launch a kernel are left out; sizes are
    # compared with the library's own answers through the normal build
    out = []
    lib = test_abi._mx().lib()
    for fn, args, expect in lines:
        if expect is None:
            if fn.startswith("mxgemm_preshuffle"):
                expect = getattr(lib, fn)(*args)
            else:
                continue
        out.append("%s %s %d" % (fn, " ".join(str(int(a or 0)) for a in args), expect))
    return out


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm toolchain not found")
def test_host_layer_under_asan_ubsan(tmp_path):
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    inc = os.path.join(ROOT, "include")
    # host code only (no device compilation); each -fsanitize= applies to
    # the host side
    flags = ["--offload-host-only", "-x", "hip", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-I", inc, "-I", CSRC]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC] + flags + ["-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return obj

    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, srcs))
    # A host-only object refers to its translation unit's device binary by
    # a symbol that the device compilation would define.  Define each as an
    # empty offload bundle (magic, zero entries): the runtime records it at
    # load and would only parse it for a kernel launch, which never happens.
    syms = set()
    for o in objs:
        nm = subprocess.run(["/opt/rocm/llvm/bin/llvm-objdump", "-t", o], capture_output=True, text=True)
        syms |= {ln.split()[-1] for ln in nm.stdout.splitlines() if "*UND*" in ln and "__hip_fatbin_" in ln}
    stub = tmp_path / "fatbin_stubs.c"
    stub.write_text("".join(
        '__attribute__((aligned(4096))) const char %s[32] = "__CLANG_OFFLOAD_BUNDLE__";\n' % n for n in sorted(syms)))
    stub_obj = str(tmp_path / "fatbin_stubs.o")
    r = subprocess.run([CLANG, "-c", str(stub), "-o", stub_obj], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    objs.append(stub_obj)
    drv_obj = str(tmp_path / "abi_driver.o")
    r = subprocess.run([CLANG, "-O1", "-g", "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", inc, "-I", "/opt/rocm/include",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-c",
                        os.path.join(ROOT, "tests", "sanitize", "abi_driver.c"), "-o", drv_obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    exe = str(tmp_path / "abi_driver")
    r = subprocess.run([CLANGXX, "-fsanitize=address,undefined", drv_obj] + objs
                       + ["-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    lines = _driver_lines()
    env = dict(os.environ)
    env.update({"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    proc = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, env=env,
                          timeout=300)
    out = _check_clean(proc, "host layer")
    assert "%d calls, 0 mismatches" % len(lines) in out, out[-3000:]
