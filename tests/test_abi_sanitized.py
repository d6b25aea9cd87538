"""The C ABI's host-side validation and workspace sizing, built for the CPU with
AddressSanitizer and UndefinedBehaviorSanitizer (plus unsigned-overflow
checks) and driven by tests/abi_sanitize/driver.cpp: invalid arguments, sizes
at INT_MAX, windows at INT_MAX, the no-alloc scratch boundary, and valid calls
whose launches are recorded by stand-ins instead of enqueued (no GPU, no HIP
runtime).  The library source is compiled as plain C++ (it holds no device
code), so the sanitizers instrument exactly the code the entry points run
before a launch."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "abi_sanitize")
CSRC = os.path.join(ROOT, "transformer_attention_qknorm_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "abi_sanitize")

SANITIZE = ["-fsanitize=address,undefined,unsigned-integer-overflow", "-fno-sanitize-recover=all",
            "-fno-omit-frame-pointer", "-g", "-O1"]


def _clang():
    for c in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++")):
        if c and os.path.exists(c):
            return c
    return None


@pytest.fixture(scope="module")
def driver():
    cxx = _clang()
    if cxx is None:
        pytest.skip("no clang++ with sanitizer runtimes")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "abi_driver")
    inc = ["-I/opt/rocm/include", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", f"-I{HERE}",
           "-D__HIP_PLATFORM_AMD__", "-std=c++17"]
    objs = []
    for src, lang in ((os.path.join(CSRC, "ncattn_api.hip"), "c++"), (os.path.join(HERE, "stubs.cpp"), None),
                      (os.path.join(HERE, "driver.cpp"), None)):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        cmd = [cxx, *(["-x", lang] if lang else []), *inc, *SANITIZE, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"compile failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}"
        objs.append(obj)
    r = subprocess.run([cxx, *SANITIZE, *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, f"link failed:\n{r.stdout}{r.stderr}"
    return exe


def test_validation_under_asan_ubsan(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.pop("LD_PRELOAD", None) if "asan" in env.get("LD_PRELOAD", "") else None
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=120)
    print(r.stdout)
    print(r.stderr)
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    assert r.returncode == 0, r.stdout + r.stderr
    assert "failures=0" in r.stdout
