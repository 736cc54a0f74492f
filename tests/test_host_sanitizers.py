"""Host sanitizer tier (CPU only): the oracle and the C-ABI host validation under AddressSanitizer and
UndefinedBehaviorSanitizer.

Two sanitized builds go to a temporary directory:
  * oracle.c, compiled with clang -fsanitize=address,undefined (no recovery from UB);
  * api.cpp (every host-side argument check and the dispatch of the C ABI), compiled with the same host
    sanitizers and linked with the library's other, unchanged objects (their device code cannot be sanitized
    here, and the host tests never launch it).
Then the oracle's pin tests, the C-ABI tests and the binding checks run in a child process that loads the
sanitizer runtime first and uses the sanitized builds (LFM2SC_LIB / LFM2SC_ORACLE_LIB); any report aborts it.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_short_causal_amd", "csrc")
BUILD = os.path.join(ROOT, "gated_short_causal_amd", "_build")
LLVM = "/opt/rocm/llvm/bin/clang"
HIPCC = "/opt/rocm/bin/hipcc"
OBJS = ["fwd.hip.o", "bwd.hip.o", "fused.hip.o", "fused_split.hip.o", "interop.hip.o", "check.hip.o", "noalloc.hip.o"]
TESTS = ["tests/test_oracle_pins.py", "tests/test_oracle_pins_grad.py", "tests/test_oracle_pins_conv_update.py",
         "tests/test_oracle_pins_fused.py", "tests/test_abi.py", "tests/test_binding_checks.py"]


def _runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def test_oracle_and_host_validation_under_asan_ubsan(tmp_path):
    rt = _runtime()
    if rt is None or not os.path.exists(LLVM) or not os.path.exists(HIPCC):
        pytest.skip("clang sanitizer runtime or ROCm compilers not found")
    missing = [o for o in OBJS if not os.path.exists(os.path.join(BUILD, o))]
    if missing:
        pytest.skip(f"library objects not built yet ({missing}): run __graft_entry__.build() first")
    san_c = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
    oracle = str(tmp_path / "liboracle_san.so")
    _run([LLVM, "-std=c99", "-O1", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", *san_c,
          os.path.join(ROOT, "oracle", "oracle.c"), "-o", oracle])
    host = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    api_o = str(tmp_path / "api_san.o")
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, *host, "-x", "hip", "-c",
          os.path.join(CSRC, "api.cpp"), "-o", api_o])
    lib = str(tmp_path / "liblfm2sc_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, api_o,
          *[os.path.join(BUILD, o) for o in OBJS]])
    nm = _run(["nm", "-D", lib]).stdout
    assert "__asan_" in nm and "__ubsan_" in nm, "api.cpp was not instrumented"

    env = dict(os.environ)
    env["LD_PRELOAD"] = rt + (" " + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["LFM2SC_LIB"] = lib
    env["LFM2SC_ORACLE_LIB"] = oracle
    # the sanitizer runtime is live in the child
    probe = _run([sys.executable, "-c", "import ctypes; print(hasattr(ctypes.CDLL(None), '__asan_init'))"], env=env)
    assert probe.stdout.strip() == "True", probe.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *TESTS], cwd=ROOT,
                       env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, f"sanitized run failed:\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    assert "passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]
