"""Build liblfm2sc.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

``python -m gated_short_causal_amd.build`` or ``__graft_entry__.build()``.
Always recompiles.  Sources are compiled in parallel, then linked.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblfm2sc.so")
SOURCES = ["fwd.hip", "bwd.hip", "fused.hip", "fused_split.hip", "interop.hip", "check.hip", "noalloc.hip", "api.cpp"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build liblfm2sc.so)")


def compile_flags():
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
        # keep fp32 arithmetic on plain VALU ops (no packed-fp32 forms)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        "-I", INCLUDE, "-I", CSRC,
    ]


def _compile(src: str, verbose: bool, build_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *compile_flags(), *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature and says so; drop that noise
    noise = ("packed-fp32-ops", "is not a recognized feature", "warning generated")
    msgs = "\n".join(l for l in (r.stderr or "").splitlines() if not any(n in l for n in noise))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if msgs.strip() and verbose:
        print(msgs, file=sys.stderr)
    return obj


def build(verbose: bool = False, out: str = LIB, extra=()) -> str:
    """Compile and link; `out` and `extra` (additional hipcc flags, e.g. -D tuning knobs) default to
    the in-tree library with the default configuration."""
    build_dir = BUILD_DIR if out == LIB else os.path.join(os.path.dirname(out), "_build")
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, extra), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
