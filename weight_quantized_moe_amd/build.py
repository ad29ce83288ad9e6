"""Build libmoe_quant.so for gfx950 with hipcc (in-tree, next to this file).

    python -m weight_quantized_moe_amd.build

Each source compiles to its own object in ``_build/`` (in parallel), then one
hipcc call links the shared library.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_quant.so")
OBJ_DIR = os.path.join(HERE, "..", "_build")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # never emit packed FP32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError(f"hipcc not found (tried {cand})")
    return cand


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    return res


def build(verbose: bool = False, extra_flags=(), out: str = LIB) -> str:
    """Compile every HIP/C++ source into ``out`` (libmoe_quant.so); returns its path.

    ``extra_flags`` are added to every compile and to the link (for instance a
    host-only sanitizer build: ``-Xarch_host -fsanitize=address``).
    """
    os.makedirs(OBJ_DIR, exist_ok=True)
    tag = "" if out == LIB else "_" + os.path.splitext(os.path.basename(out))[0]
    inc = ["-I", os.path.join(HERE, "..", "include")]
    jobs = []
    for src in sources():
        obj = os.path.join(OBJ_DIR, os.path.basename(src) + tag + ".o")
        jobs.append((src, obj, [hipcc(), *HIPCC_FLAGS, *extra_flags, *inc, "-c", src, "-o", obj]))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "8"))))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(lambda j: _run(j[2], verbose), jobs))
    warn = []
    for (src, _, _), res in zip(jobs, results):
        text = res.stdout + res.stderr
        if res.returncode != 0:
            sys.stderr.write(text)
            raise RuntimeError(f"hipcc failed compiling {os.path.basename(src)}")
        warn += [ln for ln in text.splitlines() if "warning" in ln and "packed-fp32-ops" not in ln]
    tmp = out + ".tmp"
    res = _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *extra_flags,
                *[j[1] for j in jobs], "-o", tmp], verbose)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed linking libmoe_quant.so")
    if verbose and warn:
        print("\n".join(warn))
    os.replace(tmp, out)
    return out


ASAN_LIB = os.path.join(OBJ_DIR, "libmoe_quant_asan.so")
ASAN_FLAGS = ("-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
              "-Xarch_host", "-shared-libasan")


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime to preload for the host-ASan build."""
    cands = sorted(glob.glob(os.path.join(os.path.dirname(hipcc()), "..", "lib", "llvm", "lib", "clang",
                                          "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not cands:
        cands = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not cands:
        raise RuntimeError("clang AddressSanitizer runtime not found")
    return os.path.realpath(cands[-1])


def build_asan(verbose: bool = False) -> str:
    """The library with AddressSanitizer on its host code only (the device code
    is built as usual), for running the host-side ABI tests under ASan."""
    return build(verbose, extra_flags=ASAN_FLAGS, out=ASAN_LIB)


if __name__ == "__main__":
    print(build(verbose=True))
