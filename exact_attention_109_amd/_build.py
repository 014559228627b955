"""Build libfa.so (the C-ABI attention library) for gfx950 with hipcc.

Every HIP/C++ source under csrc/ is compiled to an object in _build/ and the
objects are linked into exact_attention_109_amd/libfa.so. The library is built
in-tree so that it travels with the source tree.

Two check builds of the same sources sit beside it (never loaded by the
product path):
  * libfa_hostsan.so: host code with AddressSanitizer and
    UndefinedBehaviorSanitizer (device code unchanged), for the argument
    validation tests on the CPU (load it with the sanitizer runtime preloaded);
  * libfa_debugsync.so: every fence-free workgroup barrier made a full one
    (FA_DEBUG_SYNC), whose results the GPU tests require to be bitwise equal
    to libfa.so's.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")
# check builds: name -> (library, extra compile flags)
VARIANTS = {
    "hostsan": (os.path.join(PKG, "libfa_hostsan.so"),
                ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]),
    "debugsync": (os.path.join(PKG, "libfa_debugsync.so"), ["-DFA_DEBUG_SYNC"]),
}


def sanitizer_runtime() -> str:
    """The AddressSanitizer runtime of the ROCm compiler (to LD_PRELOAD into a
    process that loads libfa_hostsan.so)."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    f"--offload-arch={ARCH}",
    # Keep the compiler from emitting packed fp32 VALU ops (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, extra, build_dir: str = BUILD) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *extra, "-c", src, "-o", obj]
    if src.endswith(".hip"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(extra=(), jobs: int | None = None, verbose: bool = False, variant: str | None = None) -> str:
    """Compile every source and link libfa.so (or the check build `variant`,
    a key of VARIANTS). Returns the library path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    lib, vflags = (LIB, []) if variant is None else VARIANTS[variant]
    build_dir = BUILD if variant is None else f"{BUILD}_{variant}"
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2)))
    flags = list(extra) + vflags
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, flags, build_dir), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources")
    return lib


def build_all(verbose: bool = False) -> str:
    """libfa.so and the check builds. Returns libfa.so's path."""
    lib = build(verbose=verbose)
    for name in VARIANTS:
        build(verbose=verbose, variant=name)
    return lib


def clean():
    shutil.rmtree(BUILD, ignore_errors=True)
    for name, (lib, _) in VARIANTS.items():
        shutil.rmtree(f"{BUILD}_{name}", ignore_errors=True)
        if os.path.exists(lib):
            os.remove(lib)
    if os.path.exists(LIB):
        os.remove(LIB)


if __name__ == "__main__":
    build_all(verbose=True)
