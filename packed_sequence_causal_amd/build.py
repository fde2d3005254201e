"""Build libpsc.so in-tree with hipcc for gfx950.

    python -m packed_sequence_causal_amd.build             # release library
    python -m packed_sequence_causal_amd.build --debug     # also libpsc_debug.so
    python -m packed_sequence_causal_amd.build --sanitize  # also libpsc_san.so

Every HIP source under csrc/ is compiled to an object in csrc/../_build and
linked into packed_sequence_causal_amd/libpsc.so.  The debug variant
(objects in _build_debug, library libpsc_debug.so) is the same code built with
PSC_DEBUG_CHECKS: its attention calls validate cu_seqlens on the device before
launching.  Packed-fp32 instruction selection is switched off for all device
code.

The sanitizer variant (objects in _build_san, library libpsc_san.so) is the
same code with its host side built with AddressSanitizer and
UndefinedBehaviorSanitizer (device code as in the release library): it puts
argument checks, sizing and workspace carving under the sanitizers, on a
machine without a GPU.  It loads only with the ASan runtime preloaded
(asan_runtime()).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpsc.so")
BUILD_DEBUG = os.path.join(PKG, "_build_debug")
LIB_DEBUG = os.path.join(PKG, "libpsc_debug.so")
ARCH = os.environ.get("PSC_OFFLOAD_ARCH", "gfx950")
BUILD_SAN = os.path.join(PKG, "_build_san")
LIB_SAN = os.path.join(PKG, "libpsc_san.so")
# every sanitizer flag is host-side only
SAN_FLAGS = ("-Xarch_host -g -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
             "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer").split()

COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(PKG, "..", "include"),
]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; the HIP extension cannot be built")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(job):
    src, outdir, extra = job
    obj = os.path.join(outdir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj, r.stderr


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def stale(lib: str) -> bool:
    """True when `lib` is missing or older than a source or header it is built from."""
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    inc = os.path.join(PKG, "..", "include")
    deps = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + [os.path.join(inc, f) for f in os.listdir(inc)]
    return any(os.path.getmtime(f) > t for f in deps)


def asan_runtime() -> str:
    """Path of the ASan runtime (with the UBSan handlers) that a process
    loading libpsc_san.so must preload."""
    r = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError(f"ASan runtime not found ({path!r})")
    return path


def build(verbose: bool = False, debug: bool = False, sanitize: bool = False, release: bool = True) -> str:
    """Compile and link libpsc.so (unless release=False), libpsc_debug.so when
    debug=True and libpsc_san.so when sanitize=True."""
    variants = [(BUILD, LIB, [])] if release else []
    if debug:
        variants.append((BUILD_DEBUG, LIB_DEBUG, ["-DPSC_DEBUG_CHECKS"]))
    if sanitize:
        variants.append((BUILD_SAN, LIB_SAN, SAN_FLAGS))
    jobs = []
    for outdir, _, extra in variants:
        os.makedirs(outdir, exist_ok=True)
        jobs += [(src, outdir, extra) for src in sources()]
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(_compile, jobs))
    if verbose:
        for _, err in results:
            lines = [ln for ln in err.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
            if lines:
                print("\n".join(lines), file=sys.stderr)
    for outdir, lib, extra in variants:
        _link([o for o, _ in results if os.path.dirname(o) == outdir], lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, debug="--debug" in sys.argv, sanitize="--sanitize" in sys.argv))
