"""Build the C-ABI library ``libpa.so`` for gfx950 with hipcc, in-tree.

    python paged_kv_cache_395_amd/build.py

compiles every source under ``csrc/`` (in parallel) and links
``paged_kv_cache_395_amd/lib/libpa.so``.  It is run as a script (or loaded
by path), never imported through the package, whose import loads the
library.  hipcc cross-compiles for gfx950
without a GPU present.

    python paged_kv_cache_395_amd/build.py --sanitize

builds the same library with the host code (block manager, scheduler,
argument checks, launchers) instrumented by AddressSanitizer and
UndefinedBehaviorSanitizer, errors fatal, into
``paged_kv_cache_395_amd/lib/sanitize/libpa.so``; device code is built as
usual.  The CPU test suite runs against it with the sanitizer runtime
preloaded and ``PA_LIBRARY`` naming that file (the command is printed).
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "lib", "_build")
LIB = os.path.join(PKG, "lib", "libpa.so")
SAN_BUILD = os.path.join(PKG, "lib", "sanitize", "_build")
SAN_LIB = os.path.join(PKG, "lib", "sanitize", "libpa.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 instructions are switched off for device code: the compiler
# would otherwise emit v_pk_{add,mul,fma}_f32 from ordinary float code.
# Matrix-core accumulators are kept in ordinary VGPRs (gfx950 allows either
# file): the online-softmax rescale multiplies them on the vector ALUs, and
# in the accumulator file every rescale would copy them out and back.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function"] + DEVICE_FLAGS


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


# host-side sanitizers only (each flag after -Xarch_host): device code is not instrumented
SANITIZERS = ("address", "undefined")
SAN_FLAGS = [f for k in SANITIZERS for f in ("-Xarch_host", "-fsanitize=" + k)] + [
    "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, "-c", src, "-o", obj] + COMMON + list(extra)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"  # host pass does not know the device feature
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    build_dir, lib = (SAN_BUILD, SAN_LIB) if sanitize else (BUILD, LIB)
    extra = SAN_FLAGS if sanitize else []
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, extra), srcs))
    tmp = lib + ".tmp"
    link_extra = [f for k in SANITIZERS for f in ("-fsanitize=" + k,)] + ["-shared-libsan"] if sanitize else []
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs + link_extra
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def sanitizer_runtime() -> str:
    """The clang AddressSanitizer runtime the sanitized library links against."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if not os.path.isabs(path):  # older layouts: ask for the runtime directory
        rd = subprocess.run([HIPCC, "-print-runtime-dir"], capture_output=True, text=True).stdout.strip()
        path = os.path.join(rd, "libclang_rt.asan-x86_64.so")
    return path


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        lib = build(verbose=True, sanitize=True)
        print("run the CPU tests against it with:\n"
              f"  LD_PRELOAD={sanitizer_runtime()} ASAN_OPTIONS=detect_leaks=0 PA_LIBRARY={lib} "
              "python -m pytest tests/ -q -m \"not gpu\"")
    else:
        build(verbose=True)
