"""Build libcskv.so for gfx950 with hipcc (in-tree; run on a machine with or without a GPU).

    python -m compressed_sparse_kv_03_amd.build_lib            # libcskv.so and libcskv_peaks.so
    python -m compressed_sparse_kv_03_amd.build_lib --sanitize # _build/asan/libcskv_asan.so

The sanitized build instruments the host code only (argument checks, planning, launch setup)
with AddressSanitizer and UndefinedBehaviorSanitizer; its device code is the ordinary build's.
It is for CPU tests of the host paths, loaded into a process that preloads the ASan runtime.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcskv.so")
# measurement helpers (include/cskv_peaks.h): the measured HBM and MFMA ceilings bench.py reports
PEAKS_SRC = os.path.join(PKG, "peaks")
PEAKS_LIB = os.path.join(PKG, "libcskv_peaks.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
    # keep hipcc from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources(d=CSRC):
    return sorted(os.path.join(d, f) for f in os.listdir(d) if f.endswith(".hip"))


ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libcskv_asan.so")
# host-side sanitizers only: each -fsanitize= follows -Xarch_host
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
SAN_FLAGS = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g", "-fno-omit-frame-pointer"] + SAN


def asan_runtime():
    """Path of clang's shared ASan runtime (which a process must preload to load ASAN_LIB), or None."""
    d = os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib", "clang")
    if not os.path.isdir(d):
        return None
    for ver in sorted(os.listdir(d), reverse=True):
        p = os.path.join(d, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


def _compile(src, flags=FLAGS, out_dir=BUILD):
    obj = os.path.join(out_dir, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC] + flags + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    return obj, msgs


def _build(lib, flags, out_dir, link_extra, verbose, src_dir=CSRC):
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources(src_dir)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda src: _compile(src, flags, out_dir), srcs))
    for obj, msgs in results:
        if msgs.strip() and verbose:
            print(msgs, file=sys.stderr)
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + link_extra + ["-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def build(verbose=True):
    _build(PEAKS_LIB, FLAGS, os.path.join(BUILD, "peaks"), [], verbose, PEAKS_SRC)
    return _build(LIB, FLAGS, BUILD, [], verbose)


def build_sanitized(verbose=True):
    return _build(ASAN_LIB, SAN_FLAGS, ASAN_DIR, ["-shared-libsan"] + SAN, verbose)


if __name__ == "__main__":
    build_sanitized() if "--sanitize" in sys.argv[1:] else build()
