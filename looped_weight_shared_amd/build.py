"""Build libtl.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Every call compiles from source; the library is written next to this file,
together with libtl.so.stamp, a hash of the sources, the public header and the
compiler flags it was built from. is_current() compares that stamp with the
sources on disk, so a library older than its sources is rebuilt, not loaded.
Run directly (this file does not import the package): python looped_weight_shared_amd/build.py
"""
import concurrent.futures
import glob
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libtl.so")
STAMP = LIB + ".stamp"
OBJDIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed-FP32 VALU forms are kept out of the generated code on purpose.
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-result"]
# Per-source device-only flags. The decode GEMV takes LLVM's memory-clause
# machine scheduler (same instructions, reordered so each wave's weight
# requests leave together): decode steps measured 1.1-1.5% faster with it,
# while the prefill GEMM measured slower under it and keeps the default.
DEVICE_FLAGS = {"w4gemv.hip": ["-Xarch_device", "-mllvm=-amdgpu-sched-strategy=max-memory-clause"]}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the GPU target feature above; drop that note
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, out



def source_hash() -> str:
    """sha256 over the HIP sources, the kernel headers, include/tl.h and the flags."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h"))
                   + glob.glob(os.path.join(INCLUDE, "*.h")))
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    # the flags with the include directories relative to the repository, so
    # that a copy of the tree at another path keeps the same stamp
    flags = [f.replace(ROOT, ".") for f in FLAGS]
    h.update(" ".join([ARCH] + flags).encode())
    for name in sorted(DEVICE_FLAGS):
        h.update((name + ":" + " ".join(DEVICE_FLAGS[name])).encode())
    return h.hexdigest()


def is_current() -> bool:
    """libtl.so exists and was built from the sources now on disk."""
    if not (os.path.exists(LIB) and os.path.exists(STAMP)):
        return False
    with open(STAMP) as f:
        return f.read().strip() == source_hash()


def ensure_current(verbose: bool = False) -> str:
    """Builds libtl.so unless the one on disk matches the sources."""
    if not is_current():
        print(f"[build] {LIB} is missing or older than its sources: building", file=sys.stderr, flush=True)
        build(verbose)
    return LIB


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(OBJDIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda so: _run([HIPCC, *FLAGS, *DEVICE_FLAGS.get(os.path.basename(so[0]), []), "-c", so[0], "-o", so[1]]), zip(srcs, objs)))
    for (rc, out), src in zip(results, srcs):
        if verbose and out.strip():
            print(out)
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{out}")
    digest = source_hash()  # taken before compiling: an edit during the build leaves the stamp stale
    tmp = LIB + ".tmp"
    rc, out = _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp])
    if rc != 0:
        raise RuntimeError(f"link failed:\n{out}")
    os.replace(tmp, LIB)
    with open(STAMP + ".tmp", "w") as f:
        f.write(digest + "\n")
    os.replace(STAMP + ".tmp", STAMP)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
