"""Build the host code with AddressSanitizer and UndefinedBehaviorSanitizer.

Test infrastructure: the host sources of libpa (C ABI, block allocator, prefix cache,
validators) are compiled by g++ with both sanitizers and linked with the library's HIP
objects (built as usual; device code is not instrumented), and the C oracle by gcc. The
results go to <repo>/_build/san/: libpa.so and liboracle.so. Load them with the sanitizer
runtimes preloaded (LD_PRELOAD) and PA_LIBRARY / PA_ORACLE_LIBRARY pointing at them.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from paged_kv_cache_298_amd import build as B  # noqa: E402

OUT = os.path.join(ROOT, "_build", "san")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def runtimes():
    """The sanitizer runtimes to preload, in order."""
    out = []
    for name in ("libasan.so", "libubsan.so"):
        p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
        out.append(p)
    return out


def build(verbose=False):
    os.makedirs(OUT, exist_ok=True)
    hip_objs = [os.path.join(B.BUILD, src + ".o") for src in B.HIP_SOURCES]
    if not all(os.path.exists(o) for o in hip_objs):
        B.build(verbose)        # the device objects of the normal build
    objs = list(hip_objs)
    for src in B.HOST_SOURCES:
        obj = os.path.join(OUT, src + ".o")
        B._run(["g++", *B.HOST_FLAGS, *SAN, "-c", os.path.join(B.CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    lib = os.path.join(OUT, "libpa.so")
    B._run([B.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", lib], verbose)
    orc = os.path.join(OUT, "liboracle.so")
    B._run(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra", "-fno-fast-math",
            *SAN, os.path.join(ROOT, "oracle", "pa_oracle.c"), "-o", orc, "-lm"], verbose)
    return lib, orc


if __name__ == "__main__":
    print(build(verbose=True))
