"""Host AddressSanitizer build of the C-ABI layer, for CPU-side checks.

api.cpp (argument validation, workspace sizing, descriptor handling: all
host code) is compiled by g++ with -fsanitize=address and linked with the
regular device objects of the in-tree build into _build/asan/libv4attn_asan.so.
The device code is not instrumented.  Load it with the ASan runtime preloaded
(Python itself is not instrumented):

    LD_PRELOAD=$(gcc -print-file-name=libasan.so) ASAN_OPTIONS=detect_leaks=0 \\
    V4ATTN_LIB=_build/asan/libv4attn_asan.so python -m pytest tests/test_abi.py -m "not gpu"
"""

import os
import subprocess
import sys

from . import build as B

OUT_DIR = os.path.join(B.BUILD, "asan")
OUT = os.path.join(OUT_DIR, "libv4attn_asan.so")
DEVICE_SOURCES = [s for s in B.SOURCES if s.endswith(".hip")]


def asan_runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("gcc's libasan.so not found")
    return path


def build_asan():
    """Compile api.cpp with ASan and link it with the device objects (the
    regular build is run first, so they are current).  Returns the path."""
    B.build()
    os.makedirs(OUT_DIR, exist_ok=True)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    obj = os.path.join(OUT_DIR, "api.o")
    cxx = ["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-fsanitize=address", "-fno-omit-frame-pointer",
           "-w", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
           "-I", os.path.join(B.ROOT, "include"), "-c", os.path.join(B.CSRC, "api.cpp"), "-o", obj]
    r = subprocess.run(cxx, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cxx)}\n{r.stdout}{r.stderr}")
    dev = [os.path.join(B.BUILD, s + ".o") for s in DEVICE_SOURCES]
    link = ["g++", "-shared", "-fsanitize=address", "-o", OUT, obj] + dev + [
        "-L", os.path.join(rocm, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(link)}\n{r.stdout}{r.stderr}")
    return OUT


if __name__ == "__main__":
    print(build_asan())
    sys.exit(0)
