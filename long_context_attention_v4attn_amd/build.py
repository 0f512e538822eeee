"""Build libv4attn.so for gfx950 in-tree (hipcc; one object per source, linked
into long_context_attention_v4attn_amd/libv4attn.so)."""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
OUT = os.path.join(HERE, "libv4attn.so")
SOURCES = ["api.cpp", "compress.hip", "index.hip", "attend.hip"]
ARCH = "gfx950"
# packed fp32 VALU ops (v_pk_*_f32) are disabled for every device pass
HIPFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


# per-source device flags: the index scans consume each MFMA result at once
# in the VALU epilogue, so their accumulators are taken in VGPRs (no
# accumulator-register reads)
EXTRA = {"index.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src, verbose):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc()] + HIPFLAGS + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc(), "-O2", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__",
               "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{msgs}")
    if verbose and msgs:
        print(msgs)
    return obj


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
