"""Build libdmm.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Compiles every time it is called.  Output: dense_matmul_amd/libdmm.so, built
in-tree so that it travels with the source tree.
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdmm.so")
SOURCES = ["gemm_a8w8.hip", "gemm_bf16.hip", "quant.hip", "calib.hip", "api.cpp"]
ARCH = "gfx950"
# packed-fp32 instructions are kept out of every kernel (-packed-fp32-ops)
FLAGS = ["-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(lib=LIB, jobs=4):
    """Compile all sources to objects in parallel, then link libdmm.so."""
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        objs.append(obj)
        lang = [] if src.endswith(".hip") else ["-x", "hip"]
        cmd = [hipcc(), *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append((src, out))
        elif out.strip():
            sys.stderr.write(out + "\n")
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(f"--- {s}\n{o}" for s, o in failed))
    tmp = lib + ".tmp"
    subprocess.run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], check=True)
    os.replace(tmp, lib)
    return lib


def device_asm(src="gemm_a8w8.hip", out=None):
    """gfx950 assembly of one source file (for auditing waits and barriers)."""
    out = out or os.path.join(ROOT, "_build", src + ".s")
    cmd = [hipcc(), *FLAGS, "-S", "--cuda-device-only", os.path.join(CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, stderr=subprocess.DEVNULL)
    return out


if __name__ == "__main__":
    print(build())
