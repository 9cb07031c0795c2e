"""Build libdmm.so (the HIP kernels and the C ABI) for gfx950 with hipcc,
and the benchmark's calibration library libdmm_calib.so beside it.

Compiles every time it is called.  Outputs: dense_matmul_amd/libdmm.so and
dense_matmul_amd/calib/libdmm_calib.so, built in-tree so that they travel
with the source tree.
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdmm.so")
SOURCES = ["gemm_a8w8.hip", "gemm_bf16.hip", "quant.hip", "api.cpp"]
# the benchmark's matrix-op calibration kernel: its own library, not libdmm
CALIB_SRC = os.path.join(HERE, "calib", "calib.hip")
CALIB_LIB = os.path.join(HERE, "calib", "libdmm_calib.so")
ARCH = "gfx950"
# packed-fp32 instructions are kept out of every kernel (-packed-fp32-ops)
FLAGS = ["-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(lib=LIB, calib_lib=CALIB_LIB):
    """Compile all sources to objects in parallel, then link libdmm.so and
    libdmm_calib.so."""
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    for src in SOURCES + [CALIB_SRC]:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        if src != CALIB_SRC:
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
    for out, ins in ((lib, objs), (calib_lib, [os.path.join(objdir, "calib.hip.o")])):
        tmp = out + ".tmp"
        subprocess.run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *ins, "-o", tmp], check=True)
        os.replace(tmp, out)
    return lib


def device_asm(src="gemm_a8w8.hip", out=None):
    """gfx950 assembly of one source file (for auditing waits and barriers)."""
    out = out or os.path.join(ROOT, "_build", src + ".s")
    cmd = [hipcc(), *FLAGS, "-S", "--cuda-device-only", os.path.join(CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, stderr=subprocess.DEVNULL)
    return out


def disassemble(src="gemm_a8w8.hip"):
    """gfx950 disassembly of the kernels build() compiled from one source
    file (the device code object inside _build/<src>.o, which build() leaves
    there), for audits of the emitted waits, barriers and loads."""
    obj = os.path.join(ROOT, "_build", src + ".o")
    if not os.path.exists(obj):
        build()
    llvm = "/opt/rocm/llvm/bin"
    work = os.path.join(ROOT, "_build", "disasm")
    os.makedirs(work, exist_ok=True)
    fat, co = os.path.join(work, src + ".fatbin"), os.path.join(work, src + ".co")
    subprocess.run(["objcopy", "--dump-section", f".hip_fatbin={fat}", obj], check=True)
    subprocess.run([f"{llvm}/clang-offload-bundler", "--unbundle", "--type=o", f"--input={fat}",
                    f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}", f"--output={co}"], check=True)
    return subprocess.run([f"{llvm}/llvm-objdump", "-d", f"--mcpu={ARCH}", co], check=True,
                          capture_output=True, text=True).stdout


if __name__ == "__main__":
    print(build())
