"""Compile the HIP sources of the VDN library into libvdn.so (gfx950).

Run as `python -m softmax_attention_video_amd._build`.  Every call compiles
all sources (objects under _build/, the shared library next to this file).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libvdn.so")

ARCH = os.environ.get("VDN_OFFLOAD_ARCH", "gfx950")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # keep the compiler from forming packed-fp32 VALU ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


# Per-source extra flags: the window Softmax and merge GEMM kernels keep MFMA
# results in arch VGPRs (two waves per SIMD fit in 256 registers; the
# softmax arithmetic reads S without accumulator-register moves).
EXTRA = {"k_window_softmax.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "k_vda_solve.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "k_window_softmax_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "k_merge.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = min(len(srcs), max(1, min(16, len(os.sched_getaffinity(0)))))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


# Host-side sanitizer build (a test build, never loaded by the product path):
# vdn_host.hip -- argument checks, workspace carving, the host work-item and
# plan loops -- with AddressSanitizer and UndefinedBehaviorSanitizer on the
# host pass only; the kernel sources as in build().
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def build_sanitized(out_dir: str) -> str:
    os.makedirs(out_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = []
    todo = []
    for src in srcs:
        name = os.path.basename(src)
        if name == "vdn_host.hip":
            todo.append((src, os.path.join(out_dir, name + ".san.o"), SAN_HOST))
        else:
            o = os.path.join(OBJ, name + ".o")
            if os.path.exists(o) and os.path.getmtime(o) >= os.path.getmtime(src):
                objs.append(o)
            else:
                todo.append((src, os.path.join(out_dir, name + ".o"), []))

    def comp(job):
        src, obj, extra = job
        cmd = [hipcc(), *FLAGS, *EXTRA.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        return obj

    jobs = min(len(todo), max(1, min(16, len(os.sched_getaffinity(0))))) or 1
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs += list(ex.map(comp, todo))
    lib = os.path.join(out_dir, "libvdn_san.so")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-fsanitize=address,undefined",
           "-shared-libasan", *objs, "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return lib


def asan_runtime() -> str:
    """Path of the shared AddressSanitizer runtime of the HIP compiler."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        for c in glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"):
            return c
        raise RuntimeError("shared ASan runtime not found")
    return path


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
