"""Build libmoe.so (the gfx950 HIP library behind include/moe.h) and the
benchmark's calibration library libmoe_calib.so in-tree.

    python -m mixture_experts_layer_07_amd.build
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe.so")
SOURCES = ["api.hip", "route.hip", "permute.hip", "ffn.hip", "fused.hip", "finalize.hip",
           "quant.hip", "noalloc.hip"]
CALIB_SOURCE = "calib.hip"
CALIB_LIB = os.path.join(HERE, "libmoe_calib.so")
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 ops stay off (compiler-generated v_pk_* fp32 forms excluded)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def _hipcc():
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def build(verbose: bool = True, jobs: int = 5) -> str:
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(obj_dir, src.replace(".hip", ".o"))
        cmd = [_hipcc(), *HIPCC_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), out))
        if verbose and out.strip():
            print(out, flush=True)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stdout + r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB, flush=True)
    # the benchmark's HBM read calibration kernel, a library of its own
    obj = compile_one(CALIB_SOURCE)
    tmp = CALIB_LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stdout + r.stderr))
    os.replace(tmp, CALIB_LIB)
    if verbose:
        print("built", CALIB_LIB, flush=True)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
