"""Build libfp8q.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Every source is compiled for gfx950 only, with -ffp-contract=off (the exact division and
rounding steps are written out explicitly and must not be fused) and with packed FP32
instructions disabled.  No fast-math flag is ever used: the per-group scale and the
reciprocal rely on IEEE binary32 division.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libfp8q.so")
SOURCES = ["fp8q_api.hip", "fp8q_quant.hip", "fp8q_gemm.hip", "fp8q_gemm_prefill.hip",
           "fp8q_gemv.hip", "fp8q_kv.hip", "fp8q_calib.hip"]
ARCH = "gfx950"


def hipcc_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def build(verbose: bool = False, jobs: int = 5) -> str:
    from concurrent.futures import ThreadPoolExecutor

    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *hipcc_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
