"""Build libmoe_a16w4.so (gfx950 only) in-tree with hipcc.

Every source under csrc/ is compiled for --offload-arch=gfx950 and linked
into mxfp4_grouped_gemm_amd/libmoe_a16w4.so. Packed-fp32 VALU ops are kept
off (-packed-fp32-ops) and fp32 division/sqrt stay correctly rounded.
"""
import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe_a16w4.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["abi.cpp", "route.hip", "route_t1.hip", "align_sort.hip", "gemm_stream.hip", "gemm_decode.hip", "gemm_gemv.hip", "gemv_mfma.hip", "gemv_resident.hip", "gemm_prefill.hip", "gemm_prefill_int4.hip", "decode_t1.hip", "combine.hip", "requant.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
]


# Per-file extra flags. The int4 single-wave tiles read their MFMA results
# back every 32-group; with the results in VGPRs instead of AGPRs no
# v_accvgpr_read is needed (the option must not reach the 4-wave kernels,
# which need AGPRs for 256 accumulator registers).
FILE_FLAGS = {"gemm_prefill_int4.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
