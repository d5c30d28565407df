"""Build libtq.so (HIP, gfx950) in-tree with hipcc, and beside it
libtq_ceiling.so (the HBM-stream and matrix-core ceiling kernels of
include/tq_ceiling.h, used only for measurement).

``python kv_cache_vector_pi_amd/build.py`` (run as a file: importing the
package would load the library being rebuilt) or ``build()``.  Every call
recompiles; the objects are built in parallel and linked into
``kv_cache_vector_pi_amd/libtq.so``.
"""
import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtq.so")
CEIL_LIB = os.path.join(HERE, "libtq_ceiling.so")
CEIL_SRC = os.path.join(HERE, "ceiling", "ceiling.hip")
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["tq_host.cpp", "tq_logits.hip", "tq_quantize.hip", "tq_quantize128.hip",
           "tq_quantize_big.hip",
           "tq_search.hip", "tq_attn_out.hip",
           "tq_decode.hip", "tq_step.hip"]
ARCH = os.environ.get("TQ_OFFLOAD_ARCH", "gfx950")

COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-fvisibility=hidden",
          "-Wall", "-Wno-unused-function",
          # never emit packed fp32 VALU ops
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# Per-source flags.  The value-accumulation kernels keep their int8 MFMA
# accumulators in VGPRs: in AGPRs every chunk paid a zeroing write and a
# read-back per accumulator register.
EXTRA = {"tq_attn_out.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "tq_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC] + COMMON + EXTRA.get(src, []) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    warn = "\n".join(l for l in r.stderr.splitlines() if noise not in l and l.strip())
    return obj, warn


def _build_ceiling():
    tmp = CEIL_LIB + ".tmp"
    cmd = [HIPCC] + COMMON + ["-shared", CEIL_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for ceiling.hip:\n{r.stderr}")
    os.replace(tmp, CEIL_LIB)
    return CEIL_LIB, ""


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
        ceil = ex.submit(_build_ceiling)
        results = list(ex.map(_compile, SOURCES))
        ceil.result()
    objs = [o for o, _ in results]
    if verbose:
        for (o, w) in results:
            if w:
                print(w)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
