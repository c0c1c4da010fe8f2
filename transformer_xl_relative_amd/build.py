"""Build libxlrel.so (HIP for gfx950) in-tree with hipcc.

Each source compiles to an object in _build/, then one shared library is linked
next to this file. Packed-FP32 instructions are disabled for every device
compile.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libxlrel.so")
SOURCES = ["api.hip", "relpos.hip", "gemm.hip", "gemm_bf16.hip", "attn.hip", "attn_bf16.hip", "ln.hip", "attn_bwd.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fno-gpu-rdc", "-munsafe-fp-atomics"]


# Keep MFMA accumulators in ordinary VGPRs: the softmax and the ring writes
# read them with vector instructions, which AGPRs would force through copies.
# IEEE mode off (no NaNs occur): maxima compile to v_max3 without quieting.
PER_SOURCE = {"attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mno-amdgpu-ieee", "-fno-honor-nans"],
              "attn_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mno-amdgpu-ieee", "-fno-honor-nans"],
              "gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


# AddressSanitizer and UndefinedBehaviorSanitizer on the host code only (the
# validation, layout and launch code; the kernels are built as usual), for a
# process that preloads clang's ASan runtime: each flag goes to the host pass.
HOST_SANITIZE = [f for opt in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
                               "-fno-omit-frame-pointer") for f in ("-Xarch_host", opt)]


def _compile(src: str, verbose: bool, build_dir: str, defines, host_sanitize: bool = False) -> str:
    obj = os.path.join(build_dir, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *PER_SOURCE.get(src, []), *(HOST_SANITIZE if host_sanitize else []),
           *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature; that warning is harmless
    noise = "not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip() and verbose:
        print(msg)
    return obj


def build(verbose: bool = False, out: str = LIB, defines=(), host_sanitize: bool = False) -> str:
    build_dir = BUILD if out == LIB else os.path.join(os.path.dirname(os.path.abspath(out)), "_build")
    os.makedirs(build_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, defines, host_sanitize), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
