"""Build libfoscar.so (HIP, gfx950) in-tree with hipcc.

    python -m bit_quantized_kv_split_amd.build             # or build() from Python
    python -m bit_quantized_kv_split_amd.build --timeline  # libfoscar_timeline.so (see timeline.py)

Every source is compiled with packed fp32 arithmetic disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops) and without the compiler's
wave-level atomic rewrite (-amdgpu-atomic-optimizer-strategy=None): every
atomic here runs in one lane, and the rewrite makes the issuing wave wait for
the result right away, where the kernels issue a work-counter increment early
and read it much later.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfoscar.so")
LIB_TIMELINE = os.path.join(HERE, "libfoscar_timeline.so")
SOURCES = ["api.hip", "decode.hip", "decode_paged.hip", "decode_rot.hip", "decode_paged_rot.hip", "decode_generic.hip",
           "pack.hip", "quant.hip"]
ARCH = os.environ.get("FOSCAR_ARCH", "gfx950")

FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
         "-Wno-unused-command-line-argument"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, timeline: bool = False) -> str:
    """Compile every source and link the library.  timeline: the same kernels
    with the per-work-group timeline marks compiled in (-DFOSCAR_TIMELINE),
    linked as libfoscar_timeline.so; the default library has none."""
    hipcc = _hipcc()
    bdir = BUILD + ("_timeline" if timeline else "")
    lib = LIB_TIMELINE if timeline else LIB
    extra = ["-DFOSCAR_TIMELINE"] if timeline else []
    os.makedirs(bdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(bdir, src + ".o")
        cmd = [hipcc, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = lib + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True, timeline="--timeline" in sys.argv[1:]))
