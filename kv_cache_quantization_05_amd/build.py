"""Build libtq.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m kv_cache_quantization_05_amd.build [--jobs N]

Every translation unit under csrc/ is compiled to an object file (the
general decode kernels, tq_attend_dims.hip, once per head dimension), then
all are linked into kv_cache_quantization_05_amd/libtq.so.  Packed-FP32 VALU
instructions are disabled for device code (-packed-fp32-ops).
"""

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libtq.so")
BUILD = os.path.join(PKG, "_build")
ARCH = "gfx950"

COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
          f"-I{os.path.join(os.path.dirname(PKG), 'include')}"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics",
          # keep MFMA accumulators in ordinary VGPRs (no AGPR copies in loops)
          "-mllvm", "-amdgpu-mfma-vgpr-form"]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


HEAD_DIMS = (32, 64, 128, 256)
PER_DIM = "tq_attend_dims.hip"  # compiled once per head dimension


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def units():
    """(source, extra flags, object name) of every compile job."""
    out = []
    for src in sources():
        if src == PER_DIM:
            out += [(src, [f"-DTQ_HEAD_DIM={d}"], f"{src}.d{d}.o") for d in HEAD_DIMS]
        else:
            out.append((src, [], src + ".o"))
    return out


def _compile(unit):
    src, extra, name = unit
    obj = os.path.join(BUILD, name)
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + extra
    if src.endswith(".hip"):
        cmd += DEVICE
    else:
        cmd += ["-x", "c++", "-D__HIP_PLATFORM_AMD__"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs=8, verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    srcs = units()
    # the slowest units first, so that they do not start last
    srcs.sort(key=lambda u: u[0] != PER_DIM)
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT} from {len(sources())} sources ({len(srcs)} objects)")
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    args = ap.parse_args()
    try:
        build(args.jobs)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
