"""Build libtp.so (the HIP/gfx950 library behind include/tp.h) with hipcc.

Every .hip file under csrc/ is compiled for gfx950 into _build/ and linked
into transformer_tensor_shard_amd/libtp.so.  hipcc cross-compiles, so this
runs on a machine without a GPU.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtp.so")
ARCH = os.environ.get("TP_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtp.so)")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-fvisibility=hidden", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            # packed f32 instructions stay off: hipcc must not emit v_pk_*_f32
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"]


# Per-source code-generation options.  The attention kernels keep their MFMA
# accumulators in VGPRs (the default AGPR form costs hundreds of register
# moves per tile there, to zero the score accumulators and to read them for
# the exponentials).
FILE_FLAGS = {"attention_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
              "attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *_flags(), *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def resource_usage(name: str) -> dict:
    """Per-kernel register and scratch use of csrc/<name>, as the compiler
    reports it (device code only, same flags as the library build):
    {mangled kernel name: {"VGPRs": int, "AGPRs": int, "ScratchSize": int
    (bytes per lane), "VGPRs Spill": int, "Occupancy": int (waves per SIMD),
    "LDS Size": int (bytes per workgroup)}}."""
    import re
    import tempfile
    src = os.path.join(CSRC, name)
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [hipcc(), *_flags(), *FILE_FLAGS.get(name, []), "--cuda-device-only",
               "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o",
               os.path.join(tmp, "dev.o")]
        r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    out, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark:\s+(.*?)\s*\[-Rpass-analysis", line)
        if not m:
            continue
        text = m.group(1)
        if text.startswith("Function Name:"):
            cur = out.setdefault(text.split(":", 1)[1].strip(), {})
            continue
        key, _, val = text.rpartition(":")
        key = re.sub(r"\s*\[.*\]", "", key).strip()
        if cur is not None and val.strip().isdigit():
            cur[key] = int(val)
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
