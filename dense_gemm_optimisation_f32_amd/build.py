"""Build libmi355gemm.so (the HIP kernels plus the C ABI) in-tree for gfx950.

    python -m dense_gemm_optimisation_f32_amd.build

Every source under csrc/ is compiled by hipcc to an object under _build/, in
parallel, and the objects are linked into dense_gemm_optimisation_f32_amd/
libmi355gemm.so.  Packed fp32 VALU instructions are disabled for the device
code (-target-feature -packed-fp32-ops); hipcc's host pass warns that it does
not know that feature, which is harmless.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmi355gemm.so")
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-command-line-argument"]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def resource_usage() -> list[dict]:
    """The compiler's resource usage of every kernel in the HIP sources, from hipcc's
    kernel-resource-usage remarks (device code only, nothing written): per kernel its
    demangled name and the remark fields as printed (VGPRs, AGPRs, TotalSGPRs,
    "ScratchSize [bytes/lane]", "Occupancy [waves/SIMD]", "VGPRs Spill", "SGPRs Spill",
    "LDS Size [bytes/block]")."""
    import re

    recs = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        cmd = [HIPCC, *COMMON, "--cuda-device-only", "-Rpass-analysis=kernel-resource-usage", "-c", src,
               "-o", os.devnull]
        out = subprocess.run(cmd, capture_output=True, text=True)
        if out.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{out.stderr[-2000:]}")
        cur = None
        for line in out.stderr.splitlines():
            m = re.search(r"remark: Function Name: (\S+)", line)
            if m:
                cur = {"symbol": m.group(1), "source": os.path.basename(src)}
                recs.append(cur)
                continue
            m = re.search(r"remark:\s+(.+?): (\S+) \[-Rpass-analysis", line)
            if m and cur is not None:
                cur[m.group(1).strip()] = m.group(2)
    filt = shutil.which("c++filt") or shutil.which("llvm-cxxfilt")
    names = [r["symbol"] for r in recs]
    if filt:
        names = subprocess.run([filt], input="\n".join(names), capture_output=True, text=True,
                               check=True).stdout.splitlines()
    for r, n in zip(recs, names):
        r["kernel"] = n
    return recs


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs = []
    objs = []
    for src in sources():
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        cmd = [HIPCC, *COMMON, *(extra or []), "-c", src, "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = []
    for src, pr in procs:
        out, _ = pr.communicate()
        lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
        if pr.returncode != 0:
            failed.append(src)
            sys.stderr.write("\n".join(lines) + "\n")
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError(f"hipcc failed on {failed}")
    tmp = LIB + ".tmp"
    link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
