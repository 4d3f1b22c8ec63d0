"""Builds libglu_mx.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

Flags:
  --offload-arch=gfx950                      CDNA4 only; no other targets, no host fallback.
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                             no packed FP32 instructions in device code.
  -fno-gpu-flush-denormals-to-zero           FP32 subnormals are kept (BF16 inputs and
                                             outputs have subnormals).
  -fno-fast-math                             the quantizer's decisions rely on IEEE FP32.
Each translation unit is compiled in parallel; the result replaces the old library
atomically.

`python glu_activation_microscaling_amd/build.py --resources` prints the per-kernel resource
table (VGPRs, AGPRs, SGPRs, scratch, spills, LDS, occupancy) that the compiler reports for
these sources with these flags (-Rpass-analysis=kernel-resource-usage).
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libglu_mx.so")
SOURCES = ["api.cpp", "glu_bf16.hip", "glu_mxfp8.hip", "glu_nvfp4.hip", "glu_gemm.hip", "glu_stream.hip"]
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero", "-fno-fast-math",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, "-c", "-x", "hip", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(6, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


_FIELDS = {"VGPRs": "vgpr", "AGPRs": "agpr", "TotalSGPRs": "sgpr", "ScratchSize [bytes/lane]": "scratch",
           "VGPRs Spill": "vgpr_spill", "SGPRs Spill": "sgpr_spill", "LDS Size [bytes/block]": "lds",
           "Occupancy [waves/SIMD]": "occupancy"}


def resource_table():
    """Markdown table of every kernel's resources as the compiler reports them."""
    import re
    rows = []
    for src in SOURCES:
        if not src.endswith(".hip"):
            continue
        cmd = [_hipcc(), *COMMON, "--cuda-device-only", "-c", "-x", "hip", os.path.join(CSRC, src),
               "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        cur = None
        for line in r.stderr.splitlines():
            m = re.search(r"remark: Function Name: (\S+)", line)
            if m:
                cur = {"file": src, "name": m.group(1)}
                rows.append(cur)
                continue
            m = re.search(r"remark:\s+(.+?): (\S+) \[-Rpass", line)
            if m and cur is not None and m.group(1) in _FIELDS:
                cur[_FIELDS[m.group(1)]] = m.group(2)
    names = subprocess.run(["c++filt"], input="\n".join(r["name"] for r in rows), capture_output=True,
                           text=True).stdout.splitlines()
    out = ["| file | kernel | VGPRs | AGPRs | SGPRs | scratch B/lane | VGPR spill | SGPR spill | LDS B | waves/SIMD |",
           "|---|---|---|---|---|---|---|---|---|---|"]
    for r, n in zip(rows, names):
        n = n.replace("glu::(anonymous namespace)::", "").split("(")[0]
        out.append(f"| {r['file']} | `{n}` | {r.get('vgpr')} | {r.get('agpr')} | {r.get('sgpr')} | {r.get('scratch')} | "
                   f"{r.get('vgpr_spill')} | {r.get('sgpr_spill')} | {r.get('lds')} | {r.get('occupancy')} |")
    return "\n".join(out)


def device_asm(src: str) -> str:
    """gfx950 assembly of one kernel source, compiled with the library's flags (device code
    only): what the code-generation tests inspect."""
    cmd = [_hipcc(), *COMMON, "--cuda-device-only", "-S", "-x", "hip", os.path.join(CSRC, src), "-o", "-"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return r.stdout


if __name__ == "__main__":
    if "--resources" in sys.argv:
        print(resource_table())
    else:
        build(verbose="-v" in sys.argv)
        print(LIB)
