"""Build the HIP library for gfx950 with hipcc (in-tree, no JIT).

Each table_*.hip translation unit and the C-ABI unit compile in parallel to
objects under ``_build/``; they link into ``lib/librow_wise_softmax.so``.
Compile flags: -O3 for gfx950, C++17, and the packed-fp32 target feature
switched off (plain fp32 VALU code only).  Never -ffast-math: the -inf
handling relies on IEEE semantics.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "librow_wise_softmax.so")

ARCH = "gfx950"
SOURCES = ["softmax_abi.hip", "table_f32.hip", "table_f16.hip", "table_bf16.hip", "unfused.hip", "attention.hip"]
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-6000:]}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link the shared library. Returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc link failed:\n{r.stderr[-6000:]}")
    os.replace(tmp, LIB)
    return LIB


def resource_usage(out_path: str | None = None) -> str:
    """Compile every HIP source for the device only with the compiler's
    kernel-resource-usage remarks and write a table of each kernel's VGPRs,
    AGPRs, SGPRs, scratch bytes per lane, LDS bytes and the occupancy bound
    (waves per SIMD) those imply.  Returns the table as Markdown; writes it to
    `out_path` if given.  Runs on the CPU (no GPU needed)."""
    import re

    rows = []
    for src in SOURCES:
        cmd = [HIPCC, *COMMON, "--cuda-device-only", "-c", os.path.join(CSRC, src), "-o", os.devnull,
               "-Rpass-analysis=kernel-resource-usage"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-4000:]}")
        cur = None
        for line in r.stderr.splitlines():
            m = re.search(r"Function Name: (\S+)", line)
            if m:
                cur = {"mangled": m.group(1), "src": src}
                rows.append(cur)
                continue
            if cur is None:
                continue
            for key, pat in (("vgpr", r" VGPRs: (\d+)"), ("agpr", r" AGPRs: (\d+)"), ("sgpr", r"TotalSGPRs: (\d+)"),
                             ("vspill", r"VGPRs Spill: (\d+)"), ("sspill", r"SGPRs Spill: (\d+)"),
                             ("scratch", r"ScratchSize \[bytes/lane\]: (\d+)"),
                             ("occupancy", r"Occupancy \[waves/SIMD\]: (\d+)"),
                             ("lds", r"LDS Size \[bytes/block\]: (\d+)")):
                m = re.search(pat, line)
                if m:
                    cur[key] = int(m.group(1))
    names = subprocess.run(["c++filt"], input="\n".join(r["mangled"] for r in rows), capture_output=True,
                           text=True).stdout.splitlines()
    for r, n in zip(rows, names):
        r["name"] = n.replace("void ", "", 1).replace("(anonymous namespace)::", "").split("(")[0]
    rows.sort(key=lambda r: (r["src"], r["name"]))
    out = ["# Register, scratch and LDS use of every kernel, gfx950", "",
           "Command (repository root, CPU only):", "",
           "    python3 -m row_wise_softmax_amd.build --resource-usage", "",
           "From hipcc's `-Rpass-analysis=kernel-resource-usage` remarks with the library's own flags"
           " (`-O3`, packed fp32 off).  Occupancy is the compiler's bound in waves per SIMD (8 at most);"
           " any non-zero scratch would be a register spill.", "",
           "| source | kernel | VGPRs | AGPRs | SGPRs | spilled V/S | scratch B/lane | LDS B | waves/SIMD |",
           "|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {r['src']} | `{r['name']}` | {r.get('vgpr', '')} | {r.get('agpr', '')} | {r.get('sgpr', '')} | "
                   f"{r.get('vspill', '')}/{r.get('sspill', '')} | {r.get('scratch', '')} | {r.get('lds', '')} | "
                   f"{r.get('occupancy', '')} |")
    spills = [r["name"] for r in rows if r.get("scratch", 0) or r.get("vspill", 0) or r.get("sspill", 0)]
    out += ["", f"Kernels: {len(rows)}.  Kernels with scratch memory: "
            f"{sum(1 for r in rows if r.get('scratch', 0))}.  Kernels that spill registers (an SGPR spill goes to"
            f" VGPR lanes, not to memory): {len(spills)}" + (": " + ", ".join(f"`{n}`" for n in spills) if spills else ".")]
    text = "\n".join(out) + "\n"
    if out_path:
        with open(out_path, "w") as f:
            f.write(text)
    return text


if __name__ == "__main__":
    import sys
    if "--resource-usage" in sys.argv:
        path = os.path.join(ROOT, "profiles", "kernel_resources.md")
        resource_usage(path)
        print(path)
    else:
        print(build(verbose=True))
