"""Build libvarlen_attn.so in-tree with hipcc for gfx950.

Every HIP source is compiled for gfx950 only, with packed fp32 instructions
disabled (the compiler may otherwise fuse pairs of fp32 operations into
v_pk_* forms), then linked into one shared library next to this file.

    python -m packed_varlen_scaled_amd.build [--jobs N] [--verbose]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB_NAME = "libvarlen_attn.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
# Per-kernel register / scratch use reported by the compiler for the last build.
RESOURCES_PATH = os.path.join(HERE, "libvarlen_attn.resources.json")
BUILD_DIR = os.path.join(ROOT, "_build")

HIP_SOURCES = ["prefill_mfma.hip", "decode.hip", "prefill_f32.hip", "sched.hip", "rope_append.hip"]
HOST_SOURCES = ["varlen_attn.cpp"]
ARCH = "gfx950"


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else (shutil.which("hipcc") or "hipcc")


COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, verbose: bool):
    """Compile one source; returns (object path, kernel resource records)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc()] + COMMON + DEVICE + ["-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(CSRC, src),
                                          "-o", obj]
    if src.endswith(".cpp"):
        cmd = [_hipcc()] + COMMON + ["-x", "hip"] + DEVICE + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj, _parse_resources(res.stderr, src)


_FIELDS = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch_bytes_per_lane",
           "VGPRs Spill": "vgpr_spill", "SGPRs Spill": "sgpr_spill", "Occupancy [waves/SIMD]": "waves_per_simd",
           "LDS Size [bytes/block]": "lds_bytes"}


def _parse_resources(text: str, src: str):
    """Records of the compiler's kernel-resource-usage remarks, one per kernel."""
    out, cur = [], None
    for line in text.splitlines():
        m = re.search(r"remark:\s+(.*?):\s+(\S+)\s*\[-Rpass-analysis", line)
        if not m:
            continue
        key, val = m.group(1).strip(), m.group(2)
        if key == "Function Name":
            cur = {"source": src, "kernel": val}
            out.append(cur)
        elif cur is not None and key in _FIELDS:
            try:
                cur[_FIELDS[key]] = int(val)
            except ValueError:
                pass
    return out


def build(jobs: int = 4, verbose: bool = False) -> str:
    """Compile every source and link the shared library. Returns its path."""
    srcs = HIP_SOURCES + HOST_SOURCES
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose), srcs))
    objs = [r[0] for r in results]
    resources = [rec for r in results for rec in r[1]]
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    missing = undefined_kernel_stubs(tmp)
    if missing:
        os.unlink(tmp)
        raise RuntimeError("kernel launch stubs left undefined (a kernel body was dropped by the host "
                           "compile): " + ", ".join(missing[:4]))
    os.replace(tmp, LIB_PATH)
    with open(RESOURCES_PATH + ".tmp", "w") as f:
        json.dump(resources, f, indent=1)
    os.replace(RESOURCES_PATH + ".tmp", RESOURCES_PATH)
    return LIB_PATH


def undefined_kernel_stubs(lib_path: str):
    """Names of kernel launch stubs the library references but does not define."""
    nm = shutil.which("nm") or os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "llvm-nm")
    res = subprocess.run([nm, "-C", lib_path], capture_output=True, text=True, check=True)
    return [line.split(" U ", 1)[1] for line in res.stdout.splitlines()
            if " U " in line and "__device_stub__" in line]


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 4))
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    path = build(a.jobs, a.verbose)
    print(path)
    return 0


if __name__ == "__main__":
    sys.exit(main())
