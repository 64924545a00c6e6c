"""Builds libsamba_scan.so in-tree with hipcc for gfx950 (the scan and the
sliding-window attention kernels, one library).

Usage:  python -m selective_state_space_05_amd.build   (always recompiles)
"""
from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
SRCS = (PKG / "csrc" / "samba_scan.hip", PKG / "csrc" / "samba_scan_groups.hip", PKG / "csrc" / "samba_swa.hip",
        PKG / "csrc" / "samba_ssd.hip", PKG / "csrc" / "samba_gla.hip")
HEADERS = (ROOT / "include" / "samba_scan.h", ROOT / "include" / "samba_swa.h", ROOT / "include" / "samba_ssd.h",
           ROOT / "include" / "samba_gla.h")
LIB = PKG / "libsamba_scan.so"

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep the compiler from emitting packed fp32 ALU forms (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (Path(cand).exists() or cand == "hipcc"):
            return cand
    raise FileNotFoundError("hipcc not found")


def build(out: Path = LIB, extra=()) -> Path:
    """Compile the HIP library (kernels + C ABI) into `out`."""
    tmp = out.with_suffix(".so.tmp%d" % os.getpid())
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", str(ROOT / "include"), "-o", str(tmp), *(str(p) for p in SRCS)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(), file=sys.stderr)
