"""Builds libsamba_scan.so in-tree with hipcc for gfx950 (the scan and the
sliding-window attention kernels, one library), and libsamba_probe.so (the
ALU issue-rate probes the benchmark measures the prefill's ceiling with).

Usage:  python -m selective_state_space_05_amd.build   (always recompiles)
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
SRCS = tuple(PKG / "csrc" / n for n in ("samba_scan.hip", "samba_scan_fwd_ilp.hip", "samba_scan_groups.hip",
                                         "samba_swa.hip", "samba_ssd.hip", "samba_gla.hip"))
# Flags for single sources: the inference copy of the prefill kernel is scheduled by LLVM's max-ILP machine
# scheduler (same instructions, another order; measured faster for those launch plans only).
SRC_FLAGS = {PKG / "csrc" / "samba_scan_fwd_ilp.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}
HEADERS = (ROOT / "include" / "samba_scan.h", ROOT / "include" / "samba_swa.h", ROOT / "include" / "samba_ssd.h",
           ROOT / "include" / "samba_gla.h")
LIB = PKG / "libsamba_scan.so"
PROBE_SRC = PKG / "csrc" / "samba_probe.hip"
PROBE_LIB = PKG / "libsamba_probe.so"

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
COMPILE_FLAGS = [f for f in HIPCC_FLAGS if f != "-shared"]   # one source to one object
LINK_FLAGS = ["--offload-arch=gfx950", "-fPIC", "-shared"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (Path(cand).exists() or cand == "hipcc"):
            return cand
    raise FileNotFoundError("hipcc not found")


def _run(cmd) -> None:
    res = subprocess.run([str(c) for c in cmd], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(str(c) for c in cmd) + "\n" + res.stdout + res.stderr)


def _compile(srcs, out: Path, extra=()) -> Path:
    """Each source to an object (with its SRC_FLAGS), compiled in parallel, then linked into `out`."""
    tmp = out.with_suffix(".so.tmp%d" % os.getpid())
    with tempfile.TemporaryDirectory(prefix="samba_build_") as objdir:
        objs = [Path(objdir) / ("%d_%s.o" % (i, Path(src).stem)) for i, src in enumerate(srcs)]
        jobs = [[hipcc(), *COMPILE_FLAGS, *extra, *SRC_FLAGS.get(Path(src), ()), "-I", ROOT / "include", "-c",
                 "-o", obj, src] for obj, src in zip(objs, srcs)]
        with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1, 8)) as pool:
            list(pool.map(_run, jobs))
        _run([hipcc(), *LINK_FLAGS, "-o", tmp, *objs])
    os.replace(tmp, out)
    return out


def build(out: Path = LIB, extra=(), probe: bool = True) -> Path:
    """Compile the HIP library (kernels + C ABI) into `out`, and the ALU probe library beside it."""
    _compile(SRCS, out, extra)
    if probe:
        _compile((PROBE_SRC,), PROBE_LIB, extra)
    return out


# Host-side sanitizers only: the device code is built as usual; -Xarch_host applies each flag to the host
# compilation (validation, launch plans, the C ABI), which the ABI tests then exercise.
SANITIZER_FLAGS = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libasan"]


def asan_runtime() -> Path:
    """The clang AddressSanitizer runtime a process must preload to load the sanitized library."""
    cands = sorted(Path("/opt/rocm/llvm/lib/clang").glob("*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not cands:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm/lib/clang")
    return cands[-1]


def build_sanitized(out: Path) -> Path:
    """libsamba_scan.so with AddressSanitizer and UndefinedBehaviorSanitizer on its host code, at `out` (one
    hipcc command; without SRC_FLAGS, which only order the device instructions)."""
    flags = [f for f in HIPCC_FLAGS if f != "-O3"] + SANITIZER_FLAGS
    tmp = Path(out).with_suffix(".so.tmp%d" % os.getpid())
    cmd = [hipcc(), *flags, "-I", str(ROOT / "include"), "-o", str(tmp), *(str(p) for p in SRCS)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    os.replace(tmp, out)
    return Path(out)


if __name__ == "__main__":
    print(build(), file=sys.stderr)
