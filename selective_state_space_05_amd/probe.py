"""Python binding of libsamba_probe.so (include/samba_probe.h): issue-rate probes of the vector ALU forms
the scan's prefill is made of.  Measurement only; the benchmark times each probe launch with HIP events on
the launch stream and turns the instruction count into a rate.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "libsamba_probe.so"
KINDS = {"fmac_vop2": 0, "fma_vop3": 1, "mul_vop2": 2, "fmac_sgpr": 3, "exp": 4, "log": 5, "rcp": 6,
         "add_dpp": 7, "mix_4fmac_1exp": 8}
THREADS_PER_BLOCK = 256
_lib = None


def load_library():
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise ImportError("libsamba_probe.so not built at %s: run python -m selective_state_space_05_amd.build"
                              % LIB_PATH)
        lib = ctypes.CDLL(str(LIB_PATH))
        lib.samba_probe_alu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        lib.samba_probe_alu.restype = ctypes.c_int
        lib.samba_probe_instructions_per_round.argtypes = [ctypes.c_int]
        lib.samba_probe_instructions_per_round.restype = ctypes.c_int
        _lib = lib
    return _lib


def instructions_per_round(kind: str) -> int:
    return load_library().samba_probe_instructions_per_round(KINDS[kind])


def launch(kind: str, blocks: int, iters: int, out, stream) -> None:
    """Enqueue one probe launch; `out` is a float32 device tensor of at least blocks * 256 elements."""
    assert out.numel() >= blocks * THREADS_PER_BLOCK and out.is_cuda
    st = load_library().samba_probe_alu(KINDS[kind], blocks, iters, ctypes.c_void_p(out.data_ptr()),
                                        ctypes.c_void_p(stream.cuda_stream))
    if st != 0:
        raise RuntimeError("samba_probe_alu(%s) failed with %d" % (kind, st))
