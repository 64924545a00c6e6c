"""Python binding of the state-space duality prefill (include/samba_ssd.h).

Argument marshalling only: the chunked products run in the HIP kernel of
libsamba_scan.so (loaded through scan.load_library, which raises if the library
is missing: there is no fallback).  torch provides device memory and the
current stream.

Layouts: x, z, y [batch][seqlen][heads][64] or packed [tokens][heads][64] (with
cu_seqlens for several sequences); dt [.., heads]; B, C [.., ngroups][dstate];
A, D, dt_bias fp32 [heads]; states fp32 [nseq][heads][64][dstate].
"""
from __future__ import annotations

import ctypes

from . import scan as _scan
from .scan import SambaError, _check_dev, _dtype_code, _ptr, _stream_handle

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
HEAD_DIM = 64


class SsdArgs(ctypes.Structure):
    """Mirror of samba_ssd_args."""
    _fields_ = [("struct_size", ctypes.c_uint32), ("batch", _I32), ("seqlen", _I32), ("heads", _I32),
                ("head_dim", _I32), ("dstate", _I32), ("ngroups", _I32), ("cu_seqlens", _P), ("nseq", _I32),
                ("y_dtype", _I32), ("x", _P), ("dt", _P), ("z", _P), ("B", _P), ("C", _P), ("A", _P), ("D", _P),
                ("dt_bias", _P), ("h0", _P), ("h_last", _P), ("y", _P), ("workspace", _P),
                ("workspace_bytes", ctypes.c_size_t), ("cb_mode", _I32)]


# samba_ssd_cb_mode: where C Bᵀ is formed
CB_AUTO, CB_PREPASS, CB_IN_KERNEL = 0, 1, 2


_bound = set()


def load_library(path=None):
    """The scan library with the SSD entry point's signature set."""
    lib = _scan.load_library(path)
    if id(lib) not in _bound:
        lib.samba_ssd_fwd.argtypes = [ctypes.POINTER(SsdArgs), _P]
        lib.samba_ssd_fwd.restype = ctypes.c_int
        lib.samba_ssd_workspace_size.argtypes = [ctypes.POINTER(SsdArgs), ctypes.POINTER(ctypes.c_size_t)]
        lib.samba_ssd_workspace_size.restype = ctypes.c_int
        lib.samba_ssd_fwd_noalloc.argtypes = [ctypes.POINTER(SsdArgs), _P]
        lib.samba_ssd_fwd_noalloc.restype = ctypes.c_int
        _bound.add(id(lib))
    return lib


def _shape(x, cu_seqlens):
    """(batch, seqlen, heads, head_dim, nseq) of x."""
    if x.dim() == 4:
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens needs packed [tokens][heads][head_dim] inputs")
        return x.shape[0], x.shape[1], x.shape[2], x.shape[3], x.shape[0]
    if x.dim() == 3:
        return 1, x.shape[0], x.shape[1], x.shape[2], (1 if cu_seqlens is None else cu_seqlens.numel() - 1)
    raise ValueError("x must be [batch][seqlen][heads][head_dim] or [tokens][heads][head_dim]")


def workspace_bytes(a: SsdArgs) -> int:
    n = ctypes.c_size_t(0)
    st = load_library().samba_ssd_workspace_size(ctypes.byref(a), ctypes.byref(n))
    if st != 0:
        raise SambaError(st, "samba_ssd_workspace_size")
    return n.value


def attach_workspace(a: SsdArgs, device, workspace=None):
    """Give the args a workspace of the size the call needs (a new uint8 device tensor unless one is passed);
    returns the tensor, which must outlive the call."""
    import torch
    need = workspace_bytes(a)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    if workspace.numel() < need:
        raise ValueError("workspace too small: %d < %d bytes" % (workspace.numel(), need))
    a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    return workspace


def fwd_args(x, dt, B, C, A, D, dt_bias, *, y, z=None, h0=None, h_last=None, cu_seqlens=None,
             cb_mode: int = CB_AUTO) -> SsdArgs:
    batch, seqlen, heads, hd, nseq = _shape(x, cu_seqlens)
    a = SsdArgs()
    a.struct_size = ctypes.sizeof(SsdArgs)
    a.batch, a.seqlen, a.heads, a.head_dim = batch, seqlen, heads, hd
    a.ngroups, a.dstate = B.shape[-2], B.shape[-1]
    a.cu_seqlens, a.nseq = _ptr(cu_seqlens), (nseq if cu_seqlens is not None else 0)
    a.y_dtype = _dtype_code(y)
    a.x, a.dt, a.z, a.B, a.C = _ptr(x), _ptr(dt), _ptr(z), _ptr(B), _ptr(C)
    a.A, a.D, a.dt_bias = _ptr(A), _ptr(D), _ptr(dt_bias)
    a.h0, a.h_last, a.y = _ptr(h0), _ptr(h_last), _ptr(y)
    a.cb_mode = cb_mode
    return a


def ssd_fwd(x, dt, B, C, A, D, dt_bias, *, z=None, h0=None, h_last=None, y=None, y_dtype=None, cu_seqlens=None,
            return_last_state: bool = True, workspace=None, cb_mode: int = CB_AUTO, stream=None):
    """Chunked SSD prefill through samba_ssd_fwd.  x bf16 [batch][L][heads][64] (or [tokens][heads][64]);
    dt bf16 [.., heads]; B, C bf16 [.., ngroups][dstate] with dstate 64 or 128; z optional (no gate when
    None); workspace: a uint8 device tensor of at least samba_ssd_workspace_size() bytes (allocated per call
    when None and needed); cb_mode: CB_AUTO, CB_PREPASS or CB_IN_KERNEL.  Returns (y, h_last) with h_last
    fp32 [nseq][heads][64][dstate]."""
    import torch
    _check_dev(x, dt, z, B, C, A, D, dt_bias, h0, h_last, y, cu_seqlens)
    batch, seqlen, heads, hd, nseq = _shape(x, cu_seqlens)
    N = B.shape[-1]
    if y is None:
        y = torch.empty(x.shape, dtype=y_dtype or x.dtype, device=x.device)
    if h_last is None and return_last_state:
        h_last = torch.empty(nseq, heads, hd, N, dtype=torch.float32, device=x.device)
    a = fwd_args(x, dt, B, C, A, D, dt_bias, y=y, z=z, h0=h0, h_last=h_last, cu_seqlens=cu_seqlens,
                 cb_mode=cb_mode)
    ws = attach_workspace(a, x.device, workspace)
    st = load_library().samba_ssd_fwd(ctypes.byref(a), _P(_stream_handle(stream)))
    del ws   # torch reuses the freed block only for later work on this stream, which runs after the call
    if st != 0:
        raise SambaError(st, "samba_ssd_fwd")
    return y, h_last


SCRATCH_BYTES = 16 << 20   # SAMBA_SSD_SCRATCH_BYTES


def ssd_fwd_noalloc(x, dt, B, C, A, D, dt_bias, *, z=None, h0=None, h_last=None, y=None, cu_seqlens=None,
                    cb_mode: int = CB_AUTO, stream=None):
    """samba_ssd_fwd_noalloc: as ssd_fwd, but the library's static per-GPU scratch holds the C Bᵀ tiles
    (no workspace; calls needing more than SCRATCH_BYTES are refused).  y and h_last must be given here
    (this wrapper allocates nothing either)."""
    _check_dev(x, dt, z, B, C, A, D, dt_bias, h0, h_last, y, cu_seqlens)
    if y is None:
        raise ValueError("ssd_fwd_noalloc takes a preallocated y")
    a = fwd_args(x, dt, B, C, A, D, dt_bias, y=y, z=z, h0=h0, h_last=h_last, cu_seqlens=cu_seqlens,
                 cb_mode=cb_mode)
    st = load_library().samba_ssd_fwd_noalloc(ctypes.byref(a), _P(_stream_handle(stream)))
    if st != 0:
        raise SambaError(st, "samba_ssd_fwd_noalloc")
    return y, h_last
