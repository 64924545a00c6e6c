"""Python binding of gated linear attention (include/samba_gla.h).

Argument marshalling only: the layer runs in the HIP kernels of libsamba_scan.so (loaded through
scan.load_library, which raises if the library is missing: there is no fallback), as the chunked form (bf16
inputs, 128 or 256 keys, value sizes a multiple of 32; needs a workspace) or as the recurrence (the other
shapes).  torch provides device memory, the workspace and the current stream.

Layouts: q, k, gk [batch][seqlen][heads][dstate] or packed [tokens][heads][dstate] (with cu_seqlens for
several sequences); v, o [.., heads][head_dim]; states fp32 [nseq][heads][head_dim][dstate].
"""
from __future__ import annotations

import ctypes

from . import scan as _scan
from .scan import SambaError, _check_dev, _dtype_code, _ptr, _stream_handle

_P = ctypes.c_void_p
_I32 = ctypes.c_int32


class GlaArgs(ctypes.Structure):
    """Mirror of samba_gla_args."""
    _fields_ = [("struct_size", ctypes.c_uint32), ("batch", _I32), ("seqlen", _I32), ("heads", _I32),
                ("head_dim", _I32), ("dstate", _I32), ("cu_seqlens", _P), ("nseq", _I32), ("in_dtype", _I32),
                ("y_dtype", _I32), ("q", _P), ("k", _P), ("gk", _P), ("v", _P), ("h0", _P), ("h_last", _P),
                ("o", _P), ("workspace", _P), ("workspace_bytes", ctypes.c_size_t)]


_bound = set()


def load_library(path=None):
    """The scan library with the GLA entry point's signature set."""
    lib = _scan.load_library(path)
    if id(lib) not in _bound:
        lib.samba_gla_fwd.argtypes = [ctypes.POINTER(GlaArgs), _P]
        lib.samba_gla_fwd.restype = ctypes.c_int
        lib.samba_gla_workspace_size.argtypes = [ctypes.POINTER(GlaArgs), ctypes.POINTER(ctypes.c_size_t)]
        lib.samba_gla_workspace_size.restype = ctypes.c_int
        _bound.add(id(lib))
    return lib


def _shape(v, cu_seqlens):
    """(batch, seqlen, heads, head_dim, nseq) of v."""
    if v.dim() == 4:
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens needs packed [tokens][heads][head_dim] inputs")
        return v.shape[0], v.shape[1], v.shape[2], v.shape[3], v.shape[0]
    if v.dim() == 3:
        return 1, v.shape[0], v.shape[1], v.shape[2], (1 if cu_seqlens is None else cu_seqlens.numel() - 1)
    raise ValueError("v must be [batch][seqlen][heads][head_dim] or [tokens][heads][head_dim]")


def workspace_bytes(a: GlaArgs) -> int:
    n = ctypes.c_size_t(0)
    st = load_library().samba_gla_workspace_size(ctypes.byref(a), ctypes.byref(n))
    if st != 0:
        raise SambaError(st, "samba_gla_workspace_size")
    return n.value


def attach_workspace(a: GlaArgs, device, workspace=None):
    """Give the args a workspace of the size the call needs (a new uint8 device tensor unless one is passed;
    none when the call needs none); returns the tensor, which must outlive the call."""
    import torch
    need = workspace_bytes(a)
    if workspace is None:
        if need == 0:
            return None
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if workspace.numel() < need:
        raise ValueError("workspace too small: %d < %d bytes" % (workspace.numel(), need))
    a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    return workspace


def fwd_args(q, k, v, gk, *, o, h0=None, h_last=None, cu_seqlens=None) -> GlaArgs:
    batch, seqlen, heads, hd, nseq = _shape(v, cu_seqlens)
    a = GlaArgs()
    a.struct_size = ctypes.sizeof(GlaArgs)
    a.batch, a.seqlen, a.heads, a.head_dim, a.dstate = batch, seqlen, heads, hd, q.shape[-1]
    a.cu_seqlens, a.nseq = _ptr(cu_seqlens), (nseq if cu_seqlens is not None else 0)
    a.in_dtype, a.y_dtype = _dtype_code(v), _dtype_code(o)
    a.q, a.k, a.gk, a.v = _ptr(q), _ptr(k), _ptr(gk), _ptr(v)
    a.h0, a.h_last, a.o = _ptr(h0), _ptr(h_last), _ptr(o)
    return a


def gla_fwd(q, k, v, gk, *, h0=None, h_last=None, o=None, y_dtype=None, cu_seqlens=None,
            return_last_state: bool = True, workspace=None, stream=None):
    """GLA through samba_gla_fwd: q, k, gk [batch][L][heads][N] (N = 16 .. 256; gk the log decay), v
    [batch][L][heads][P] (P a multiple of 256 / N), all bf16 or all fp32.  Returns (o, h_last) with h_last
    fp32 [nseq][heads][P][N]."""
    import torch
    _check_dev(q, k, v, gk, h0, h_last, o, cu_seqlens)
    batch, seqlen, heads, hd, nseq = _shape(v, cu_seqlens)
    N = q.shape[-1]
    if o is None:
        o = torch.empty(v.shape, dtype=y_dtype or v.dtype, device=v.device)
    if h_last is None and return_last_state:
        h_last = torch.empty(nseq, heads, hd, N, dtype=torch.float32, device=v.device)
    a = fwd_args(q, k, v, gk, o=o, h0=h0, h_last=h_last, cu_seqlens=cu_seqlens)
    ws = attach_workspace(a, v.device, workspace)
    st = load_library().samba_gla_fwd(ctypes.byref(a), _P(_stream_handle(stream)))
    if st != 0:
        raise SambaError(st, "samba_gla_fwd")
    del ws   # (the stream orders any later reuse of its memory after the call)
    return o, h_last
