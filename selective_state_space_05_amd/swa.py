"""Python binding of the sliding-window attention entry points (include/samba_swa.h).

Argument marshalling only: RoPE, the prefill attention and the decode step run
in the HIP kernels of libsamba_scan.so (loaded through scan.load_library, which
raises if the library is missing: there is no fallback).  torch provides device
memory and the current stream.

Layouts: q, k, v are bf16 [batch][seqlen][heads][head_dim] or packed
[tokens][heads][head_dim] (with cu_seqlens for several sequences); RoPE tables
are fp32 [npos][head_dim / 2].
"""
from __future__ import annotations

import ctypes

from . import scan as _scan
from .scan import SambaError, _check_dev, _dtype_code, _ptr, _stream_handle

_P = ctypes.c_void_p
_I32 = ctypes.c_int32


class RopeArgs(ctypes.Structure):
    """Mirror of samba_rope_args."""
    _fields_ = [("struct_size", ctypes.c_uint32), ("batch", _I32), ("seqlen", _I32), ("heads", _I32),
                ("head_dim", _I32), ("cu_seqlens", _P), ("nseq", _I32), ("pos0", _P), ("cos", _P), ("sin", _P),
                ("npos", _I32), ("q_in", _P), ("k_in", _P), ("q_out", _P), ("k_out", _P)]


class SwaFwdArgs(ctypes.Structure):
    """Mirror of samba_swa_fwd_args."""
    _fields_ = [("struct_size", ctypes.c_uint32), ("batch", _I32), ("seqlen", _I32), ("heads", _I32),
                ("head_dim", _I32), ("cu_seqlens", _P), ("nseq", _I32), ("window", _I32), ("out_dtype", _I32),
                ("q", _P), ("k", _P), ("v", _P), ("o", _P)]


class SwaDecodeArgs(ctypes.Structure):
    """Mirror of samba_swa_decode_args."""
    _fields_ = [("struct_size", ctypes.c_uint32), ("batch", _I32), ("heads", _I32), ("head_dim", _I32),
                ("window", _I32), ("cache_len", _I32), ("out_dtype", _I32), ("pos", _P), ("q", _P), ("k", _P),
                ("v", _P), ("k_cache", _P), ("v_cache", _P), ("o", _P)]


_bound = set()


def load_library(path=None):
    """The scan library with the attention entry points' signatures set."""
    lib = _scan.load_library(path)
    if id(lib) not in _bound:
        lib.samba_rope.argtypes = [ctypes.POINTER(RopeArgs), _P]
        lib.samba_rope.restype = ctypes.c_int
        lib.samba_swa_fwd.argtypes = [ctypes.POINTER(SwaFwdArgs), _P]
        lib.samba_swa_fwd.restype = ctypes.c_int
        lib.samba_swa_decode.argtypes = [ctypes.POINTER(SwaDecodeArgs), _P]
        lib.samba_swa_decode.restype = ctypes.c_int
        _bound.add(id(lib))
    return lib


def _tok_shape(x, cu_seqlens):
    """(batch, seqlen, heads, head_dim, nseq) of a q/k/v tensor."""
    if x.dim() == 4:
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens needs packed [tokens][heads][head_dim] inputs")
        return x.shape[0], x.shape[1], x.shape[2], x.shape[3], x.shape[0]
    if x.dim() == 3:
        return 1, x.shape[0], x.shape[1], x.shape[2], (1 if cu_seqlens is None else cu_seqlens.numel() - 1)
    raise ValueError("q/k/v must be [batch][seqlen][heads][head_dim] or [tokens][heads][head_dim]")


def rope_args(q, k, cos, sin, *, q_out, k_out, cu_seqlens=None, pos0=None) -> RopeArgs:
    ref = q if q is not None else k
    batch, seqlen, heads, hd, nseq = _tok_shape(ref, cu_seqlens)
    a = RopeArgs()
    a.struct_size = ctypes.sizeof(RopeArgs)
    a.batch, a.seqlen, a.heads, a.head_dim = batch, seqlen, heads, hd
    a.cu_seqlens, a.nseq = _ptr(cu_seqlens), (nseq if cu_seqlens is not None else 0)
    a.pos0 = _ptr(pos0)
    a.cos, a.sin, a.npos = _ptr(cos), _ptr(sin), cos.shape[0]
    a.q_in, a.k_in, a.q_out, a.k_out = _ptr(q), _ptr(k), _ptr(q_out), _ptr(k_out)
    return a


def rope(q, k, cos, sin, *, cu_seqlens=None, pos0=None, q_out=None, k_out=None, in_place=False, stream=None):
    """Rotate q and k (either may be None) by each token's position inside its sequence (+ pos0[s]).
    Returns (q_rot, k_rot): new tensors, the given outputs, or q and k themselves with in_place=True."""
    import torch
    _check_dev(q, k, cos, sin, cu_seqlens, pos0, q_out, k_out)
    if in_place:
        q_out, k_out = q, k
    else:
        q_out = torch.empty_like(q) if (q is not None and q_out is None) else q_out
        k_out = torch.empty_like(k) if (k is not None and k_out is None) else k_out
    a = rope_args(q, k, cos, sin, q_out=q_out, k_out=k_out, cu_seqlens=cu_seqlens, pos0=pos0)
    st = load_library().samba_rope(ctypes.byref(a), _P(_stream_handle(stream)))
    if st != 0:
        raise SambaError(st, "samba_rope")
    return q_out, k_out


def fwd_args(q, k, v, window: int, *, o, cu_seqlens=None) -> SwaFwdArgs:
    batch, seqlen, heads, hd, nseq = _tok_shape(q, cu_seqlens)
    a = SwaFwdArgs()
    a.struct_size = ctypes.sizeof(SwaFwdArgs)
    a.batch, a.seqlen, a.heads, a.head_dim = batch, seqlen, heads, hd
    a.cu_seqlens, a.nseq = _ptr(cu_seqlens), (nseq if cu_seqlens is not None else 0)
    a.window = int(window)
    a.out_dtype = _dtype_code(o)
    a.q, a.k, a.v, a.o = _ptr(q), _ptr(k), _ptr(v), _ptr(o)
    return a


def swa_fwd(q, k, v, window: int, *, cu_seqlens=None, o=None, out_dtype=None, stream=None):
    """Sliding-window attention of rotated q, k and v (bf16): query i sees keys i-window .. i of its sequence.
    Returns o, shaped like q, in out_dtype (default bf16)."""
    import torch
    _check_dev(q, k, v, cu_seqlens, o)
    o = torch.empty(q.shape, dtype=out_dtype or torch.bfloat16, device=q.device) if o is None else o
    a = fwd_args(q, k, v, window, o=o, cu_seqlens=cu_seqlens)
    st = load_library().samba_swa_fwd(ctypes.byref(a), _P(_stream_handle(stream)))
    if st != 0:
        raise SambaError(st, "samba_swa_fwd")
    return o


def attention(q, k, v, window: int, cos, sin, *, cu_seqlens=None, out_dtype=None, stream=None):
    """RoPE then sliding-window attention (two library calls); q and k are left unrotated."""
    qr, kr = rope(q, k, cos, sin, cu_seqlens=cu_seqlens, stream=stream)
    return swa_fwd(qr, kr, v, window, cu_seqlens=cu_seqlens, out_dtype=out_dtype, stream=stream)


def decode_args(q, k, v, k_cache, v_cache, pos, window: int, *, o) -> SwaDecodeArgs:
    a = SwaDecodeArgs()
    a.struct_size = ctypes.sizeof(SwaDecodeArgs)
    a.batch, a.heads, a.head_dim = q.shape[0], q.shape[1], q.shape[2]
    a.window, a.cache_len = int(window), k_cache.shape[2]
    a.out_dtype = _dtype_code(o)
    a.pos, a.q, a.k, a.v = _ptr(pos), _ptr(q), _ptr(k), _ptr(v)
    a.k_cache, a.v_cache, a.o = _ptr(k_cache), _ptr(v_cache), _ptr(o)
    return a


def swa_decode(q, k, v, k_cache, v_cache, pos, window: int, *, o=None, out_dtype=None, stream=None):
    """One decode step: q, k, v [batch][heads][head_dim] (q, k rotated at pos), caches
    [batch][heads][cache_len][head_dim] updated in place at slot pos % cache_len; pos int32 [batch].
    Returns o [batch][heads][head_dim]."""
    import torch
    _check_dev(q, k, v, k_cache, v_cache, pos, o)
    o = torch.empty(q.shape, dtype=out_dtype or torch.bfloat16, device=q.device) if o is None else o
    a = decode_args(q, k, v, k_cache, v_cache, pos, window, o=o)
    st = load_library().samba_swa_decode(ctypes.byref(a), _P(_stream_handle(stream)))
    if st != 0:
        raise SambaError(st, "samba_swa_decode")
    return o
