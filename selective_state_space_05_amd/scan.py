"""Python binding of libsamba_scan.so (the C ABI in include/samba_scan.h; the
attention entry points of include/samba_swa.h are bound in swa.py, the state-space
duality prefill of include/samba_ssd.h in ssd.py, gated linear attention of include/samba_gla.h in gla.py).

Argument marshalling only: every step of the scan runs in the HIP kernels of
the shared library.  torch provides device memory and the current stream.  If
the library is missing, loading raises immediately; there is no fallback.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "libsamba_scan.so"
DSTATE = 16
ABI_VERSION = 13

SAMBA_F32, SAMBA_BF16 = 0, 1
STATUS_NAMES = {0: "SAMBA_OK", 1: "SAMBA_ERR_NULL_ARG", 2: "SAMBA_ERR_BAD_SHAPE", 3: "SAMBA_ERR_BAD_DTYPE",
                4: "SAMBA_ERR_MISALIGNED", 5: "SAMBA_ERR_ALIASING", 6: "SAMBA_ERR_UNSUPPORTED",
                7: "SAMBA_ERR_BAD_STRUCT", 8: "SAMBA_ERR_HIP", 9: "SAMBA_ERR_WORKSPACE"}
EXPORTED = ("samba_scan_fwd", "samba_scan_step", "samba_scan_fwd_plan", "samba_scan_bwd",
            "samba_scan_bwd_workspace_size", "samba_scan_ckpt_bytes", "samba_proj", "samba_status_string",
            "samba_scan_abi_version", "samba_rope", "samba_swa_fwd", "samba_swa_decode", "samba_scan_fwd_groups",
            "samba_scan_step_groups", "samba_ssd_fwd", "samba_ssd_workspace_size", "samba_ssd_fwd_noalloc",
            "samba_gla_fwd", "samba_gla_workspace_size")

_P = ctypes.c_void_p
_I32 = ctypes.c_int32


class FwdArgs(ctypes.Structure):
    """Mirror of samba_scan_fwd_args."""
    _fields_ = [("struct_size", ctypes.c_uint32), ("batch", _I32), ("seqlen", _I32), ("dim", _I32),
                ("dstate", _I32), ("cu_seqlens", _P), ("nseq", _I32), ("in_dtype", _I32), ("y_dtype", _I32),
                ("time_slices", _I32), ("x", _P), ("dt", _P), ("z", _P), ("B", _P), ("C", _P), ("A", _P),
                ("D", _P), ("dt_bias", _P), ("h0", _P), ("h_last", _P), ("y", _P), ("h_ckpt", _P),
                ("lanes_per_channel", _I32)]


class StepArgs(ctypes.Structure):
    """Mirror of samba_scan_step_args."""
    _fields_ = [("struct_size", ctypes.c_uint32), ("batch", _I32), ("dim", _I32), ("dstate", _I32),
                ("in_dtype", _I32), ("y_dtype", _I32), ("state", _P), ("x", _P), ("dt", _P), ("z", _P),
                ("B", _P), ("C", _P), ("A", _P), ("D", _P), ("dt_bias", _P), ("y", _P)]


class BwdArgs(ctypes.Structure):
    """Mirror of samba_scan_bwd_args."""
    _fields_ = [("struct_size", ctypes.c_uint32), ("batch", _I32), ("seqlen", _I32), ("dim", _I32),
                ("dstate", _I32), ("cu_seqlens", _P), ("nseq", _I32), ("in_dtype", _I32), ("time_slices", _I32),
                ("x", _P), ("dt", _P), ("z", _P), ("B", _P), ("C", _P), ("A", _P), ("D", _P), ("dt_bias", _P),
                ("h0", _P), ("dy", _P), ("dh_last", _P), ("h_ckpt", _P), ("dx", _P), ("ddt", _P), ("dz", _P), ("dB", _P),
                ("dC", _P), ("dA", _P), ("dD", _P), ("ddt_bias", _P), ("dh0", _P), ("workspace", _P),
                ("workspace_bytes", ctypes.c_size_t)]


class ProjArgs(ctypes.Structure):
    """Mirror of samba_proj_args."""
    _fields_ = [("struct_size", ctypes.c_uint32), ("tokens", _I32), ("dim", _I32), ("dstate", _I32),
                ("in_dtype", _I32), ("out_dtype", _I32), ("x", _P), ("W", _P), ("dt", _P), ("B", _P), ("C", _P)]


class GroupsArgs(ctypes.Structure):
    """Mirror of samba_scan_groups_args."""
    _fields_ = [("struct_size", ctypes.c_uint32), ("batch", _I32), ("seqlen", _I32), ("dim", _I32),
                ("dstate", _I32), ("ngroups", _I32), ("cu_seqlens", _P), ("nseq", _I32), ("in_dtype", _I32),
                ("y_dtype", _I32), ("x", _P), ("dt", _P), ("z", _P), ("B", _P), ("C", _P), ("A", _P), ("D", _P),
                ("dt_bias", _P), ("h0", _P), ("h_last", _P), ("y", _P)]


class StepGroupsArgs(ctypes.Structure):
    """Mirror of samba_scan_step_groups_args."""
    _fields_ = [("struct_size", ctypes.c_uint32), ("batch", _I32), ("dim", _I32), ("dstate", _I32),
                ("ngroups", _I32), ("in_dtype", _I32), ("y_dtype", _I32), ("state", _P), ("x", _P), ("dt", _P),
                ("z", _P), ("B", _P), ("C", _P), ("A", _P), ("D", _P), ("dt_bias", _P), ("y", _P)]


class SambaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: %s (%s)" % (what, STATUS_NAMES.get(status, status), _status_string(status)))


_lib = None
_libs_by_path = {}


def load_library(path: Path | str | None = None):
    """Load libsamba_scan.so (or the library at `path`, one shared handle per path, so that the other
    bindings' signatures land on the same object); raises (no fallback) if it is absent or stale."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    if path is not None and str(Path(path).resolve()) in _libs_by_path:
        return _libs_by_path[str(Path(path).resolve())]
    p = Path(path) if path is not None else LIB_PATH
    if not p.exists():
        raise ImportError("libsamba_scan.so not built at %s: run __graft_entry__.build() or "
                          "python -m selective_state_space_05_amd.build" % p)
    lib = ctypes.CDLL(str(p))
    lib.samba_scan_fwd.argtypes = [ctypes.POINTER(FwdArgs), _P]
    lib.samba_scan_fwd.restype = ctypes.c_int
    lib.samba_scan_step.argtypes = [ctypes.POINTER(StepArgs), _P]
    lib.samba_scan_step.restype = ctypes.c_int
    lib.samba_scan_fwd_plan.argtypes = [ctypes.POINTER(FwdArgs), ctypes.POINTER(_I32), ctypes.POINTER(_I32),
                                        ctypes.POINTER(_I32), ctypes.POINTER(_I32)]
    lib.samba_scan_fwd_plan.restype = ctypes.c_int
    lib.samba_scan_bwd.argtypes = [ctypes.POINTER(BwdArgs), _P]
    lib.samba_scan_bwd.restype = ctypes.c_int
    lib.samba_scan_bwd_workspace_size.argtypes = [ctypes.POINTER(BwdArgs), ctypes.POINTER(ctypes.c_size_t)]
    lib.samba_scan_bwd_workspace_size.restype = ctypes.c_int
    lib.samba_scan_ckpt_bytes.argtypes = [_I32, _I32, _I32, _I32, ctypes.POINTER(ctypes.c_size_t)]
    lib.samba_scan_ckpt_bytes.restype = ctypes.c_int
    lib.samba_proj.argtypes = [ctypes.POINTER(ProjArgs), _P]
    lib.samba_proj.restype = ctypes.c_int
    lib.samba_scan_fwd_groups.argtypes = [ctypes.POINTER(GroupsArgs), _P]
    lib.samba_scan_fwd_groups.restype = ctypes.c_int
    lib.samba_scan_step_groups.argtypes = [ctypes.POINTER(StepGroupsArgs), _P]
    lib.samba_scan_step_groups.restype = ctypes.c_int
    lib.samba_status_string.argtypes = [ctypes.c_int]
    lib.samba_status_string.restype = ctypes.c_char_p
    lib.samba_scan_abi_version.restype = ctypes.c_int
    if lib.samba_scan_abi_version() != ABI_VERSION:
        raise ImportError("libsamba_scan.so ABI %d != binding ABI %d" % (lib.samba_scan_abi_version(), ABI_VERSION))
    if path is None:
        _lib = lib
    else:
        _libs_by_path[str(Path(path).resolve())] = lib
    return lib


def _status_string(status: int) -> str:
    try:
        return load_library().samba_status_string(status).decode()
    except Exception:
        return "?"


# --------------------------------------------------------------------------- #
# torch marshalling
# --------------------------------------------------------------------------- #
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return SAMBA_BF16
    if t.dtype == torch.float32:
        return SAMBA_F32
    raise TypeError("unsupported dtype %s (bf16 or fp32)" % t.dtype)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check_dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _stream_handle(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _seq_shape(x, cu_seqlens):
    """(batch, seqlen, dim, nseq) of the token layout."""
    if x.dim() == 3:
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens needs packed [tokens][dim] inputs")
        return x.shape[0], x.shape[1], x.shape[2], x.shape[0]
    if x.dim() == 2:
        return 1, x.shape[0], x.shape[1], (1 if cu_seqlens is None else cu_seqlens.numel() - 1)
    raise ValueError("x must be [batch][seqlen][dim] or [tokens][dim]")


def alloc_ckpt(x, cu_seqlens=None):
    """An h_ckpt array for these inputs: fp32 [slots][dim][16], slots = tokens/8 + nseq + 1."""
    import torch
    batch, seqlen, dim, nseq = _seq_shape(x, cu_seqlens)
    n = ctypes.c_size_t()
    st = load_library().samba_scan_ckpt_bytes(batch, seqlen, nseq, dim, ctypes.byref(n))
    if st != 0:
        raise SambaError(st, "samba_scan_ckpt_bytes")
    return torch.empty(n.value // (DSTATE * 4 * dim), dim, DSTATE, dtype=torch.float32, device=x.device)


def fwd_args(x, dt, z, B, C, A, D, dt_bias, *, y, h0=None, h_last=None, cu_seqlens=None,
             time_slices: int = 0, h_ckpt=None, lanes_per_channel: int = 0) -> FwdArgs:
    """Fill a samba_scan_fwd_args from tensors (shapes as in scan_fwd)."""
    if x.dim() == 3:
        batch, seqlen, dim = x.shape
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens needs packed [tokens][dim] inputs")
        nseq = 0
    elif x.dim() == 2:
        seqlen, dim = x.shape
        batch = 1
        nseq = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    else:
        raise ValueError("x must be [batch][seqlen][dim] or [tokens][dim]")
    a = FwdArgs()
    a.struct_size = ctypes.sizeof(FwdArgs)
    a.batch, a.seqlen, a.dim, a.dstate = batch, seqlen, dim, A.shape[-1]
    a.cu_seqlens = _ptr(cu_seqlens)
    a.nseq = nseq
    a.in_dtype = _dtype_code(x)
    a.y_dtype = _dtype_code(y)
    a.time_slices = int(time_slices)
    a.x, a.dt, a.z, a.B, a.C = _ptr(x), _ptr(dt), _ptr(z), _ptr(B), _ptr(C)
    a.A, a.D, a.dt_bias = _ptr(A), _ptr(D), _ptr(dt_bias)
    a.h0, a.h_last, a.y = _ptr(h0), _ptr(h_last), _ptr(y)
    a.h_ckpt = _ptr(h_ckpt)
    a.lanes_per_channel = int(lanes_per_channel)
    return a


def scan_fwd(x, dt, z, B, C, A, D, dt_bias, *, h0=None, h_last=None, y=None, return_last_state: bool = True,
             cu_seqlens=None, y_dtype=None, time_slices: int = 0, h_ckpt=None, lanes_per_channel: int = 0,
             stream=None):
    """Selective-scan prefill through samba_scan_fwd.

    x, dt, z : [batch][seqlen][dim]  (or [tokens][dim] with cu_seqlens)   bf16 or fp32
    B, C     : [batch][seqlen][16]   (or [tokens][16])                     same dtype as x
    A        : [dim][16] fp32;  D, dt_bias : [dim] fp32
    h0       : [nseq][dim][16] fp32 or None (zeros)
    cu_seqlens: int32 [nseq+1] device tensor of packed sequence offsets, or None
    h_ckpt   : optional output from alloc_ckpt(x, cu_seqlens): states every 8 tokens, for scan_bwd
    time_slices, lanes_per_channel: 0 = the library's launch plan; other values force it (see the header)
    Returns (y, h_last); h_last is None when neither given nor requested.
    """
    import torch
    _check_dev(x, dt, z, B, C, A, D, dt_bias, h0, h_last, y, cu_seqlens, h_ckpt)
    if y is None:
        y = torch.empty(x.shape, dtype=y_dtype or x.dtype, device=x.device)
    if h_last is None and return_last_state:
        nseq = x.shape[0] if cu_seqlens is None and x.dim() == 3 else (
            cu_seqlens.numel() - 1 if cu_seqlens is not None else 1)
        h_last = torch.empty((nseq, x.shape[-1], DSTATE), dtype=torch.float32, device=x.device)
    a = fwd_args(x, dt, z, B, C, A, D, dt_bias, y=y, h0=h0, h_last=h_last, cu_seqlens=cu_seqlens,
                 time_slices=time_slices, h_ckpt=h_ckpt, lanes_per_channel=lanes_per_channel)
    st = load_library().samba_scan_fwd(ctypes.byref(a), _P(_stream_handle(stream)))
    if st != 0:
        raise SambaError(st, "samba_scan_fwd")
    return y, h_last


def fwd_plan(x, dt, z, B, C, A, D, dt_bias, *, y, h0=None, h_last=None, cu_seqlens=None, time_slices: int = 0,
             lanes_per_channel: int = 0, h_ckpt=None):
    """(time_slices, workgroups, threads_per_workgroup, lanes_per_channel) the library would launch."""
    a = fwd_args(x, dt, z, B, C, A, D, dt_bias, y=y, h0=h0, h_last=h_last, cu_seqlens=cu_seqlens,
                 time_slices=time_slices, lanes_per_channel=lanes_per_channel, h_ckpt=h_ckpt)
    w, g, t, q = _I32(), _I32(), _I32(), _I32()
    st = load_library().samba_scan_fwd_plan(ctypes.byref(a), ctypes.byref(w), ctypes.byref(g), ctypes.byref(t),
                                            ctypes.byref(q))
    if st != 0:
        raise SambaError(st, "samba_scan_fwd_plan")
    return w.value, g.value, t.value, q.value


def step_args(state, x, dt, z, B, C, A, D, dt_bias, *, y) -> StepArgs:
    batch, dim = x.shape
    a = StepArgs()
    a.struct_size = ctypes.sizeof(StepArgs)
    a.batch, a.dim, a.dstate = batch, dim, A.shape[-1]
    a.in_dtype, a.y_dtype = _dtype_code(x), _dtype_code(y)
    a.state = _ptr(state)
    a.x, a.dt, a.z, a.B, a.C = _ptr(x), _ptr(dt), _ptr(z), _ptr(B), _ptr(C)
    a.A, a.D, a.dt_bias, a.y = _ptr(A), _ptr(D), _ptr(dt_bias), _ptr(y)
    return a


def scan_step(state, x, dt, z, B, C, A, D, dt_bias, *, y=None, y_dtype=None, stream=None):
    """One decode token through samba_scan_step; `state` [batch][dim][16] fp32 is updated in place.

    x, dt, z : [batch][dim];  B, C : [batch][16];  returns y [batch][dim].
    """
    import torch
    _check_dev(state, x, dt, z, B, C, A, D, dt_bias, y)
    if y is None:
        y = torch.empty(x.shape, dtype=y_dtype or x.dtype, device=x.device)
    a = step_args(state, x, dt, z, B, C, A, D, dt_bias, y=y)
    st = load_library().samba_scan_step(ctypes.byref(a), _P(_stream_handle(stream)))
    if st != 0:
        raise SambaError(st, "samba_scan_step")
    return y


def bwd_args(x, dt, z, B, C, A, D, dt_bias, dy, *, dx, ddt, dz, dB, dC, dA, dD, ddt_bias, h0=None, dh_last=None,
             dh0=None, cu_seqlens=None, workspace=None, time_slices: int = 0, h_ckpt=None) -> BwdArgs:
    """Fill a samba_scan_bwd_args from tensors (shapes as in scan_bwd)."""
    if x.dim() == 3:
        batch, seqlen, dim = x.shape
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens needs packed [tokens][dim] inputs")
        nseq = 0
    elif x.dim() == 2:
        seqlen, dim = x.shape
        batch = 1
        nseq = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    else:
        raise ValueError("x must be [batch][seqlen][dim] or [tokens][dim]")
    a = BwdArgs()
    a.struct_size = ctypes.sizeof(BwdArgs)
    a.batch, a.seqlen, a.dim, a.dstate = batch, seqlen, dim, A.shape[-1]
    a.cu_seqlens = _ptr(cu_seqlens)
    a.nseq = nseq
    a.in_dtype = _dtype_code(x)
    a.time_slices = int(time_slices)
    a.x, a.dt, a.z, a.B, a.C = _ptr(x), _ptr(dt), _ptr(z), _ptr(B), _ptr(C)
    a.A, a.D, a.dt_bias, a.h0 = _ptr(A), _ptr(D), _ptr(dt_bias), _ptr(h0)
    a.dy, a.dh_last, a.h_ckpt = _ptr(dy), _ptr(dh_last), _ptr(h_ckpt)
    a.dx, a.ddt, a.dz, a.dB, a.dC = _ptr(dx), _ptr(ddt), _ptr(dz), _ptr(dB), _ptr(dC)
    a.dA, a.dD, a.ddt_bias, a.dh0 = _ptr(dA), _ptr(dD), _ptr(ddt_bias), _ptr(dh0)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return a


def bwd_workspace_bytes(a: BwdArgs) -> int:
    n = ctypes.c_size_t()
    st = load_library().samba_scan_bwd_workspace_size(ctypes.byref(a), ctypes.byref(n))
    if st != 0:
        raise SambaError(st, "samba_scan_bwd_workspace_size")
    return n.value


def scan_bwd(x, dt, z, B, C, A, D, dt_bias, dy, *, h0=None, dh_last=None, cu_seqlens=None, workspace=None,
             want_dh0: bool = True, time_slices: int = 0, h_ckpt=None, stream=None):
    """Gradients of scan_fwd through samba_scan_bwd.

    Inputs as for scan_fwd, plus dy (shaped like y, same dtype as x) and dh_last ([nseq][dim][16] fp32 or None).
    `workspace` is a device tensor (any dtype) of at least the size the library asks for, or None (allocated
    here).  h_ckpt: the checkpoints a scan_fwd of the same inputs wrote (skips their recomputation), or None.
    Returns a dict: dx, ddt, dz (like x), dB, dC (like B, fp32), dA [dim][16], dD, ddt_bias [dim] and
    dh0 [nseq][dim][16] (fp32; None unless want_dh0).
    """
    import torch
    _check_dev(x, dt, z, B, C, A, D, dt_bias, dy, h0, dh_last, cu_seqlens, workspace, h_ckpt)
    dev = x.device
    dim = x.shape[-1]
    nseq = x.shape[0] if cu_seqlens is None and x.dim() == 3 else (
        cu_seqlens.numel() - 1 if cu_seqlens is not None else 1)
    out = {k: torch.empty_like(x) for k in ("dx", "ddt", "dz")}
    out["dB"] = torch.empty(B.shape, dtype=torch.float32, device=dev)
    out["dC"] = torch.empty(C.shape, dtype=torch.float32, device=dev)
    out["dA"] = torch.empty((dim, DSTATE), dtype=torch.float32, device=dev)
    out["dD"] = torch.empty(dim, dtype=torch.float32, device=dev)
    out["ddt_bias"] = torch.empty(dim, dtype=torch.float32, device=dev)
    out["dh0"] = torch.empty((nseq, dim, DSTATE), dtype=torch.float32, device=dev) if want_dh0 else None
    a = bwd_args(x, dt, z, B, C, A, D, dt_bias, dy, h0=h0, dh_last=dh_last, cu_seqlens=cu_seqlens,
                 workspace=workspace, time_slices=time_slices, h_ckpt=h_ckpt, **out)
    if workspace is None:
        workspace = torch.empty(max(bwd_workspace_bytes(a), 1), dtype=torch.uint8, device=dev)
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    st = load_library().samba_scan_bwd(ctypes.byref(a), _P(_stream_handle(stream)))
    if st != 0:
        raise SambaError(st, "samba_scan_bwd")
    return out


def proj_args(x, W, *, dt, B, C) -> ProjArgs:
    """Fill a samba_proj_args: x [tokens][dim] bf16, W [dim + 2*dstate][dim] bf16; outputs as in proj."""
    a = ProjArgs()
    a.struct_size = ctypes.sizeof(ProjArgs)
    a.tokens, a.dim = x.shape[0], x.shape[1]
    a.dstate = (W.shape[0] - x.shape[1]) // 2
    a.in_dtype = _dtype_code(x)
    a.out_dtype = _dtype_code(dt)
    a.x, a.W, a.dt, a.B, a.C = _ptr(x), _ptr(W), _ptr(dt), _ptr(B), _ptr(C)
    return a


def proj(x, W, *, out_dtype=None, dt=None, B=None, C=None, stream=None):
    """Selection projections through samba_proj: x [tokens][dim] bf16 and W [dim + 2*dstate][dim] bf16 ->
    (dt_raw [tokens][dim], B [tokens][dstate], C [tokens][dstate]) in out_dtype (default bf16)."""
    import torch
    _check_dev(x, W, dt, B, C)
    T, dim = x.shape
    N = (W.shape[0] - dim) // 2
    od = out_dtype or torch.bfloat16
    dt = torch.empty(T, dim, dtype=od, device=x.device) if dt is None else dt
    B = torch.empty(T, N, dtype=od, device=x.device) if B is None else B
    C = torch.empty(T, N, dtype=od, device=x.device) if C is None else C
    a = proj_args(x, W, dt=dt, B=B, C=C)
    st = load_library().samba_proj(ctypes.byref(a), _P(_stream_handle(stream)))
    if st != 0:
        raise SambaError(st, "samba_proj")
    return dt, B, C


def groups_args(x, dt, z, B, C, A, D, dt_bias, *, y, h0=None, h_last=None, cu_seqlens=None) -> GroupsArgs:
    """Fill a samba_scan_groups_args: B, C [batch][L][G][N] (or [tokens][G][N] packed)."""
    batch, seqlen, dim, nseq = _seq_shape(x, cu_seqlens)
    a = GroupsArgs()
    a.struct_size = ctypes.sizeof(GroupsArgs)
    a.batch, a.seqlen, a.dim = batch, seqlen, dim
    a.ngroups, a.dstate = B.shape[-2], B.shape[-1]
    a.cu_seqlens, a.nseq = _ptr(cu_seqlens), (nseq if cu_seqlens is not None else 0)
    a.in_dtype, a.y_dtype = _dtype_code(x), _dtype_code(y)
    a.x, a.dt, a.z, a.B, a.C = _ptr(x), _ptr(dt), _ptr(z), _ptr(B), _ptr(C)
    a.A, a.D, a.dt_bias = _ptr(A), _ptr(D), _ptr(dt_bias)
    a.h0, a.h_last, a.y = _ptr(h0), _ptr(h_last), _ptr(y)
    return a


def scan_fwd_groups(x, dt, z, B, C, A, D, dt_bias, *, h0=None, h_last=None, y=None, y_dtype=None, cu_seqlens=None,
                    return_last_state: bool = True, stream=None):
    """Grouped prefill through samba_scan_fwd_groups: B, C [batch][L][G][N] (or [tokens][G][N]); channel d
    reads group d // (dim // G); N in 16, 32, 64, 128, 256.  Returns (y, h_last)."""
    import torch
    _check_dev(x, dt, z, B, C, A, D, dt_bias, h0, h_last, y, cu_seqlens)
    batch, seqlen, dim, nseq = _seq_shape(x, cu_seqlens)
    N = B.shape[-1]
    if y is None:
        y = torch.empty(x.shape, dtype=y_dtype or x.dtype, device=x.device)
    if h_last is None and return_last_state:
        h_last = torch.empty(nseq, dim, N, dtype=torch.float32, device=x.device)
    a = groups_args(x, dt, z, B, C, A, D, dt_bias, y=y, h0=h0, h_last=h_last, cu_seqlens=cu_seqlens)
    st = load_library().samba_scan_fwd_groups(ctypes.byref(a), _P(_stream_handle(stream)))
    if st != 0:
        raise SambaError(st, "samba_scan_fwd_groups")
    return y, h_last


def step_groups_args(state, x, dt, z, B, C, A, D, dt_bias, *, y) -> StepGroupsArgs:
    a = StepGroupsArgs()
    a.struct_size = ctypes.sizeof(StepGroupsArgs)
    a.batch, a.dim = x.shape
    a.ngroups, a.dstate = B.shape[-2], B.shape[-1]
    a.in_dtype, a.y_dtype = _dtype_code(x), _dtype_code(y)
    a.state, a.x, a.dt, a.z, a.B, a.C = _ptr(state), _ptr(x), _ptr(dt), _ptr(z), _ptr(B), _ptr(C)
    a.A, a.D, a.dt_bias, a.y = _ptr(A), _ptr(D), _ptr(dt_bias), _ptr(y)
    return a


def scan_step_groups(state, x, dt, z, B, C, A, D, dt_bias, *, y=None, y_dtype=None, stream=None):
    """Grouped decode step through samba_scan_step_groups: x, dt, z [batch][dim]; B, C [batch][G][N]; state
    [batch][dim][N] fp32 updated in place.  Returns y [batch][dim]."""
    import torch
    _check_dev(state, x, dt, z, B, C, A, D, dt_bias, y)
    y = torch.empty(x.shape, dtype=y_dtype or x.dtype, device=x.device) if y is None else y
    a = step_groups_args(state, x, dt, z, B, C, A, D, dt_bias, y=y)
    st = load_library().samba_scan_step_groups(ctypes.byref(a), _P(_stream_handle(stream)))
    if st != 0:
        raise SambaError(st, "samba_scan_step_groups")
    return y
