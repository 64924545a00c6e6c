"""Python front of the fp64 oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the CPU
baseline leg of the benchmark; never by the library.  It converts arrays to
float64, calls the C loop through ctypes and returns float64 results.  It
imports nothing from the GPU package.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SRC = HERE / "oracle.c"
LIB = HERE / "liboracle.so"
CFLAGS = ["-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c99"]

_lib = None


def build(force: bool = True, src: Path = SRC, out: Path = LIB) -> Path:
    """Compile oracle.c with gcc (no fast-math, no FP contraction)."""
    if not force and out.exists() and out.stat().st_mtime >= src.stat().st_mtime:
        return out
    tmp = out.with_suffix(".so.tmp%d" % os.getpid())
    subprocess.check_call(["gcc", *CFLAGS, "-o", str(tmp), str(src), "-lm"])
    os.replace(tmp, out)
    return out


def load(path: Path | None = None):
    """Load (building first if absent) the oracle shared library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(str(path)))
    if _lib is None:
        if not LIB.exists() or LIB.stat().st_mtime < SRC.stat().st_mtime:
            build()
        _lib = _bind(ctypes.CDLL(str(LIB)))
    return _lib


def _bind(lib):
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_scan_fwd.argtypes = [I64, P, I64, I64, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_int]
    lib.oracle_scan_fwd.restype = ctypes.c_int
    lib.oracle_scan_step.argtypes = [I64, I64, I64, P, P, P, P, P, P, P, P, P, P, ctypes.c_int]
    lib.oracle_scan_step.restype = ctypes.c_int
    lib.oracle_scan_bwd.argtypes = [I64, P, I64, I64] + [P] * 20 + [ctypes.c_int]
    lib.oracle_scan_bwd.restype = ctypes.c_int
    lib.oracle_proj.argtypes = [I64, I64, I64, P, P, P, P, P, ctypes.c_int]
    lib.oracle_proj.restype = ctypes.c_int
    lib.oracle_swa.argtypes = [I64, P, I64, I64, I64, P, P, P, P, P, P, ctypes.c_int]
    lib.oracle_swa.restype = ctypes.c_int
    lib.oracle_swa_rows.argtypes = [I64, P, I64, I64, I64, P, P, P, P, P, P, I64, P, ctypes.c_int]
    lib.oracle_swa_rows.restype = ctypes.c_int
    lib.oracle_rope.argtypes = [I64, I64, I64, P, P, P, P, P]
    lib.oracle_rope.restype = ctypes.c_int
    lib.oracle_scan_fwd_groups.argtypes = [I64, P, I64, I64, I64] + [P] * 11 + [ctypes.c_int]
    lib.oracle_scan_fwd_groups.restype = ctypes.c_int
    lib.oracle_ssd.argtypes = [I64, P, I64, I64, I64, I64] + [P] * 11 + [ctypes.c_int]
    lib.oracle_ssd.restype = ctypes.c_int
    lib.oracle_gla.argtypes = [I64, P, I64, I64, I64] + [P] * 7 + [ctypes.c_int]
    lib.oracle_gla.restype = ctypes.c_int
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def scan_fwd(x, dt, z, B, C, A, D, dt_bias, h0=None, seq_start=None, nthreads: int = 0, lib=None):
    """Selective scan prefill in fp64.

    x, dt, z : [T][dim] (or [batch][L][dim] with seq_start None: equal-length rows)
    B, C     : [T][dstate] (or [batch][L][dstate])
    A        : [dim][dstate];  D, dt_bias : [dim]
    h0       : [nseq][dim][dstate] or None
    seq_start: [nseq+1] token offsets of a packed stream, or None
    Returns (y [same leading shape as x], h_last [nseq][dim][dstate]).
    """
    lib = lib or load()
    x = _f64(x)
    shape = x.shape
    if x.ndim == 3:
        batch, L, dim = shape
        if seq_start is None:
            seq_start = np.arange(batch + 1, dtype=np.int64) * L
        x = x.reshape(batch * L, dim)
        dt, z = _f64(dt).reshape(batch * L, dim), _f64(z).reshape(batch * L, dim)
        B, C = _f64(B).reshape(batch * L, -1), _f64(C).reshape(batch * L, -1)
    else:
        dim = shape[1]
        if seq_start is None:
            seq_start = np.array([0, shape[0]], dtype=np.int64)
        dt, z, B, C = _f64(dt), _f64(z), _f64(B), _f64(C)
    A, D, dt_bias = _f64(A), _f64(D), _f64(dt_bias)
    dstate = A.shape[1]
    T = x.shape[0]
    seq_start = np.ascontiguousarray(np.asarray(seq_start, dtype=np.int64))
    nseq = len(seq_start) - 1
    assert seq_start[0] == 0 and seq_start[-1] == T
    assert dt.shape == z.shape == (T, dim) and B.shape == C.shape == (T, dstate) and A.shape == (dim, dstate)
    h0 = None if h0 is None else _f64(h0).reshape(nseq, dim, dstate)
    y = np.empty((T, dim), dtype=np.float64)
    h_last = np.empty((nseq, dim, dstate), dtype=np.float64)
    rc = lib.oracle_scan_fwd(nseq, _ptr(seq_start), dim, dstate, _ptr(x), _ptr(dt), _ptr(z), _ptr(B), _ptr(C),
                             _ptr(A), _ptr(D), _ptr(dt_bias), _ptr(h0), _ptr(y), _ptr(h_last), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_scan_fwd failed (%d)" % rc)
    return y.reshape(shape), h_last


def scan_fwd_groups(x, dt, z, B, C, A, D, dt_bias, h0=None, seq_start=None, nthreads: int = 0, lib=None):
    """Prefill with G groups of (B, C) per token: B, C [T][G][N] (or [batch][L][G][N]); channel d reads
    group d // (dim // G).  Otherwise as scan_fwd."""
    lib = lib or load()
    x = _f64(x)
    shape = x.shape
    if x.ndim == 3:
        batch, L, dim = shape
        if seq_start is None:
            seq_start = np.arange(batch + 1, dtype=np.int64) * L
        x = x.reshape(batch * L, dim)
        dt, z = _f64(dt).reshape(batch * L, dim), _f64(z).reshape(batch * L, dim)
        B, C = _f64(B).reshape(batch * L, *np.shape(B)[2:]), _f64(C).reshape(batch * L, *np.shape(C)[2:])
    else:
        dim = shape[1]
        if seq_start is None:
            seq_start = np.array([0, shape[0]], dtype=np.int64)
        dt, z, B, C = _f64(dt), _f64(z), _f64(B), _f64(C)
    A, D, dt_bias = _f64(A), _f64(D), _f64(dt_bias)
    T = x.shape[0]
    G, dstate = B.shape[1], B.shape[2]
    seq_start = np.ascontiguousarray(np.asarray(seq_start, dtype=np.int64))
    nseq = len(seq_start) - 1
    assert seq_start[0] == 0 and seq_start[-1] == T
    assert B.shape == C.shape == (T, G, dstate) and A.shape == (dim, dstate)
    h0 = None if h0 is None else _f64(h0).reshape(nseq, dim, dstate)
    y = np.empty((T, dim), dtype=np.float64)
    h_last = np.empty((nseq, dim, dstate), dtype=np.float64)
    rc = lib.oracle_scan_fwd_groups(nseq, _ptr(seq_start), dim, dstate, G, _ptr(x), _ptr(dt), _ptr(z), _ptr(B),
                                    _ptr(C), _ptr(A), _ptr(D), _ptr(dt_bias), _ptr(h0), _ptr(y), _ptr(h_last),
                                    int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_scan_fwd_groups failed (%d)" % rc)
    return y.reshape(shape), h_last


def scan_bwd(x, dt, z, B, C, A, D, dt_bias, dy, h0=None, dh_last=None, seq_start=None, nthreads: int = 0,
             lib=None):
    """Gradients of scan_fwd's outputs (y, h_last) in fp64, for upstream gradients dy (shaped like y) and
    dh_last ([nseq][dim][dstate] or None = zeros).

    Returns a dict: dx, ddt, dz (shaped like x), dB, dC (shaped like B), dA [dim][dstate], dD, ddt_bias [dim],
    dh0 [nseq][dim][dstate] (the gradient of h0, whether h0 was given or zero).
    """
    lib = lib or load()
    x = _f64(x)
    shape, bshape = x.shape, np.shape(B)
    if x.ndim == 3:
        batch, L, dim = shape
        if seq_start is None:
            seq_start = np.arange(batch + 1, dtype=np.int64) * L
        x = x.reshape(batch * L, dim)
        dt, z, dy = (_f64(a).reshape(batch * L, dim) for a in (dt, z, dy))
        B, C = _f64(B).reshape(batch * L, -1), _f64(C).reshape(batch * L, -1)
    else:
        dim = shape[1]
        if seq_start is None:
            seq_start = np.array([0, shape[0]], dtype=np.int64)
        dt, z, dy, B, C = _f64(dt), _f64(z), _f64(dy), _f64(B), _f64(C)
    A, D, dt_bias = _f64(A), _f64(D), _f64(dt_bias)
    dstate = A.shape[1]
    T = x.shape[0]
    seq_start = np.ascontiguousarray(np.asarray(seq_start, dtype=np.int64))
    nseq = len(seq_start) - 1
    assert seq_start[0] == 0 and seq_start[-1] == T
    assert dt.shape == z.shape == dy.shape == (T, dim) and B.shape == C.shape == (T, dstate)
    h0 = None if h0 is None else _f64(h0).reshape(nseq, dim, dstate)
    dh_last = None if dh_last is None else _f64(dh_last).reshape(nseq, dim, dstate)
    out = {k: np.empty((T, dim)) for k in ("dx", "ddt", "dz")}
    out.update({k: np.empty((T, dstate)) for k in ("dB", "dC")})
    out["dA"] = np.empty((dim, dstate))
    out["dD"], out["ddt_bias"] = np.empty(dim), np.empty(dim)
    out["dh0"] = np.empty((nseq, dim, dstate))
    rc = lib.oracle_scan_bwd(nseq, _ptr(seq_start), dim, dstate, _ptr(x), _ptr(dt), _ptr(z), _ptr(B), _ptr(C),
                             _ptr(A), _ptr(D), _ptr(dt_bias), _ptr(h0), _ptr(dy), _ptr(dh_last),
                             *(_ptr(out[k]) for k in ("dx", "ddt", "dz", "dB", "dC", "dA", "dD", "ddt_bias", "dh0")),
                             int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_scan_bwd failed (%d)" % rc)
    for k in ("dx", "ddt", "dz"):
        out[k] = out[k].reshape(shape)
    for k in ("dB", "dC"):
        out[k] = out[k].reshape(bshape)
    return out


def proj(x, W, dstate: int = 16, nthreads: int = 0, lib=None):
    """Selection projections in fp64: x [T][dim], W [dim + 2*dstate][dim] -> (dt_raw [T][dim], B, C [T][dstate])."""
    lib = lib or load()
    x, W = _f64(x), _f64(W)
    T, dim = x.shape
    assert W.shape == (dim + 2 * dstate, dim)
    dt = np.empty((T, dim))
    B, C = np.empty((T, dstate)), np.empty((T, dstate))
    rc = lib.oracle_proj(T, dim, dstate, _ptr(x), _ptr(W), _ptr(dt), _ptr(B), _ptr(C), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_proj failed (%d)" % rc)
    return dt, B, C


def swa(q, k, v, window: int, rope_cos=None, rope_sin=None, seq_start=None, rows=None, nthreads: int = 0,
        lib=None):
    """Causal sliding-window attention in fp64.  q, k, v: [T][H][hd] (or [batch][L][H][hd]); rope tables
    [positions][hd/2] or None.  Query i sees keys i-window .. i of its own sequence.  Returns o like q;
    with `rows` (packed row indices) only those rows are computed and the others are NaN."""
    lib = lib or load()
    q = _f64(q)
    shape = q.shape
    if q.ndim == 4:
        b, L, H, hd = shape
        if seq_start is None:
            seq_start = np.arange(b + 1, dtype=np.int64) * L
        q = q.reshape(b * L, H, hd)
        k, v = _f64(k).reshape(b * L, H, hd), _f64(v).reshape(b * L, H, hd)
    else:
        H, hd = shape[1], shape[2]
        if seq_start is None:
            seq_start = np.array([0, shape[0]], dtype=np.int64)
        k, v = _f64(k), _f64(v)
    T = q.shape[0]
    seq_start = np.ascontiguousarray(np.asarray(seq_start, dtype=np.int64))
    assert seq_start[0] == 0 and seq_start[-1] == T and k.shape == v.shape == q.shape
    cs = None if rope_cos is None else _f64(rope_cos)
    sn = None if rope_sin is None else _f64(rope_sin)
    if rows is None:
        o = np.empty_like(q)
        rc = lib.oracle_swa(len(seq_start) - 1, _ptr(seq_start), H, hd, int(window), _ptr(q), _ptr(k), _ptr(v),
                            _ptr(cs), _ptr(sn), _ptr(o), int(nthreads))
    else:
        o = np.full_like(q, np.nan)
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        rc = lib.oracle_swa_rows(len(seq_start) - 1, _ptr(seq_start), H, hd, int(window), _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(cs), _ptr(sn), _ptr(r), len(r), _ptr(o), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_swa failed (%d)" % rc)
    return o.reshape(shape)


def rope(x, rope_cos, rope_sin, positions, lib=None):
    """RoPE alone in fp64: x [T][H][hd], row t rotated by table row positions[t]."""
    lib = lib or load()
    x = _f64(x)
    T, H, hd = x.shape
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int64))
    assert pos.shape == (T,)
    cs, sn = _f64(rope_cos), _f64(rope_sin)
    assert pos.size == 0 or (pos.max() < cs.shape[0])
    out = np.empty_like(x)
    rc = lib.oracle_rope(T, H, hd, _ptr(x), _ptr(pos), _ptr(cs), _ptr(sn), _ptr(out))
    if rc != 0:
        raise RuntimeError("oracle_rope failed (%d)" % rc)
    return out


def ssd(x, dt, B, C, A, D, dt_bias, z=None, h0=None, seq_start=None, nthreads: int = 0, lib=None):
    """State-space duality layer in fp64 (its recurrence).  x [T][H][P] (or [batch][L][H][P]), dt [T][H],
    B, C [T][G][N], A, D, dt_bias [H], z like x or None, h0 [nseq][H][P][N] or None.
    Returns (y like x, h_last [nseq][H][P][N])."""
    lib = lib or load()
    x = _f64(x)
    shape = x.shape
    if x.ndim == 4:
        b, L, H, P = shape
        if seq_start is None:
            seq_start = np.arange(b + 1, dtype=np.int64) * L
        x = x.reshape(b * L, H, P)
        dt = _f64(dt).reshape(b * L, H)
        B, C = _f64(B).reshape(b * L, *np.shape(B)[2:]), _f64(C).reshape(b * L, *np.shape(C)[2:])
        z = None if z is None else _f64(z).reshape(b * L, H, P)
    else:
        H, P = shape[1], shape[2]
        if seq_start is None:
            seq_start = np.array([0, shape[0]], dtype=np.int64)
        dt, B, C = _f64(dt), _f64(B), _f64(C)
        z = None if z is None else _f64(z)
    T = x.shape[0]
    G, N = B.shape[1], B.shape[2]
    A, D, dt_bias = _f64(A), _f64(D), _f64(dt_bias)
    seq_start = np.ascontiguousarray(np.asarray(seq_start, dtype=np.int64))
    nseq = len(seq_start) - 1
    assert seq_start[0] == 0 and seq_start[-1] == T and dt.shape == (T, H) and C.shape == B.shape == (T, G, N)
    h0 = None if h0 is None else _f64(h0).reshape(nseq, H, P, N)
    y = np.empty((T, H, P))
    h_last = np.empty((nseq, H, P, N))
    rc = lib.oracle_ssd(nseq, _ptr(seq_start), H, P, N, G, _ptr(x), _ptr(dt), _ptr(z), _ptr(B), _ptr(C), _ptr(A),
                        _ptr(D), _ptr(dt_bias), _ptr(h0), _ptr(y), _ptr(h_last), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_ssd failed (%d)" % rc)
    return y.reshape(shape), h_last


def gla(q, k, v, gk, h0=None, seq_start=None, nthreads: int = 0, lib=None):
    """Gated linear attention in fp64 (its recurrence).  q, k, gk [T][H][N] (or [batch][L][H][N]), v [T][H][P],
    h0 [nseq][H][P][N] or None.  Returns (o like v, h_last [nseq][H][P][N])."""
    lib = lib or load()
    v = _f64(v)
    shape = v.shape
    if v.ndim == 4:
        b, L, H, P = shape
        if seq_start is None:
            seq_start = np.arange(b + 1, dtype=np.int64) * L
        v = v.reshape(b * L, H, P)
        q, k, gk = (_f64(a).reshape(b * L, H, -1) for a in (q, k, gk))
    else:
        H, P = shape[1], shape[2]
        if seq_start is None:
            seq_start = np.array([0, shape[0]], dtype=np.int64)
        q, k, gk = _f64(q), _f64(k), _f64(gk)
    T, N = v.shape[0], q.shape[2]
    assert q.shape == k.shape == gk.shape == (T, H, N)
    seq_start = np.ascontiguousarray(np.asarray(seq_start, dtype=np.int64))
    nseq = len(seq_start) - 1
    assert seq_start[0] == 0 and seq_start[-1] == T
    h0 = None if h0 is None else _f64(h0).reshape(nseq, H, P, N)
    o = np.empty((T, H, P))
    h_last = np.empty((nseq, H, P, N))
    rc = lib.oracle_gla(nseq, _ptr(seq_start), H, P, N, _ptr(q), _ptr(k), _ptr(v), _ptr(gk), _ptr(h0), _ptr(o),
                        _ptr(h_last), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_gla failed (%d)" % rc)
    return o.reshape(shape), h_last


def scan_step(state, x, dt, z, B, C, A, D, dt_bias, nthreads: int = 0, lib=None):
    """One decode token in fp64; returns (y [batch][dim], new_state [batch][dim][dstate])."""
    lib = lib or load()
    st = _f64(state).copy()
    x, dt, z, B, C = _f64(x), _f64(dt), _f64(z), _f64(B), _f64(C)
    A, D, dt_bias = _f64(A), _f64(D), _f64(dt_bias)
    batch, dim = x.shape
    dstate = A.shape[1]
    assert st.shape == (batch, dim, dstate) and B.shape == C.shape == (batch, dstate)
    y = np.empty((batch, dim), dtype=np.float64)
    rc = lib.oracle_scan_step(batch, dim, dstate, _ptr(st), _ptr(x), _ptr(dt), _ptr(z), _ptr(B), _ptr(C),
                              _ptr(A), _ptr(D), _ptr(dt_bias), _ptr(y), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_scan_step failed (%d)" % rc)
    return y, st


def max_threads(lib=None) -> int:
    return int((lib or load()).oracle_max_threads())
