"""Seeded synthetic inputs for the selective scan.

This module only draws random numbers and packs them; it holds none of the
scan's arithmetic, so both the GPU tests/bench and the fp64 oracle can take
their inputs from it without sharing any compute code.

Recipe (every config; sizes differ):
  * grouped prefill: B, C ~ N(0, 1) per (token, group, state); the other
    tensors as above with A [dim][dstate]
  * attention: q, k, v ~ N(0, 1) per (token, head, feature), rounded to bf16;
    RoPE tables cos/sin of p * 10000^(-2c / head_dim) (the layer's fixed
    parameter, computed in float64 and handed to both sides: fp64 to the
    oracle, rounded to fp32 for the library); decode positions drawn
    uniformly from a range the test names
  * x, z, dt_raw ~ N(0, 1) per (token, channel)
  * dt_bias[d] = log(expm1(U(1e-3, 1e-1)))  -> softplus(dt_bias) lies in [1e-3, 1e-1]
  * A[d, n] = -exp(U(0, ln 16))             -> A in [-16, -1], diagonal, negative real
  * B, C ~ N(0, 1) per (token, state)
  * D[d] ~ U(0, 1)
  * h0 = 0 unless a test asks for a random carry-in
  * selection projections: W [dim + 2N][dim] ~ N(0, 1/dim) (a linear layer's
    scale, so dt_raw, B and C come out ~N(0, 1) like the scan's own inputs)
  * backward: upstream gradients dy ~ N(0, 1) per (token, channel) (in the
    input dtype) and, where a test asks for one, dh_last ~ N(0, 1) per
    (sequence, channel, state)
bf16 tensors are produced from fp32 draws by integer round-to-nearest-even, so
the exact values the kernels read are known bit for bit on the host.

Two back ends draw from the same recipe: NumPy (PCG64 seeded from
SeedSequence([20240611, config, tensor_id])) for host-sized cases that the
oracle checks whole, and torch generators on the device for the full-size
workloads (their values differ from NumPy's but are equally seeded; full-size
checks copy the sampled slices of the very same device tensors to the host).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

SEED_ROOT = 20240611
TENSOR_IDS = {"x": 0, "z": 1, "dt": 2, "dt_init": 3, "A": 4, "B": 5, "C": 6, "D": 7,
              "lengths": 8, "h0": 9, "dy": 10, "dh_last": 11, "W_sel": 12, "q": 13, "k": 14, "v": 15,
              "pos": 16, "gk": 17}
ROPE_BASE = 10000.0
DECODE_RING_BASE = 100
DSTATE = 16


# --------------------------------------------------------------------------- #
# bf16 helpers (bit manipulation only)
# --------------------------------------------------------------------------- #
def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 -> bf16 to nearest even; returns the uint16 bit patterns."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = bits + np.uint32(0x7FFF) + lsb
    return (rounded >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(cfg_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, cfg_id, tensor_id])))


def torch_seed(cfg_id: int, tensor_id: int) -> int:
    """63-bit seed for a torch generator, derived from the same seed tree."""
    s = np.random.SeedSequence([SEED_ROOT, cfg_id, tensor_id]).generate_state(1, np.uint64)[0]
    return int(s) & ((1 << 63) - 1)


# --------------------------------------------------------------------------- #
# Workload descriptions
# --------------------------------------------------------------------------- #
@dataclass(frozen=True)
class Workload:
    """One synthetic workload (sizes of the five standard configurations)."""
    cfg_id: int
    name: str
    batch: int
    seqlen: int
    dim: int
    dstate: int = DSTATE
    in_dtype: str = "bf16"          # "bf16" or "f32" for x, dt, z, B, C
    varlen_total: int = 0           # >0: packed variable-length stream of this many tokens
    chunks: int = 1                 # >1: the prompt is fed as this many chained calls
    decode_steps: int = 0           # >0: streaming decode after a prefill of `seqlen`
    decode_ring: int = 0            # number of distinct per-step input sets
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    0: Workload(0, "scan_fwd B1 L256 D64 N16 fp32", 1, 256, 64, in_dtype="f32"),
    1: Workload(1, "scan_fwd B1 L4096 D2048 N16 bf16", 1, 4096, 2048),
    2: Workload(2, "scan_fwd varlen T32768 D4096 N16 bf16", 1, 32768, 4096, varlen_total=32768),
    3: Workload(3, "scan_fwd L131072 D4096 N16 bf16 as 8x16384 chained", 1, 131072, 4096, chunks=8),
    4: Workload(4, "scan_step B64 D4096 N16 after L2048 prefill, 65536 steps", 64, 2048, 4096,
                decode_steps=65536, decode_ring=256),
    # training shape: context 4096, batch 4 per device (page 1, 实现细节 -> 训练配置)
    5: Workload(5, "scan_bwd B4 L4096 D4096 N16 bf16", 4, 4096, 4096),
    # sliding-window attention of Samba-3.8B (hidden 3072 = 24 heads x 128, window 2048: page 1,
    # 实现细节 -> 模型配置) on the training shape, and its decode step over a full window
    6: Workload(6, "swa_fwd B4 L4096 H24 hd128 w2048 bf16", 4, 4096, 3072,
                extra={"heads": 24, "head_dim": 128, "window": 2048}),
    7: Workload(7, "swa_decode B64 H24 hd128 w2048 cache 2049 bf16", 64, 1, 3072,
                extra={"heads": 24, "head_dim": 128, "window": 2048, "cache_len": 2049, "pos": 4096}),
    # grouped selection with a larger state: the training shape with 4 (B, C) groups of 64 states
    8: Workload(8, "scan_fwd_groups B4 L4096 D4096 G4 N64 bf16", 4, 4096, 4096, dstate=64,
                extra={"ngroups": 4}),
    # the state-space duality form on the training shape: the inner width 4096 as 64 heads of 64, one
    # (B, C) group of 128 states
    9: Workload(9, "ssd_fwd B4 L4096 H64 P64 N128 G1 bf16", 4, 4096, 4096, dstate=128,
                extra={"heads": 64, "head_dim": 64, "ngroups": 1}),
    # gated linear attention at the GLA paper's 1.3B shape on the training shape: model width 2048, 4 heads,
    # key size 256 (half the width over 4 heads), value size 512
    10: Workload(10, "gla_fwd B4 L4096 H4 K256 V512 bf16", 4, 4096, 2048, dstate=256,
                 extra={"heads": 4, "head_dim": 512}),
    # multi-scale retention through the state-space duality entry point on the training shape: width 2048
    # as 32 heads of 64 values, 128 keys per head (one (k, q) group per head), Δ = 1, A = ln γ_h, no skip
    # and no gate (make_retention_params)
    11: Workload(11, "retention B4 L4096 H32 P64 N128 G32 bf16", 4, 4096, 2048, dstate=128,
                 extra={"heads": 32, "head_dim": 64, "ngroups": 32}),
}


def varlen_lengths(cfg_id: int, total: int, lo: int = 512, hi: int = 4096) -> np.ndarray:
    """Integer lengths in [lo, hi] summing exactly to `total`.

    Lengths are drawn U[lo, hi] while more than hi + lo tokens remain; the
    remainder r is appended whole if r <= hi, else split into floor(r/2) and
    ceil(r/2) (both >= hi/2 >= lo).
    """
    g = _rng(cfg_id, TENSOR_IDS["lengths"])
    out = []
    rem = total
    while rem > hi + lo:
        L = int(g.integers(lo, hi + 1))
        out.append(L)
        rem -= L
    if rem <= hi:
        out.append(rem)
    else:
        out.extend([rem // 2, rem - rem // 2])
    arr = np.asarray(out, dtype=np.int64)
    assert arr.sum() == total and arr.min() >= min(lo, total) and arr.max() <= hi
    return arr


def cu_from_lengths(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


# --------------------------------------------------------------------------- #
# Parameters (always small: drawn with NumPy, fp32)
# --------------------------------------------------------------------------- #
def make_params(cfg_id: int, dim: int, dstate: int = DSTATE) -> dict:
    """A [dim][dstate], D [dim], dt_bias [dim] as fp32 arrays."""
    u = _rng(cfg_id, TENSOR_IDS["dt_init"]).uniform(1e-3, 1e-1, size=dim)
    dt_bias = np.log(np.expm1(u)).astype(np.float32)
    A = (-np.exp(_rng(cfg_id, TENSOR_IDS["A"]).uniform(0.0, math.log(16.0), size=(dim, dstate)))).astype(np.float32)
    D = _rng(cfg_id, TENSOR_IDS["D"]).uniform(0.0, 1.0, size=dim).astype(np.float32)
    return {"A": A, "D": D, "dt_bias": dt_bias}


def make_h0(cfg_id: int, nseq: int, dim: int, dstate: int = DSTATE, scale: float = 1.0) -> np.ndarray:
    return (scale * _rng(cfg_id, TENSOR_IDS["h0"]).standard_normal((nseq, dim, dstate))).astype(np.float32)


# --------------------------------------------------------------------------- #
# NumPy back end (host-sized cases)
# --------------------------------------------------------------------------- #
def _normal(cfg_id: int, name: str, shape) -> np.ndarray:
    return _rng(cfg_id, TENSOR_IDS[name]).standard_normal(shape, dtype=np.float32)


def make_fwd_inputs_np(cfg_id: int, rows: int, dim: int, dstate: int = DSTATE,
                       in_dtype: str = "bf16") -> dict:
    """Token-major inputs for `rows` tokens (batch*seqlen, or a packed stream).

    Returns the device-side representation (uint16 bf16 bits or fp32) under
    x, dt, z, B, C and the exact fp32 values the kernels see under *_f32.
    """
    out = {}
    for name, shape in (("x", (rows, dim)), ("z", (rows, dim)), ("dt", (rows, dim)),
                        ("B", (rows, dstate)), ("C", (rows, dstate))):
        v = _normal(cfg_id, name, shape)
        if in_dtype == "bf16":
            bits = bf16_bits_from_f32(v)
            out[name] = bits
            out[name + "_f32"] = f32_from_bf16_bits(bits)
        elif in_dtype == "f32":
            out[name] = v
            out[name + "_f32"] = v
        else:
            raise ValueError(in_dtype)
    out.update(make_params(cfg_id, dim, dstate))
    return out


def make_step_inputs_np(cfg_id: int, ring_index: int, batch: int, dim: int, dstate: int = DSTATE,
                        in_dtype: str = "bf16") -> dict:
    """One decode step's inputs (x, dt, z [batch][dim]; B, C [batch][dstate])."""
    base = DECODE_RING_BASE + ring_index * 8
    out = {}
    for k, (name, shape) in enumerate((("x", (batch, dim)), ("z", (batch, dim)), ("dt", (batch, dim)),
                                       ("B", (batch, dstate)), ("C", (batch, dstate)))):
        v = _rng(cfg_id, base + k).standard_normal(shape, dtype=np.float32)
        if in_dtype == "bf16":
            bits = bf16_bits_from_f32(v)
            out[name], out[name + "_f32"] = bits, f32_from_bf16_bits(bits)
        else:
            out[name], out[name + "_f32"] = v, v
    return out


# --------------------------------------------------------------------------- #
# torch back end (full-size workloads, generated on the device)
# --------------------------------------------------------------------------- #
def _torch_normal(torch, shape, cfg_id: int, tensor_id: int, device, dtype):
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(cfg_id, tensor_id))
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return v.to(dtype)  # fp32 -> bf16 cast rounds to nearest even


def make_fwd_inputs_torch(cfg_id: int, rows: int, dim: int, device, dstate: int = DSTATE,
                          in_dtype: str = "bf16", tensor_offset: int = 0) -> dict:
    """Device tensors x, dt, z [rows][dim], B, C [rows][dstate] (+ fp32 params).

    `tensor_offset` shifts the seed ids so that chained chunks of one long
    prompt get distinct draws.
    """
    import torch
    dt_ = torch.bfloat16 if in_dtype == "bf16" else torch.float32
    out = {}
    for name, shape in (("x", (rows, dim)), ("z", (rows, dim)), ("dt", (rows, dim)),
                        ("B", (rows, dstate)), ("C", (rows, dstate))):
        out[name] = _torch_normal(torch, shape, cfg_id, TENSOR_IDS[name] + 1000 * tensor_offset, device, dt_)
    p = make_params(cfg_id, dim, dstate)
    for k, v in p.items():
        out[k] = torch.from_numpy(v).to(device)
    return out


def make_bwd_extra_np(cfg_id: int, rows: int, dim: int, nseq: int, dstate: int = DSTATE,
                      in_dtype: str = "bf16") -> dict:
    """Upstream gradients for the backward: dy [rows][dim] (input dtype, plus dy_f32) and dh_last
    [nseq][dim][dstate] fp32."""
    v = _normal(cfg_id, "dy", (rows, dim))
    out = {}
    if in_dtype == "bf16":
        out["dy"] = bf16_bits_from_f32(v)
        out["dy_f32"] = f32_from_bf16_bits(out["dy"])
    else:
        out["dy"], out["dy_f32"] = v, v
    out["dh_last"] = _normal(cfg_id, "dh_last", (nseq, dim, dstate))
    return out


def make_bwd_extra_torch(cfg_id: int, rows: int, dim: int, nseq: int, device, dstate: int = DSTATE,
                         in_dtype: str = "bf16") -> dict:
    """Device upstream gradients: dy [rows][dim] (input dtype), dh_last [nseq][dim][dstate] fp32."""
    import torch
    dt_ = torch.bfloat16 if in_dtype == "bf16" else torch.float32
    return {"dy": _torch_normal(torch, (rows, dim), cfg_id, TENSOR_IDS["dy"], device, dt_),
            "dh_last": _torch_normal(torch, (nseq, dim, dstate), cfg_id, TENSOR_IDS["dh_last"], device,
                                     torch.float32)}


def make_proj_weight_np(cfg_id: int, dim: int, dstate: int = DSTATE) -> dict:
    """Selection-projection weight W [dim + 2*dstate][dim] as bf16 bits (W) and their fp32 values (W_f32)."""
    v = (_normal(cfg_id, "W_sel", (dim + 2 * dstate, dim)) / np.float32(math.sqrt(dim))).astype(np.float32)
    bits = bf16_bits_from_f32(v)
    return {"W": bits, "W_f32": f32_from_bf16_bits(bits)}


def make_proj_weight_torch(cfg_id: int, dim: int, device, dstate: int = DSTATE):
    """Device bf16 W [dim + 2*dstate][dim] ~ N(0, 1/dim)."""
    import torch
    w = _torch_normal(torch, (dim + 2 * dstate, dim), cfg_id, TENSOR_IDS["W_sel"], device, torch.float32)
    return (w / math.sqrt(dim)).to(torch.bfloat16)


def make_step_ring_torch(cfg_id: int, ring: int, batch: int, dim: int, device, dstate: int = DSTATE) -> dict:
    """`ring` decode input sets stacked on a leading axis: x, dt, z [ring][batch][dim], B, C [ring][batch][dstate]."""
    import torch
    out = {}
    for k, (name, shape) in enumerate((("x", (ring, batch, dim)), ("z", (ring, batch, dim)),
                                       ("dt", (ring, batch, dim)), ("B", (ring, batch, dstate)),
                                       ("C", (ring, batch, dstate)))):
        out[name] = _torch_normal(torch, shape, cfg_id, DECODE_RING_BASE + k, device, torch.bfloat16)
    return out


# --------------------------------------------------------------------------- #
# sliding-window attention
# --------------------------------------------------------------------------- #
def rope_tables(npos: int, head_dim: int, base: float = ROPE_BASE):
    """(cos, sin) float64 [npos][head_dim / 2] of the angles p * base^(-2c / head_dim): the layer's RoPE
    parameter, an input to both the library and the oracle."""
    ang = np.arange(npos, dtype=np.float64)[:, None] * base ** (-2.0 * np.arange(head_dim // 2)[None, :] / head_dim)
    return np.cos(ang), np.sin(ang)


def make_swa_inputs_np(cfg_id: int, rows: int, heads: int, head_dim: int, q_scale: float = 1.0) -> dict:
    """q, k, v [rows][heads][head_dim] as bf16 bits, with their exact fp32 values under *_f32."""
    out = {}
    for name in ("q", "k", "v"):
        v = _normal(cfg_id, name, (rows, heads, head_dim))
        if name == "q" and q_scale != 1.0:
            v = (v * np.float32(q_scale)).astype(np.float32)
        bits = bf16_bits_from_f32(v)
        out[name], out[name + "_f32"] = bits, f32_from_bf16_bits(bits)
    return out


def make_swa_inputs_torch(cfg_id: int, rows: int, heads: int, head_dim: int, device) -> dict:
    """Device bf16 q, k, v [rows][heads][head_dim] ~ N(0, 1)."""
    import torch
    return {name: _torch_normal(torch, (rows, heads, head_dim), cfg_id, TENSOR_IDS[name], device, torch.bfloat16)
            for name in ("q", "k", "v")}


def make_positions_np(cfg_id: int, n: int, lo: int, hi: int) -> np.ndarray:
    """n decode positions drawn uniformly from [lo, hi] (int32)."""
    return _rng(cfg_id, TENSOR_IDS["pos"]).integers(lo, hi + 1, size=n).astype(np.int32)


# --------------------------------------------------------------------------- #
# grouped prefill
# --------------------------------------------------------------------------- #
def make_groups_inputs_np(cfg_id: int, rows: int, dim: int, ngroups: int, dstate: int, in_dtype: str = "bf16") -> dict:
    """x, dt, z [rows][dim], B, C [rows][ngroups][dstate] (device representation and *_f32), params."""
    out = {}
    for name, shape in (("x", (rows, dim)), ("z", (rows, dim)), ("dt", (rows, dim)),
                        ("B", (rows, ngroups, dstate)), ("C", (rows, ngroups, dstate))):
        v = _normal(cfg_id, name, shape)
        if in_dtype == "bf16":
            bits = bf16_bits_from_f32(v)
            out[name], out[name + "_f32"] = bits, f32_from_bf16_bits(bits)
        else:
            out[name], out[name + "_f32"] = v, v
    out.update(make_params(cfg_id, dim, dstate))
    return out


def make_groups_inputs_torch(cfg_id: int, rows: int, dim: int, ngroups: int, dstate: int, device) -> dict:
    """Device bf16 x, dt, z [rows][dim], B, C [rows][ngroups][dstate] (+ fp32 params)."""
    import torch
    out = {}
    for name, shape in (("x", (rows, dim)), ("z", (rows, dim)), ("dt", (rows, dim)),
                        ("B", (rows, ngroups, dstate)), ("C", (rows, ngroups, dstate))):
        out[name] = _torch_normal(torch, shape, cfg_id, TENSOR_IDS[name], device, torch.bfloat16)
    for k, v in make_params(cfg_id, dim, dstate).items():
        out[k] = torch.from_numpy(v).to(device)
    return out


# --------------------------------------------------------------------------- #
# state-space duality layer: per-head parameters, [tokens][heads][head_dim] activations
# --------------------------------------------------------------------------- #
def make_ssd_params(cfg_id: int, heads: int) -> dict:
    """A [heads] = -exp(U(0, log 16)), D [heads] ~ U(0, 1), dt_bias [heads] = log(expm1(U(1e-3, 1e-1)))."""
    u = _rng(cfg_id, TENSOR_IDS["dt_init"]).uniform(1e-3, 1e-1, size=heads)
    dt_bias = np.log(np.expm1(u)).astype(np.float32)
    A = (-np.exp(_rng(cfg_id, TENSOR_IDS["A"]).uniform(0.0, math.log(16.0), size=heads))).astype(np.float32)
    D = _rng(cfg_id, TENSOR_IDS["D"]).uniform(0.0, 1.0, size=heads).astype(np.float32)
    return {"A": A, "D": D, "dt_bias": dt_bias}


def make_retention_params(heads: int) -> dict:
    """Multi-scale retention as the duality form's parameters: decay γ_h = 1 - 2^(-5-h) per head (A = ln γ_h),
    Δ = 1 (dt = 0 with dt_bias = ln(e - 1), whose softplus is 1), no skip (D = 0)."""
    gam = 1.0 - 2.0 ** (-5.0 - np.arange(heads, dtype=np.float64))
    return {"A": np.log(gam).astype(np.float32), "D": np.zeros(heads, dtype=np.float32),
            "dt_bias": np.full(heads, math.log(math.e - 1.0), dtype=np.float32)}


def _ssd_shapes(rows, heads, head_dim, ngroups, dstate):
    return (("x", (rows, heads, head_dim)), ("z", (rows, heads, head_dim)), ("dt", (rows, heads)),
            ("B", (rows, ngroups, dstate)), ("C", (rows, ngroups, dstate)))


def make_ssd_inputs_np(cfg_id: int, rows: int, heads: int, ngroups: int, dstate: int, head_dim: int = 64) -> dict:
    """bf16 bits of x, z [rows][heads][head_dim], dt [rows][heads], B, C [rows][ngroups][dstate] (and *_f32,
    their exact fp32 values), all N(0, 1); params as make_ssd_params."""
    out = {}
    for name, shape in _ssd_shapes(rows, heads, head_dim, ngroups, dstate):
        bits = bf16_bits_from_f32(_normal(cfg_id, name, shape))
        out[name], out[name + "_f32"] = bits, f32_from_bf16_bits(bits)
    out.update(make_ssd_params(cfg_id, heads))
    return out


def make_ssd_inputs_torch(cfg_id: int, rows: int, heads: int, ngroups: int, dstate: int, device,
                          head_dim: int = 64) -> dict:
    """The same tensors generated on the device (bf16; fp32 params)."""
    import torch
    out = {}
    for name, shape in _ssd_shapes(rows, heads, head_dim, ngroups, dstate):
        out[name] = _torch_normal(torch, shape, cfg_id, TENSOR_IDS[name], device, torch.bfloat16)
    for k, v in make_ssd_params(cfg_id, heads).items():
        out[k] = torch.from_numpy(v).to(device)
    return out


def make_ssd_h0(cfg_id: int, nseq: int, heads: int, dstate: int, head_dim: int = 64, scale: float = 1.0):
    return (scale * _rng(cfg_id, TENSOR_IDS["h0"]).standard_normal((nseq, heads, head_dim, dstate))).astype(np.float32)


# --------------------------------------------------------------------------- #
# gated linear attention: q, k, log decay gk [tokens][heads][N], v [tokens][heads][P]
# --------------------------------------------------------------------------- #
def _gla_values(cfg_id: int, rows: int, heads: int, dstate: int, head_dim: int) -> dict:
    """fp32 values before the bf16 rounding: q ~ N(0,1)/sqrt(N), k, v ~ N(0,1), gk = logsigmoid(N(0,1)) / 16
    (the GLA paper's gate with temperature 16: decays in (0, 1), mostly close to 1)."""
    q = _normal(cfg_id, "q", (rows, heads, dstate)) / np.float32(math.sqrt(dstate))
    k = _normal(cfg_id, "k", (rows, heads, dstate))
    v = _normal(cfg_id, "v", (rows, heads, head_dim))
    g = _normal(cfg_id, "gk", (rows, heads, dstate)).astype(np.float64)
    gk = (-np.logaddexp(0.0, -g) / 16.0).astype(np.float32)
    return {"q": q, "k": k, "v": v, "gk": gk}


def make_gla_inputs_np(cfg_id: int, rows: int, heads: int, dstate: int, head_dim: int, in_dtype: str = "bf16") -> dict:
    """q, k, gk [rows][heads][dstate], v [rows][heads][head_dim]: device representation and *_f32 (exact values)."""
    out = {}
    for name, v in _gla_values(cfg_id, rows, heads, dstate, head_dim).items():
        if in_dtype == "bf16":
            bits = bf16_bits_from_f32(v)
            out[name], out[name + "_f32"] = bits, f32_from_bf16_bits(bits)
        else:
            out[name], out[name + "_f32"] = v, v
    return out


def make_gla_inputs_torch(cfg_id: int, rows: int, heads: int, dstate: int, head_dim: int, device) -> dict:
    """The same distributions generated on the device (bf16)."""
    import torch
    q = _torch_normal(torch, (rows, heads, dstate), cfg_id, TENSOR_IDS["q"], device, torch.float32)
    k = _torch_normal(torch, (rows, heads, dstate), cfg_id, TENSOR_IDS["k"], device, torch.bfloat16)
    v = _torch_normal(torch, (rows, heads, head_dim), cfg_id, TENSOR_IDS["v"], device, torch.bfloat16)
    g = _torch_normal(torch, (rows, heads, dstate), cfg_id, TENSOR_IDS["gk"], device, torch.float32)
    return {"q": (q / math.sqrt(dstate)).to(torch.bfloat16), "k": k, "v": v,
            "gk": (torch.nn.functional.logsigmoid(g) / 16.0).to(torch.bfloat16)}
