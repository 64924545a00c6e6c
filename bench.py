"""Benchmark of the selective scan on one MI355X.

Step = one pass of the long-prompt prefill: L = 131072 tokens, D = 4096
channels, 16 states, bf16 I/O and fp32 state, fed as 8 chained calls of 16384
tokens with the state carried h0 -> h_last between calls.  Inputs are seeded
synthetic tensors already resident in HBM.  `value` is algorithmic GB/s of
that prefill (bytes the method must move: x, dt, z in and y out, B and C per
token, parameters, carry in and out).  The streaming decode (batch 64, D 4096,
65536 consecutive single-token steps over a ring of 256 input sets, state from
a 2048-token prefill) is reported in the same line under "decode", and the
backward on the training shape (batch 4 x 4096 tokens, D 4096: gradients of
every input, forward states recomputed inside the call) under "backward".
The other prefill configurations (B1 L4096 D2048; a packed 32768-token stream
of 512..4096-token sequences), the complexity checks (prefill time against L,
decode-step time against the tokens before it), a decode over 24 independent
states (384 MiB, beyond the last-level cache) and the measured ALU issue rates
that give the prefill's ceiling are reported beside them.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode] [--no-cpu]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "scan GB/s & tokens·channels/s at L=128K, % HBM roofline; decode steps/s"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak (no sparsity)
# VALU issue peak: 256 CUs x 4 SIMDs x 32 fp32 lanes/clock x 2.4 GHz (one slot = one full-rate fp32 lane op)
VALU_PEAK_TSLOT = 256 * 4 * 32 * 2.4e9 / 1e12
TRANS_SLOTS = 4            # a transcendental (exp2, log2, rcp) issues at a quarter of the fp32 rate
# Algorithmic work of the plain sequential recurrence per (token, channel):
#   16 states x (Δ*A mul, exp, Δx*B mul, state FMA, readout FMA) = 64 VALU + 16 transcendentals
#   softplus(dt + bias): add, exp, log1p (~2 VALU + 2 transcendentals); Δ*x: 1; skip: 1 FMA;
#   silu gate: exp, rcp, 2 VALU; gate multiply: 1; bf16 widen x3 + narrow x1: 4
VALU_PER_TD = 64 + 2 + 1 + 1 + 2 + 1 + 4
TRANS_PER_TD = 16 + 2 + 2
SLOTS_PER_TD = VALU_PER_TD + TRANS_SLOTS * TRANS_PER_TD
# Backward, per (token, channel), the plain algorithm: per state the forward recompute (Δ*A mul, exp, Δx*B mul,
# state FMA), the readout FMA of r, and the reverse step (adjoint FMA, Ā*h_prev, g*u, dA FMA, dΔ FMA, dx FMA,
# dB and dC products, adjoint decay, and the two channel-sum adds of dB and dC) = 16 x (15 VALU + 1 exp);
# per token and channel: softplus (2 transcendentals), sigmoid(v) and sigmoid(z) (2 each), silu' and dr, dz,
# dx, ddt, the dD and ddt_bias sums, 4 bf16 widenings and 3 narrowings (~20 VALU).
BWD_VALU_PER_TD = 16 * 15 + 20
BWD_TRANS_PER_TD = 16 + 6
BWD_SLOTS_PER_TD = BWD_VALU_PER_TD + TRANS_SLOTS * BWD_TRANS_PER_TD
# the scan's kernels: samba_scan.hip, the prefill kernel's header and its separately scheduled copy
KERNEL_SRCS = tuple(ROOT / "selective_state_space_05_amd" / "csrc" / n
                    for n in ("samba_scan.hip", "samba_scan_fwd.h", "samba_scan_fwd_ilp.hip"))
TRAFFIC_FILE = ROOT / "profiles" / "hbm_traffic_fwd_step_bwd_proj.json"
SWA_SRC = ROOT / "selective_state_space_05_amd" / "csrc" / "samba_swa.hip"
SWA_TRAFFIC_FILE = ROOT / "profiles" / "hbm_traffic_swa.json"
GROUPS_SRC = ROOT / "selective_state_space_05_amd" / "csrc" / "samba_scan_groups.hip"
GROUPS_TRAFFIC_FILE = ROOT / "profiles" / "hbm_traffic_groups.json"
SSD_SRC = ROOT / "selective_state_space_05_amd" / "csrc" / "samba_ssd.hip"
SSD_TRAFFIC_FILE = ROOT / "profiles" / "hbm_traffic_ssd.json"
GLA_SRC = ROOT / "selective_state_space_05_amd" / "csrc" / "samba_gla.hip"
GLA_TRAFFIC_FILE = ROOT / "profiles" / "hbm_traffic_gla.json"


def groups_bytes(batch: int, L: int, dim: int, ngroups: int, n: int) -> int:
    """Algorithmic bytes of one grouped prefill: x, dt, z in and y out (bf16), B and C (bf16), A, D, dt_bias,
    h_last out."""
    return batch * L * dim * 4 * 2 + batch * L * ngroups * n * 2 * 2 + dim * n * 4 + dim * 8 + batch * dim * n * 4


def visible_keys(L: int, window: int) -> int:
    """Sum over the queries of one L-token sequence of the keys each sees (min(i + 1, window + 1))."""
    m = min(L, window + 1)
    return m * (m + 1) // 2 + (L - m) * (window + 1)


def swa_flops(batch: int, L: int, heads: int, hd: int, window: int) -> int:
    """Algorithmic flops of the attention: per visible (query, key) pair a q.k dot and a p*v axpy of hd each."""
    return 4 * hd * heads * batch * visible_keys(L, window)


def swa_decode_bytes(batch: int, heads: int, hd: int, window: int) -> int:
    """Bytes one decode step must move: the window's cached keys and values (window rows each), the new q, k,
    v rows in, k and v written to the cache, o out (bf16)."""
    return batch * heads * hd * 2 * (2 * window + 3 + 2 + 1)


def prefill_bytes(tokens: int, dim: int, io_bytes: int = 2, h0: bool = True, h_last: bool = True, n: int = 16) -> int:
    b = tokens * dim * 4 * io_bytes          # x, dt, z in; y out
    b += tokens * 2 * n * io_bytes           # B, C
    b += dim * n * 4 + dim * 8               # A, D, dt_bias
    b += (dim * n * 4 if h0 else 0) + (dim * n * 4 if h_last else 0)
    return b


def bwd_bytes(tokens: int, dim: int, nseq: int, io_bytes: int = 2, n: int = 16) -> int:
    b = tokens * dim * 7 * io_bytes          # x, dt, z, dy in; dx, ddt, dz out
    b += tokens * 2 * n * io_bytes           # B, C in
    b += tokens * 2 * n * 4                  # dB, dC out (fp32)
    b += dim * n * 4 * 2 + dim * 8 * 2       # A, D, dt_bias in; dA, dD, ddt_bias out
    b += nseq * dim * n * 4                  # dh0 out
    return b


def decode_bytes(batch: int, dim: int, n: int = 16) -> int:
    return batch * dim * (2 * n * 4 + 4 * 2) + batch * 2 * n * 2 + dim * n * 4 + dim * 8


def kernel_hash() -> str:
    """Source key of the scan's counter summaries: its sources and the per-source compiler flags."""
    from selective_state_space_05_amd import build as _build
    h = hashlib.sha256()
    for src in KERNEL_SRCS:
        h.update(src.read_bytes())
    h.update(repr(sorted((k.name, v) for k, v in _build.SRC_FLAGS.items() if k in KERNEL_SRCS)).encode())
    return h.hexdigest()[:16]


def swa_hash() -> str:
    return hashlib.sha256(SWA_SRC.read_bytes()).hexdigest()[:16]


def groups_hash() -> str:
    return hashlib.sha256(GROUPS_SRC.read_bytes()).hexdigest()[:16]


def read_groups_traffic(part: str = "groups"):
    """HBM bytes per launch of the grouped prefill ("groups") or decode step ("decode") from the committed
    counter runs, if they were taken on this kernel source."""
    try:
        t = json.loads(GROUPS_TRAFFIC_FILE.read_text())
    except Exception:
        return None
    if t.get("kernel_source_sha256_16") != groups_hash():
        return None
    return t.get(part, {}).get("bytes_per_launch")


def gla_hash() -> str:
    return hashlib.sha256(GLA_SRC.read_bytes()).hexdigest()[:16]


def read_gla_traffic():
    """HBM bytes per launch of the GLA kernel from the committed counter runs, if they were taken on this
    kernel source."""
    try:
        t = json.loads(GLA_TRAFFIC_FILE.read_text())
    except Exception:
        return None
    if t.get("kernel_source_sha256_16") != gla_hash():
        return None
    return t.get("gla_call", {}).get("bytes_per_call")


def ssd_hash() -> str:
    return hashlib.sha256(SSD_SRC.read_bytes()).hexdigest()[:16]


def read_ssd_traffic():
    """HBM bytes per launch of the SSD prefill from the committed counter runs, if they were taken on this
    kernel source."""
    try:
        t = json.loads(SSD_TRAFFIC_FILE.read_text())
    except Exception:
        return None
    if t.get("kernel_source_sha256_16") != ssd_hash():
        return None
    return t.get("ssd", {}).get("bytes_per_launch")


RETENTION_TRAFFIC_FILE = ROOT / "profiles" / "hbm_traffic_retention.json"


def read_retention_traffic():
    """HBM bytes per retention call (one prefill launch) from the committed counter runs, if they were taken on
    this kernel source."""
    try:
        t = json.loads(RETENTION_TRAFFIC_FILE.read_text())
    except Exception:
        return None
    if t.get("kernel_source_sha256_16") != ssd_hash():
        return None
    return t.get("retention_call", {}).get("bytes_per_call")


def read_swa_traffic(part: str):
    """HBM bytes per launch of the attention kernels (prefill, decode) from the committed counter runs, if
    they were taken on this kernel source."""
    try:
        t = json.loads(SWA_TRAFFIC_FILE.read_text())
    except Exception:
        return None
    if t.get("kernel_source_sha256_16") != swa_hash():
        return None
    return t.get(part, {}).get("bytes_per_launch")


def read_traffic(part: str = "forward"):
    """HBM bytes per launch (forward, decode_step, projections) or per call (backward) from the committed
    rocprofv3 counter runs, if they were taken on this kernel source."""
    try:
        t = json.loads(TRAFFIC_FILE.read_text())
    except Exception:
        return None
    if t.get("kernel_source_sha256_16") != kernel_hash():
        return None
    if part == "backward":
        return t.get("backward", {}).get("bytes_per_call")
    return t.get(part, {}).get("bytes_per_launch")


def bench_prefill(steps: int, warmup: int, time_slices: int = 0):
    import torch
    from selective_state_space_05_amd import inputs as I
    from selective_state_space_05_amd import scan as S

    W = I.WORKLOADS[3]
    L, D, n = W.seqlen, W.dim, W.chunks
    cl = L // n
    dev = torch.device("cuda:0")
    inp = I.make_fwd_inputs_torch(3, L, D, dev)
    y = torch.empty(L, D, dtype=torch.bfloat16, device=dev)
    h0 = torch.zeros(1, D, 16, device=dev)
    hb = [torch.empty(1, D, 16, device=dev) for _ in range(2)]
    lib = S.load_library()
    stream = torch.cuda.current_stream()
    args = []
    prev = h0
    for i in range(n):
        sl = slice(i * cl, (i + 1) * cl)
        a = S.fwd_args(*(inp[k][sl].view(1, cl, -1) for k in ("x", "dt", "z", "B", "C")), inp["A"], inp["D"],
                       inp["dt_bias"], y=y[sl].view(1, cl, D), h0=prev, h_last=hb[i % 2], time_slices=time_slices)
        args.append(a)
        prev = hb[i % 2]
    plan = S.fwd_plan(*(inp[k][:cl].view(1, cl, -1) for k in ("x", "dt", "z", "B", "C")), inp["A"], inp["D"],
                      inp["dt_bias"], y=y[:cl].view(1, cl, D), h0=h0, h_last=hb[0], time_slices=time_slices)
    sh = ctypes.c_void_p(stream.cuda_stream)

    def one_step():
        for a in args:
            st = lib.samba_scan_fwd(ctypes.byref(a), sh)
            if st != 0:
                raise S.SambaError(st, "samba_scan_fwd")

    for _ in range(warmup):
        one_step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        one_step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    launch_ms = ms / n
    # per-call durations (each call bracketed by its own events), after the interval timing above
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n * steps + 1)]
    evs[0].record(stream)
    for s in range(steps):
        for i, a in enumerate(args):
            if lib.samba_scan_fwd(ctypes.byref(a), sh) != 0:
                raise RuntimeError("samba_scan_fwd failed")
            evs[s * n + i + 1].record(stream)
    torch.cuda.synchronize()
    per_call = sorted(evs[k].elapsed_time(evs[k + 1]) * 1e3 for k in range(n * steps))
    tokens_ch = L * D
    step_bytes = n * prefill_bytes(cl, D)
    return {
        "ms_per_step": ms,
        "gbs": step_bytes / (ms * 1e-3) / 1e9,
        "tokens_channels_per_s": tokens_ch / (ms * 1e-3),
        "launch_ms": launch_ms,
        "launch_td": cl * D,
        "bytes_per_launch": prefill_bytes(cl, D),
        "plan": {"time_slices": plan[0], "workgroups": plan[1], "threads_per_workgroup": plan[2],
                 "lanes_per_channel": plan[3]},
        "call_us": {"median": per_call[len(per_call) // 2], "min": per_call[0], "calls": len(per_call)},
    }


def bench_backward(steps: int = 10, warmup: int = 5):
    """samba_scan_bwd on the training shape: batch 4 x 4096 tokens, D 4096, bf16, no carries in or out."""
    import torch
    from selective_state_space_05_amd import inputs as I
    from selective_state_space_05_amd import scan as S

    W = I.WORKLOADS[5]
    Bt, L, D = W.batch, W.seqlen, W.dim
    dev = torch.device("cuda:0")
    inp = I.make_fwd_inputs_torch(5, Bt * L, D, dev)
    ex = I.make_bwd_extra_torch(5, Bt * L, D, Bt, dev)
    shp, bshp = (Bt, L, D), (Bt, L, 16)
    x, dt, z, dy = (t.view(shp) for t in (inp["x"], inp["dt"], inp["z"], ex["dy"]))
    B, C = inp["B"].view(bshp), inp["C"].view(bshp)
    out = {k: torch.empty_like(x) for k in ("dx", "ddt", "dz")}
    out["dB"], out["dC"] = (torch.empty(bshp, dtype=torch.float32, device=dev) for _ in range(2))
    out["dA"] = torch.empty(D, 16, dtype=torch.float32, device=dev)
    out["dD"], out["ddt_bias"] = (torch.empty(D, dtype=torch.float32, device=dev) for _ in range(2))
    out["dh0"] = torch.empty(Bt, D, 16, dtype=torch.float32, device=dev)
    a = S.bwd_args(x, dt, z, B, C, inp["A"], inp["D"], inp["dt_bias"], dy, **out)
    ws = torch.empty(S.bwd_workspace_bytes(a), dtype=torch.uint8, device=dev)
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    lib = S.load_library()
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)

    def call():
        st = lib.samba_scan_bwd(ctypes.byref(a), sh)
        if st != 0:
            raise S.SambaError(st, "samba_scan_bwd")

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    td = Bt * L * D
    nbytes = bwd_bytes(Bt * L, D, Bt)
    slots = BWD_SLOTS_PER_TD * td / (ms * 1e-3) / 1e12

    # training route: the forward writes y and the checkpoints; the backward reuses them
    y = torch.empty_like(x)
    ck = S.alloc_ckpt(x)
    fa = S.fwd_args(x, dt, z, B, C, inp["A"], inp["D"], inp["dt_bias"], y=y)
    fc = S.fwd_args(x, dt, z, B, C, inp["A"], inp["D"], inp["dt_bias"], y=y, h_ckpt=ck)
    bc = S.bwd_args(x, dt, z, B, C, inp["A"], inp["D"], inp["dt_bias"], dy, h_ckpt=ck, **out)
    bc.workspace, bc.workspace_bytes = ws.data_ptr(), ws.numel()

    def timed(args, fn):
        for _ in range(warmup):
            fn(ctypes.byref(args), sh)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            if fn(ctypes.byref(args), sh) != 0:
                raise RuntimeError("call failed")
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    fwd_ms = timed(fa, lib.samba_scan_fwd)
    fwd_ck_ms = timed(fc, lib.samba_scan_fwd)
    bwd_ck_ms = timed(bc, lib.samba_scan_bwd)
    return {"workload": "backward B=4 L=4096 D=4096 N=16 bf16 (training shape), all gradients",
            "steps": steps, "ms_per_call": ms, "tokens_channels_per_s": td / (ms * 1e-3),
            "training_route": {"fwd_ms": fwd_ms, "fwd_with_checkpoints_ms": fwd_ck_ms,
                               "bwd_from_checkpoints_ms": bwd_ck_ms,
                               "fwd_plus_bwd_ms": fwd_ck_ms + bwd_ck_ms,
                               "fwd_plus_self_contained_bwd_ms": fwd_ms + ms},
            "gbs": nbytes / (ms * 1e-3) / 1e9, "algorithmic_bytes": nbytes, "workspace_bytes": ws.numel(),
            "roofline": {"bound": "alu", "achieved": round(slots, 3), "peak": round(VALU_PEAK_TSLOT, 2),
                         "unit": "Tslot/s", "frac": round(slots / VALU_PEAK_TSLOT, 4), "traffic": None,
                         "kernel": "samba_scan_bwd call (checkpoint + backward + finish kernels)",
                         "slots_per_token_channel": BWD_SLOTS_PER_TD}}


def bench_proj(steps: int = 20, warmup: int = 5):
    """samba_proj on the long-prompt chunk: 16384 tokens, D 4096 -> dt_raw, B, C (bf16 out)."""
    import torch
    from selective_state_space_05_amd import inputs as I
    from selective_state_space_05_amd import scan as S

    T, D, N = 16384, 4096, 16
    dev = torch.device("cuda:0")
    x = I.make_fwd_inputs_torch(3, T, D, dev)["x"]
    W = I.make_proj_weight_torch(3, D, dev)
    dt = torch.empty(T, D, dtype=torch.bfloat16, device=dev)
    B = torch.empty(T, N, dtype=torch.bfloat16, device=dev)
    C = torch.empty(T, N, dtype=torch.bfloat16, device=dev)
    a = S.proj_args(x, W, dt=dt, B=B, C=C)
    lib = S.load_library()
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    for _ in range(warmup):
        lib.samba_proj(ctypes.byref(a), sh)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        if lib.samba_proj(ctypes.byref(a), sh) != 0:
            raise RuntimeError("samba_proj failed")
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 2.0 * T * (D + 2 * N) * D
    tf = flops / (ms * 1e-3) / 1e12
    nbytes = (T * D + (D + 2 * N) * D + T * (D + 2 * N)) * 2
    return {"workload": "selection projections x[16384][4096] W[4128][4096] bf16 -> dt_raw, B, C (bf16)",
            "steps": steps, "ms_per_call": ms, "tflops": tf, "tokens_per_s": T / (ms * 1e-3),
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                         "kernel": "proj_dma_kernel<bf16, BK=64, 2 stages, 2x4 waves> (v_mfma_f32_32x32x16_bf16, operands loaded straight into LDS)", "flops_per_call": flops,
                         "algorithmic_bytes_per_call": nbytes}}


def cpu_baseline_proj(rows: int = 1024):
    """The fp64 oracle's projections on `rows` tokens of the same shape (D 4096), extrapolated to TFLOP/s."""
    import numpy as np
    from oracle import oracle as O
    from selective_state_space_05_amd import inputs as I

    D = 4096
    x = I.make_fwd_inputs_np(3, rows, D, in_dtype="bf16")["x_f32"]
    W = I.make_proj_weight_np(3, D)["W_f32"]
    lib = O.load()
    t0 = time.perf_counter()
    O.proj(x, W, lib=lib)
    spent = time.perf_counter() - t0
    return {"value": 2.0 * rows * (D + 32) * D / spent / 1e12, "unit": "TFLOP/s", "cores": O.max_threads(lib),
            "kind": "oracle", "sample": "%d of the 16384 tokens, all 4128 outputs, fp64 oracle, %.1f s" % (rows, spent)}


def bench_decode(steps: int = 65536, ring: int = 256):
    import torch
    from selective_state_space_05_amd import inputs as I
    from selective_state_space_05_amd import scan as S

    W = I.WORKLOADS[4]
    Bt, L, D = W.batch, W.seqlen, W.dim
    dev = torch.device("cuda:0")
    pre = I.make_fwd_inputs_torch(4, Bt * L, D, dev)
    _, state = S.scan_fwd(*(pre[k].view(Bt, L, -1) for k in ("x", "dt", "z", "B", "C")), pre["A"], pre["D"],
                          pre["dt_bias"])
    del pre["x"], pre["dt"], pre["z"]
    rg = I.make_step_ring_torch(4, ring, Bt, D, dev)
    ys = torch.empty(ring, Bt, D, dtype=torch.bfloat16, device=dev)
    lib = S.load_library()
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    args = [S.step_args(state, rg["x"][r], rg["dt"][r], rg["z"][r], rg["B"][r], rg["C"][r], pre["A"], pre["D"],
                        pre["dt_bias"], y=ys[r]) for r in range(ring)]
    refs = [ctypes.byref(a) for a in args]
    f = lib.samba_scan_step
    for r in range(ring):
        f(refs[r], sh)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for k in range(steps):
        if f(refs[k & (ring - 1)], sh) != 0:
            raise RuntimeError("samba_scan_step failed")
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    us = ms * 1e3 / steps
    out = {"steps": steps, "us_per_step": us, "steps_per_s": steps / (ms * 1e-3),
           "gbs": decode_bytes(Bt, D) / (us * 1e-6) / 1e9}
    out["hbm_frac"] = out["gbs"] / HBM_PEAK_GBS
    # the same steps captured by the caller into a graph (one replay = one pass over the ring)
    try:
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(stream)
        with torch.cuda.stream(cs):
            f(refs[0], ctypes.c_void_p(cs.cuda_stream))
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cs):
            csh = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for r in range(ring):
                f(refs[r], csh)
        torch.cuda.synchronize()
        reps = steps // ring
        g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        gus = e0.elapsed_time(e1) * 1e3 / (reps * ring)
        out["graph"] = {"us_per_step": gus, "steps_per_s": 1e6 / gus,
                        "gbs": decode_bytes(Bt, D) / (gus * 1e-6) / 1e9}
    except Exception as ex:  # graph capture is an optional, separately reported variant
        out["graph"] = {"error": repr(ex)[:200]}
    return out


def _timed(fn, steps: int, stream):
    """Average ms of `steps` calls of fn() between two events on `stream`."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def groups_slots_per_td(n: int) -> int:
    """Algorithmic issue slots per (token, channel) of the grouped prefill with n states: per state the Δ·A
    mul, the exp (4 slots), the Δx·B mul, the state FMA and the readout FMA (8); per (token, channel)
    softplus and silu (2 transcendentals each), Δx, skip, gate and 4 bf16 conversions (28)."""
    return 8 * n + 28


def bench_groups(steps: int = 10, warmup: int = 3):
    """samba_scan_fwd_groups on B4 L4096 D4096 with 4 (B, C) groups of 64 states (bf16 I/O)."""
    import torch
    from selective_state_space_05_amd import inputs as I
    from selective_state_space_05_amd import scan as S

    wl = I.WORKLOADS[8]
    Bt, L, D, N, G = wl.batch, wl.seqlen, wl.dim, wl.dstate, wl.extra["ngroups"]
    dev = torch.device("cuda:0")
    t = I.make_groups_inputs_torch(8, Bt * L, D, G, N, dev)
    x, dt, z = (t[k].view(Bt, L, D) for k in ("x", "dt", "z"))
    B, C = (t[k].view(Bt, L, G, N) for k in ("B", "C"))
    y = torch.empty_like(x)
    hl = torch.empty(Bt, D, N, dtype=torch.float32, device=dev)
    a = S.groups_args(x, dt, z, B, C, t["A"], t["D"], t["dt_bias"], y=y, h_last=hl)
    lib = S.load_library()
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    ref = ctypes.byref(a)

    def call():
        if lib.samba_scan_fwd_groups(ref, sh) != 0:
            raise RuntimeError("samba_scan_fwd_groups failed")

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ms = _timed(call, steps, stream)
    td = Bt * L * D
    slots = groups_slots_per_td(N) * td
    achieved = slots / (ms * 1e-3) / 1e12
    nbytes = groups_bytes(Bt, L, D, G, N)
    return {"workload": "grouped prefill B=%d L=%d D=%d, %d (B, C) groups of %d states, bf16 I/O, fp32 state"
                        % (Bt, L, D, G, N),
            "steps": steps, "ms_per_call": ms, "tokens_channels_per_s": td / (ms * 1e-3),
            "gbs": nbytes / (ms * 1e-3) / 1e9,
            "roofline": {"bound": "alu", "achieved": round(achieved, 3), "peak": round(VALU_PEAK_TSLOT, 2),
                         "unit": "Tslot/s", "frac": round(achieved / VALU_PEAK_TSLOT, 4),
                         "traffic": read_groups_traffic(), "kernel": "scan_groups_kernel<bf16,bf16,N=%d>" % N, "launch_us": round(ms * 1e3, 2),
                         "slots_per_token_channel": groups_slots_per_td(N),
                         "algorithmic_bytes_per_launch": nbytes}}


def bench_groups_step(steps: int = 200, warmup: int = 20):
    """samba_scan_step_groups on 64 sequences x D 4096 with 4 groups of 64 states (state 64 MiB read and
    written per step); the state comes from random values of a prefill's scale."""
    import torch
    from selective_state_space_05_amd import inputs as I
    from selective_state_space_05_amd import scan as S

    wl = I.WORKLOADS[8]
    Bt, D, N, G = 64, wl.dim, wl.dstate, wl.extra["ngroups"]
    dev = torch.device("cuda:0")
    t = I.make_groups_inputs_torch(18, Bt, D, G, N, dev)
    state = torch.from_numpy(I.make_h0(18, Bt, D, N, scale=0.5)).to(dev)
    y = torch.empty(Bt, D, dtype=torch.bfloat16, device=dev)
    a = S.step_groups_args(state, t["x"], t["dt"], t["z"], t["B"], t["C"], t["A"], t["D"], t["dt_bias"], y=y)
    lib = S.load_library()
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    ref = ctypes.byref(a)

    def call():
        if lib.samba_scan_step_groups(ref, sh) != 0:
            raise RuntimeError("samba_scan_step_groups failed")

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ms = _timed(call, steps, stream)
    nbytes = Bt * D * N * 4 * 2 + Bt * D * 4 * 2 + Bt * G * N * 2 * 2 + D * N * 4 + D * 8
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": "grouped decode step: batch %d, D %d, %d groups of %d states, bf16 I/O" % (Bt, D, G, N),
            "steps": steps, "us_per_step": ms * 1e3, "gbs": gbs,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": read_groups_traffic("decode"),
                         "kernel": "step_groups_kernel<bf16,bf16,N=%d>" % N, "launch_us": round(ms * 1e3, 2),
                         "algorithmic_bytes_per_launch": nbytes}}


def cpu_baseline_groups(seqs: int = 1, channels: int = 512):
    """The fp64 oracle's grouped prefill on one sequence of the same shape, `channels` channels (128 per
    group), in token·channels/s."""
    import numpy as np
    from oracle import oracle as O
    from selective_state_space_05_amd import inputs as I

    wl = I.WORKLOADS[8]
    L, D, N, G = wl.seqlen, wl.dim, wl.dstate, wl.extra["ngroups"]
    inp = I.make_groups_inputs_np(8, L, D, G, N)
    per = D // G
    cols = np.concatenate([np.arange(g * per, g * per + channels // G) for g in range(G)])
    lib = O.load()
    t0 = time.perf_counter()
    O.scan_fwd_groups(inp["x_f32"][:, cols], inp["dt_f32"][:, cols], inp["z_f32"][:, cols], inp["B_f32"],
                      inp["C_f32"], inp["A"][cols], inp["D"][cols], inp["dt_bias"][cols], lib=lib)
    spent = time.perf_counter() - t0
    return {"value": L * channels / spent, "unit": "tokens*channels/s", "cores": O.max_threads(lib),
            "kind": "oracle", "sample": "one 4096-token sequence, %d of the 4096 channels (%d per group), fp64 "
                                        "oracle, %.1f s" % (channels, channels // G, spent)}


def ssd_bytes(batch: int, L: int, heads: int, hd: int, ngroups: int, n: int, gated: bool = True) -> int:
    """Algorithmic bytes of one SSD prefill: x (and z when gated) read and y written (bf16), dt (bf16), B and C
    (bf16), A, D, dt_bias, h_last out (fp32)."""
    T = batch * L
    return (T * heads * hd * 2 * (3 if gated else 2) + T * heads * 2 + T * ngroups * n * 2 * 2 + heads * 12 +
            batch * heads * hd * n * 4)


def ssd_flops(batch: int, L: int, heads: int, hd: int, n: int, q: int = 64) -> int:
    """Algorithmic flops of the chunked form per token and head: C Bᵀ (2qn), the masked product with x (2qP),
    the readout of the entering state (2nP) and the state update (2nP); full chunks, no split operands."""
    return batch * L * heads * (2 * q * n + 2 * q * hd + 4 * n * hd)


def _ssd_timed(forms, steps: int, warmup: int, rounds: int = 3):
    """ms per samba_ssd_fwd call for each args object in `forms` (a workspace attached where its form needs
    one): `rounds` rounds of `steps` calls of each in turn, after `warmup` calls of each; the median round."""
    import statistics
    import torch
    from selective_state_space_05_amd import ssd as SD

    dev = torch.device("cuda:0")
    lib = SD.load_library()
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    wss = [SD.attach_workspace(a, dev) for a in forms]

    def caller(a):
        ref = ctypes.byref(a)

        def call():
            if lib.samba_ssd_fwd(ref, sh) != 0:
                raise RuntimeError("samba_ssd_fwd failed")
        return call

    calls = [caller(a) for a in forms]
    for c in calls:
        for _ in range(warmup):
            c()
    torch.cuda.synchronize()
    per = [[_timed(c, steps, stream) for c in calls] for _ in range(rounds)]
    del wss
    return [statistics.median(r[i] for r in per) for i in range(len(forms))]


def bench_ssd(steps: int = 20, warmup: int = 5):
    """samba_ssd_fwd on B4 L4096 with 64 heads of 64, one (B, C) group of 128 states, gated, bf16 I/O: the
    default form (C B^T inside the prefill kernel) and the pre-pass form, timed in alternating rounds."""
    import torch
    from selective_state_space_05_amd import inputs as I
    from selective_state_space_05_amd import ssd as SD

    wl = I.WORKLOADS[9]
    Bt, L, H, P, N, G = (wl.batch, wl.seqlen, wl.extra["heads"], wl.extra["head_dim"], wl.dstate,
                         wl.extra["ngroups"])
    dev = torch.device("cuda:0")
    t = I.make_ssd_inputs_torch(9, Bt * L, H, G, N, dev)
    x, z = (t[k].view(Bt, L, H, P) for k in ("x", "z"))
    dt = t["dt"].view(Bt, L, H)
    B, C = (t[k].view(Bt, L, G, N) for k in ("B", "C"))
    y = torch.empty_like(x)
    hl = torch.empty(Bt, H, P, N, dtype=torch.float32, device=dev)
    mk = lambda mode: SD.fwd_args(x, dt, B, C, t["A"], t["D"], t["dt_bias"], y=y, z=z, h_last=hl, cb_mode=mode)
    ms, ms_pre = _ssd_timed([mk(SD.CB_AUTO), mk(SD.CB_PREPASS)], steps, warmup)
    nbytes = ssd_bytes(Bt, L, H, P, G, N)
    flops = ssd_flops(Bt, L, H, P, N)
    gbs = nbytes / (ms * 1e-3) / 1e9
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": "SSD prefill B=%d L=%d, %d heads of %d, %d (B, C) group of %d states, gated, bf16 I/O, "
                        "fp32 state" % (Bt, L, H, P, G, N),
            "steps": steps, "ms_per_call": ms, "tokens_per_s": Bt * L / (ms * 1e-3), "gbs": gbs,
            "mfma_tflops": round(tf, 1), "mfma_frac_bf16": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "ms_per_call_cb_prepass": ms_pre,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": read_ssd_traffic(),
                         "kernel": "ssd_fwd_kernel<bf16,N=%d,gate>, C B^T in kernel (one launch)" % N,
                         "launch_us": round(ms * 1e3, 2),
                         "algorithmic_bytes_per_launch": nbytes, "algorithmic_flops_per_launch": flops}}


def bench_retention(steps: int = 20, warmup: int = 5):
    """Multi-scale retention through samba_ssd_fwd: B4 L4096, 32 heads of 64 values with 128 keys each (one
    (k, q) group per head: B = k, C = q, x = v), Δ = 1, A = ln γ_h, no skip, no gate, bf16 I/O; the default
    form and the pre-pass form, timed in alternating rounds."""
    import torch
    from selective_state_space_05_amd import inputs as I
    from selective_state_space_05_amd import ssd as SD

    wl = I.WORKLOADS[11]
    Bt, L, H, P, N, G = (wl.batch, wl.seqlen, wl.extra["heads"], wl.extra["head_dim"], wl.dstate,
                         wl.extra["ngroups"])
    dev = torch.device("cuda:0")
    t = I.make_ssd_inputs_torch(11, Bt * L, H, G, N, dev)
    rp = {k: torch.from_numpy(v).to(dev) for k, v in I.make_retention_params(H).items()}
    x = t["x"].view(Bt, L, H, P)
    dt = torch.zeros(Bt, L, H, dtype=torch.bfloat16, device=dev)
    B, C = (t[k].view(Bt, L, G, N) for k in ("B", "C"))
    y = torch.empty_like(x)
    hl = torch.empty(Bt, H, P, N, dtype=torch.float32, device=dev)
    mk = lambda mode: SD.fwd_args(x, dt, B, C, rp["A"], rp["D"], rp["dt_bias"], y=y, h_last=hl, cb_mode=mode)
    ms, ms_pre = _ssd_timed([mk(SD.CB_AUTO), mk(SD.CB_PREPASS)], steps, warmup)
    nbytes = ssd_bytes(Bt, L, H, P, G, N, gated=False)
    flops = ssd_flops(Bt, L, H, P, N)
    gbs = nbytes / (ms * 1e-3) / 1e9
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": "multi-scale retention B=%d L=%d, %d heads of %d values and %d keys (one (k, q) group per "
                        "head), no gate, bf16 I/O, fp32 state" % (Bt, L, H, P, N),
            "steps": steps, "ms_per_call": ms, "tokens_per_s": Bt * L / (ms * 1e-3), "gbs": gbs,
            "mfma_tflops": round(tf, 1), "mfma_frac_bf16": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "ms_per_call_cb_prepass": ms_pre,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": read_retention_traffic(),
                         "kernel": "ssd_fwd_kernel<bf16,N=%d,no gate>, C B^T in kernel (one launch)" % N,
                         "launch_us": round(ms * 1e3, 2),
                         "algorithmic_bytes_per_launch": nbytes, "algorithmic_flops_per_launch": flops}}


def cpu_baseline_ssd():
    """The fp64 oracle's SSD recurrence on the whole workload (4 sequences of 4096 tokens, 64 heads), in
    tokens/s like the GPU leg."""
    import numpy as np
    from oracle import oracle as O
    from selective_state_space_05_amd import inputs as I

    wl = I.WORKLOADS[9]
    Bt, L, H, N, G = wl.batch, wl.seqlen, wl.extra["heads"], wl.dstate, wl.extra["ngroups"]
    inp = I.make_ssd_inputs_np(9, Bt * L, H, G, N)
    lib = O.load()
    t0 = time.perf_counter()
    O.ssd(inp["x_f32"], inp["dt_f32"], inp["B_f32"], inp["C_f32"], inp["A"], inp["D"], inp["dt_bias"],
          z=inp["z_f32"], seq_start=np.arange(Bt + 1, dtype=np.int64) * L, lib=lib)
    spent = time.perf_counter() - t0
    return {"value": Bt * L / spent, "unit": "tokens/s", "cores": O.max_threads(lib), "kind": "oracle",
            "sample": "the whole workload (%d x %d tokens, %d heads), fp64 oracle, %.1f s" % (Bt, L, H, spent)}


def gla_bytes(batch: int, L: int, heads: int, n: int, pv: int) -> int:
    """Algorithmic bytes of one GLA call: q, k, gk and v read, o written once (bf16), h_last out (fp32)."""
    T = batch * L
    return T * heads * (3 * n + 2 * pv) * 2 + batch * heads * pv * n * 4


def gla_flops(batch: int, L: int, heads: int, n: int, pv: int, chunk: int = 64) -> int:
    """Algorithmic flops of the chunked form: per token and head the inter-chunk readout and the state update
    (2 N P each), the intra-chunk A V and A (causal: half of 2 C P and 2 C N)."""
    T = batch * L
    return T * heads * (4 * n * pv + chunk * pv + chunk * n)


def bench_gla(steps: int = 5, warmup: int = 2):
    """samba_gla_fwd on B4 L4096 with 4 heads, keys 256, values 512 (bf16 I/O, fp32 state)."""
    import torch
    from selective_state_space_05_amd import gla as GL
    from selective_state_space_05_amd import inputs as I

    wl = I.WORKLOADS[10]
    Bt, L, H, N, P = wl.batch, wl.seqlen, wl.extra["heads"], wl.dstate, wl.extra["head_dim"]
    dev = torch.device("cuda:0")
    t = I.make_gla_inputs_torch(10, Bt * L, H, N, P, dev)
    q, k, gk = (t[n].view(Bt, L, H, N) for n in ("q", "k", "gk"))
    v = t["v"].view(Bt, L, H, P)
    o = torch.empty_like(v)
    hl = torch.empty(Bt, H, P, N, dtype=torch.float32, device=dev)
    a = GL.fwd_args(q, k, v, gk, o=o, h_last=hl)
    ws = GL.attach_workspace(a, dev)   # noqa: F841 (kept alive for the calls)
    lib = GL.load_library()
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    ref = ctypes.byref(a)

    def call():
        if lib.samba_gla_fwd(ref, sh) != 0:
            raise RuntimeError("samba_gla_fwd failed")

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ms = _timed(call, steps, stream)
    nbytes = gla_bytes(Bt, L, H, N, P)
    flops = gla_flops(Bt, L, H, N, P)
    gbs = nbytes / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    # roofline of the chunked form: flops / bytes = ~150 flop/B, below the chip's 2.5 PFLOP/s / 8 TB/s = 312
    # flop/B ridge, so the call is bound by HBM on the roofline (its actual limits are the workspace round
    # trip and the per-chunk dependency chain: see the kernel notes)
    return {"workload": "GLA B=%d L=%d, %d heads, keys %d, values %d, bf16 I/O, fp32 state" % (Bt, L, H, N, P),
            "steps": steps, "ms_per_call": ms, "tokens_per_s": Bt * L / (ms * 1e-3),
            "token_columns_per_s": Bt * L * H * P / (ms * 1e-3), "gbs": gbs, "tflops": tflops,
            "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": read_gla_traffic(),
                         "kernel": "gla_prep_kernel<256> + gla_chunk_kernel<bf16,256> (one call, chunked form)",
                         "launch_us": round(ms * 1e3, 2), "algorithmic_bytes_per_launch": nbytes,
                         "algorithmic_flops_per_launch": flops}}


def cpu_baseline_gla(columns: int = 32):
    """The fp64 oracle's GLA on the workload's 4 sequences and 4 heads, `columns` of the 512 value columns,
    in token·columns/s (the GPU figure is token_columns_per_s).  The oracle runs one thread per (sequence,
    head): 16 at most."""
    import numpy as np
    from oracle import oracle as O
    from selective_state_space_05_amd import inputs as I

    wl = I.WORKLOADS[10]
    Bt, L, H, N, P = wl.batch, wl.seqlen, wl.extra["heads"], wl.dstate, wl.extra["head_dim"]
    inp = I.make_gla_inputs_np(10, Bt * L, H, N, P)
    lib = O.load()
    t0 = time.perf_counter()
    O.gla(inp["q_f32"], inp["k_f32"], np.ascontiguousarray(inp["v_f32"][:, :, :columns]), inp["gk_f32"],
          seq_start=np.arange(Bt + 1, dtype=np.int64) * L, lib=lib)
    spent = time.perf_counter() - t0
    return {"value": Bt * L * H * columns / spent, "unit": "token*columns/s",
            "cores": min(O.max_threads(lib), Bt * H), "kind": "oracle",
            "sample": "4 sequences of 4096 tokens, 4 heads, %d of the 512 value columns, fp64 oracle, %.1f s"
                      % (columns, spent)}


def bench_swa(steps: int = 20, warmup: int = 5):
    """The sliding-window attention layer of Samba-3.8B on the training shape: batch 4 x 4096 tokens, 24 heads
    of 128, window 2048, bf16 q/k/v/o.  One layer pass = RoPE of q and k, then the attention."""
    import torch
    from selective_state_space_05_amd import inputs as I
    from selective_state_space_05_amd import swa as W

    wl = I.WORKLOADS[6]
    B, L, H, hd, w = wl.batch, wl.seqlen, wl.extra["heads"], wl.extra["head_dim"], wl.extra["window"]
    dev = torch.device("cuda:0")
    t = I.make_swa_inputs_torch(6, B * L, H, hd, dev)
    q, k, v = (t[n].view(B, L, H, hd) for n in ("q", "k", "v"))
    c, s_ = I.rope_tables(L, hd)
    ct = torch.from_numpy(c.astype("float32")).to(dev)
    st = torch.from_numpy(s_.astype("float32")).to(dev)
    qr, kr = torch.empty_like(q), torch.empty_like(k)
    o = torch.empty_like(q)
    ra = W.rope_args(q, k, ct, st, q_out=qr, k_out=kr)
    fa = W.fwd_args(qr, kr, v, w, o=o)
    lib = W.load_library()
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    rr, fr = ctypes.byref(ra), ctypes.byref(fa)

    def rope():
        if lib.samba_rope(rr, sh) != 0:
            raise RuntimeError("samba_rope failed")

    def att():
        if lib.samba_swa_fwd(fr, sh) != 0:
            raise RuntimeError("samba_swa_fwd failed")

    def layer():
        rope()
        att()

    for _ in range(warmup):
        layer()
    torch.cuda.synchronize()
    ms_layer = _timed(layer, steps, stream)
    ms_att = _timed(att, steps, stream)
    ms_rope = _timed(rope, steps, stream)
    flops = swa_flops(B, L, H, hd, w)
    tf = flops / (ms_att * 1e-3) / 1e12
    return {"workload": "sliding-window attention B=%d L=%d heads=%d head_dim=%d window=%d bf16, RoPE + "
                        "attention (Samba-3.8B layer, training shape)" % (B, L, H, hd, w),
            "steps": steps, "ms_per_layer": ms_layer, "tokens_per_s": B * L / (ms_layer * 1e-3),
            "attention_ms": ms_att, "rope_ms": ms_rope, "tflops": tf,
            "rope_gbs": (4 * B * L * H * hd * 2 + 2 * L * (hd // 2) * 4) / (ms_rope * 1e-3) / 1e9,
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": read_swa_traffic("prefill"),
                         "kernel": "swa_fwd_kernel<bf16> (v_mfma_f32_32x32x16_bf16)", "flops_per_launch": flops,
                         "launch_us": round(ms_att * 1e3, 2),
                         "algorithmic_bytes_per_launch": 4 * B * L * H * hd * 2}}


def bench_swa_decode(steps: int = 200, warmup: int = 20):
    """One decode step of the attention layer for 64 sequences at position 4096 (a full 2048-token window in
    a 2049-slot ring cache): RoPE of the new q and k, then the attention over the cache."""
    import torch
    from selective_state_space_05_amd import inputs as I
    from selective_state_space_05_amd import swa as W

    wl = I.WORKLOADS[7]
    B, H, hd, w, cl, P = (wl.batch, wl.extra["heads"], wl.extra["head_dim"], wl.extra["window"],
                          wl.extra["cache_len"], wl.extra["pos"])
    dev = torch.device("cuda:0")
    t = I.make_swa_inputs_torch(7, B * (cl + 1), H, hd, dev)
    kc = t["k"][:B * cl].view(B, cl, H, hd).permute(0, 2, 1, 3).contiguous()
    vc = t["v"][:B * cl].view(B, cl, H, hd).permute(0, 2, 1, 3).contiguous()
    q, k, v = (t[n][B * cl:].view(B, 1, H, hd) for n in ("q", "k", "v"))
    del t
    c, s_ = I.rope_tables(P + 1, hd)
    ct = torch.from_numpy(c.astype("float32")).to(dev)
    st = torch.from_numpy(s_.astype("float32")).to(dev)
    pos = torch.full((B,), P, dtype=torch.int32, device=dev)
    qr, kr = torch.empty_like(q), torch.empty_like(k)
    o = torch.empty(B, H, hd, dtype=torch.bfloat16, device=dev)
    ra = W.rope_args(q, k, ct, st, q_out=qr, k_out=kr, pos0=pos)
    da = W.decode_args(qr.view(B, H, hd), kr.view(B, H, hd), v.view(B, H, hd), kc, vc, pos, w, o=o)
    lib = W.load_library()
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    rr, dr = ctypes.byref(ra), ctypes.byref(da)

    def att():
        if lib.samba_swa_decode(dr, sh) != 0:
            raise RuntimeError("samba_swa_decode failed")

    def step():
        if lib.samba_rope(rr, sh) != 0:
            raise RuntimeError("samba_rope failed")
        att()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ms_step = _timed(step, steps, stream)
    ms_att = _timed(att, steps, stream)
    nbytes = swa_decode_bytes(B, H, hd, w)
    gbs = nbytes / (ms_att * 1e-3) / 1e9
    return {"workload": "attention decode step: batch %d, heads %d x %d, window %d, ring cache of %d slots, "
                        "position %d, bf16" % (B, H, hd, w, cl, P),
            "steps": steps, "us_per_step": ms_step * 1e3, "steps_per_s": 1e3 / ms_step,
            "attention_us": ms_att * 1e3, "gbs": gbs,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": read_swa_traffic("decode"),
                         "kernel": "swa_decode_kernel<bf16>", "launch_us": round(ms_att * 1e3, 2),
                         "algorithmic_bytes_per_launch": nbytes}}


def cpu_baseline_swa(rows: int = 2048):
    """The fp64 oracle's attention for `rows` query rows of one 4096-token sequence (all 24 heads, full
    2048-token windows), in TFLOP/s of the same algorithmic count."""
    import numpy as np
    from oracle import oracle as O
    from selective_state_space_05_amd import inputs as I

    wl = I.WORKLOADS[6]
    L, H, hd, w = wl.seqlen, wl.extra["heads"], wl.extra["head_dim"], wl.extra["window"]
    inp = I.make_swa_inputs_np(6, L, H, hd)
    c, s_ = I.rope_tables(L, hd)
    sel = np.linspace(w, L - 1, rows).astype(np.int64)
    lib = O.load()
    t0 = time.perf_counter()
    O.swa(inp["q_f32"], inp["k_f32"], inp["v_f32"], w, c, s_, rows=sel, lib=lib)
    spent = time.perf_counter() - t0
    flops = 4.0 * hd * H * rows * (w + 1)
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": O.max_threads(lib), "kind": "oracle",
            "sample": "%d query rows (full windows) of one 4096-token sequence, 24 heads, fp64 oracle with "
                      "RoPE, %.1f s" % (rows, spent)}


def cpu_baseline_swa_decode(seqs: int = 64):
    """The fp64 oracle's decode output (last row of a full window) for `seqs` of the 64 sequences,
    extrapolated to steps/s of the whole batch."""
    import numpy as np
    from oracle import oracle as O
    from selective_state_space_05_amd import inputs as I

    wl = I.WORKLOADS[7]
    B, H, hd, w, P = wl.batch, wl.extra["heads"], wl.extra["head_dim"], wl.extra["window"], wl.extra["pos"]
    c, s_ = I.rope_tables(P + 1, hd)
    lib = O.load()
    spent = 0.0
    for b in range(seqs):
        inp = I.make_swa_inputs_np(700 + b, w + 1, H, hd)
        t0 = time.perf_counter()
        O.swa(inp["q_f32"], inp["k_f32"], inp["v_f32"], w, c[P - w:], s_[P - w:], rows=[w], lib=lib)
        spent += time.perf_counter() - t0
    per_step = spent / seqs * B
    return {"value": 1.0 / per_step, "unit": "steps/s", "cores": O.max_threads(lib), "kind": "oracle",
            "sample": "%d of the 64 sequences' last rows (2049-token windows, 24 heads, fp64 oracle with RoPE), "
                      "extrapolated to the batch; %.2f s" % (seqs, spent)}


# --------------------------------------------------------------------------- #
# measured ALU ceiling (libsamba_probe.so: issue rates of the instruction forms the prefill is made of)
# --------------------------------------------------------------------------- #
PROBE_BLOCKS, PROBE_ITERS = 2048, 2048   # 8 waves per SIMD on 256 CUs, 0.3 to 1 ms per probe launch
# The prefill's algorithmic operations per (token, channel), by the instruction form that executes them:
# two-source multiplies (Δ*A and Δx*B per state, and the 11 other plain ops), fused multiply-adds (state
# update and readout per state), transcendentals (16 exp for Ā, 2 for softplus, 2 for silu).
PREFILL_MUL_PER_TD, PREFILL_FMA_PER_TD = 32 + (VALU_PER_TD - 64), 32


def alu_ceiling():
    """Issue rates measured on this GPU with the library's build flags, and the prefill ceiling they give:
    (t, d)/s = 1 / (n_mul / R_mul + n_fma / R_fma + n_trans / R_exp), R in lane operations per second (the
    faster of the two FMA forms), i.e. perfect issue of exactly the algorithmic operations."""
    import torch
    from selective_state_space_05_amd import probe as PR
    s = torch.cuda.current_stream()
    out = torch.empty(PROBE_BLOCKS * 256, device="cuda:0")
    for _ in range(3):   # settle the clocks
        PR.launch("fmac_vop2", PROBE_BLOCKS, PROBE_ITERS, out, s)
    rates = {}
    for kind in PR.KINDS:
        PR.launch(kind, PROBE_BLOCKS, 64, out, s)
        ms = _timed(lambda: PR.launch(kind, PROBE_BLOCKS, PROBE_ITERS, out, s), 3, s)
        instr = PROBE_BLOCKS * 4 * PROBE_ITERS * PR.instructions_per_round(kind)   # wave-wide instructions
        rates[kind] = {"tlane_ops_per_s": round(instr * 64 / (ms * 1e-3) / 1e12, 2),
                       "cycles_per_wave_instruction_at_2p4ghz": round(1024 * 2.4e9 * ms * 1e-3 / instr, 2)}
    r_mul = rates["mul_vop2"]["tlane_ops_per_s"] * 1e12
    r_fma = max(rates["fmac_vop2"]["tlane_ops_per_s"], rates["fma_vop3"]["tlane_ops_per_s"]) * 1e12
    r_exp = rates["exp"]["tlane_ops_per_s"] * 1e12
    td_s = 1.0 / (PREFILL_MUL_PER_TD / r_mul + PREFILL_FMA_PER_TD / r_fma + TRANS_PER_TD / r_exp)
    per_td = prefill_bytes(16384, 4096) / (16384 * 4096)
    return {"rates": rates, "probe": "%d workgroups x 256 threads, %d rounds of 16 independent instructions "
                                     "per thread (32 for VOP3 fma, 80 for the mix)" % (PROBE_BLOCKS, PROBE_ITERS),
            "prefill_ceiling_td_per_s": td_s, "prefill_ceiling_gbs": td_s * per_td / 1e9,
            "prefill_ceiling_hbm_frac": td_s * per_td / 1e9 / HBM_PEAK_GBS,
            "ops_per_td": {"mul": PREFILL_MUL_PER_TD, "fma": PREFILL_FMA_PER_TD, "trans": TRANS_PER_TD},
            "trans_cost_in_mul_slots": round(r_mul / r_exp, 2),
            "note": "transcendentals and other VALU ops measured not to overlap (the 4:1 mix costs the sum)"}


VALU_COUNTER_FILE = ROOT / "profiles" / "valu_counters_prefill.json"


def read_valu_counters():
    """Executed VALU / transcendental instructions per (token, channel) of the long-prompt prefill kernel from
    the committed counter run, if it was taken on this kernel source."""
    try:
        t = json.loads(VALU_COUNTER_FILE.read_text())
    except Exception:
        return None
    if t.get("kernel_source_sha256_16") != kernel_hash():
        return None
    return t.get("forward")


# --------------------------------------------------------------------------- #
# the other prefill configurations, complexity checks, decode over many states
# --------------------------------------------------------------------------- #
def _prefill_leg(name, launch_args, td, nbytes, steps, warmup, plan):
    """Time calls cycling over `launch_args` (one FwdArgs per input set); roofline against the VALU slot
    peak, GB/s against HBM."""
    import torch
    from selective_state_space_05_amd import scan as S
    lib = S.load_library()
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    refs = [ctypes.byref(a) for a in launch_args]

    def call(i=[0]):
        st = lib.samba_scan_fwd(refs[i[0] % len(refs)], sh)
        i[0] += 1
        if st != 0:
            raise S.SambaError(st, "samba_scan_fwd")

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ms = _timed(call, steps, stream)
    slots = SLOTS_PER_TD * td / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": name, "steps": steps, "ms_per_call": ms, "gbs": gbs, "tokens_channels_per_s": td / (ms * 1e-3),
            "hbm_frac": gbs / HBM_PEAK_GBS, "input_sets": len(refs),
            "plan": {"time_slices": plan[0], "workgroups": plan[1], "threads_per_workgroup": plan[2],
                     "lanes_per_channel": plan[3]},
            "roofline": {"bound": "alu", "achieved": round(slots, 3), "peak": round(VALU_PEAK_TSLOT, 2),
                         "unit": "Tslot/s", "frac": round(slots / VALU_PEAK_TSLOT, 4), "traffic": None,
                         "kernel": kernel_name({"time_slices": plan[0], "lanes_per_channel": plan[3]}),
                         "algorithmic_bytes_per_launch": nbytes}}


def bench_cfg1(steps: int = 40, warmup: int = 8, sets: int = 4):
    """B1 L4096 D2048, bf16 I/O, y and h_last out.  One call's 67.6 MB fits the 256 MB last-level cache,
    so the calls cycle over `sets` distinct input sets (270 MB together) and each call reads from HBM."""
    import torch
    from selective_state_space_05_amd import inputs as I
    from selective_state_space_05_amd import scan as S
    W = I.WORKLOADS[1]
    L, D = W.seqlen, W.dim
    dev = torch.device("cuda:0")
    args, keep = [], []
    for k in range(sets):
        inp = I.make_fwd_inputs_torch(1, L, D, dev, tensor_offset=k)
        y = torch.empty(1, L, D, dtype=torch.bfloat16, device=dev)
        hl = torch.empty(1, D, 16, device=dev)
        keep.append((inp, y, hl))
        args.append(S.fwd_args(*(inp[n].view(1, L, -1) for n in ("x", "dt", "z", "B", "C")), inp["A"], inp["D"],
                               inp["dt_bias"], y=y, h_last=hl))
    inp, y, hl = keep[0]
    plan = S.fwd_plan(*(inp[n].view(1, L, -1) for n in ("x", "dt", "z", "B", "C")), inp["A"], inp["D"], inp["dt_bias"],
                      y=y, h_last=hl)
    return _prefill_leg("prefill B1 L4096 D2048 N16 bf16 (y and h_last out)", args, L * D,
                        prefill_bytes(L, D, h0=False), steps, warmup, plan)


def bench_cfg2(steps: int = 10, warmup: int = 3):
    """Packed variable-length stream: T = 32768 tokens of lengths U(512, 4096), D 4096, bf16, state reset at
    every sequence start (no h0), one h_last row per sequence."""
    import torch
    from selective_state_space_05_amd import inputs as I
    from selective_state_space_05_amd import scan as S
    W = I.WORKLOADS[2]
    T, D = W.varlen_total, W.dim
    dev = torch.device("cuda:0")
    lens = I.varlen_lengths(2, T)
    cu = torch.from_numpy(I.cu_from_lengths(lens)).to(dev)
    inp = I.make_fwd_inputs_torch(2, T, D, dev)
    y = torch.empty(T, D, dtype=torch.bfloat16, device=dev)
    hl = torch.empty(len(lens), D, 16, device=dev)
    ins = [inp[n] for n in ("x", "dt", "z", "B", "C", "A", "D", "dt_bias")]
    a = S.fwd_args(*ins, y=y, h_last=hl, cu_seqlens=cu)
    plan = S.fwd_plan(*ins, y=y, h_last=hl, cu_seqlens=cu)
    nbytes = prefill_bytes(T, D, h0=False, h_last=False) + len(lens) * D * 16 * 4
    out = _prefill_leg("prefill packed T=32768 (%d sequences of 512..4096) D4096 N16 bf16, resets at sequence "
                       "starts" % len(lens), [a], T * D, nbytes, steps, warmup, plan)
    out["sequences"] = int(len(lens))
    return out


def bench_complexity():
    """Linear time in L (prefill, one sequence, D 4096, L = 4K / 16K / 64K) and constant time per decode
    step (B64 D4096: the same steps after a 0-token and after a 2048-token prefill)."""
    import torch
    from selective_state_space_05_amd import inputs as I
    from selective_state_space_05_amd import scan as S
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    D = 4096
    pre = {}
    for L in (4096, 16384, 65536):
        inp = I.make_fwd_inputs_torch(3, L, D, dev)
        y = torch.empty(1, L, D, dtype=torch.bfloat16, device=dev)
        ins = [inp[n].view(1, L, -1) for n in ("x", "dt", "z", "B", "C")] + [inp["A"], inp["D"], inp["dt_bias"]]
        call = lambda: S.scan_fwd(*ins, y=y, return_last_state=False)
        for _ in range(2):
            call()
        torch.cuda.synchronize()
        ms = _timed(call, 5, stream)
        pre[L] = {"us_per_call": ms * 1e3, "ns_per_token": ms * 1e6 / L,
                  "plan": S.fwd_plan(*ins, y=y)}
        del inp, y, ins
    ref = pre[16384]["ns_per_token"]
    for L in pre:
        pre[L]["per_token_vs_16k"] = pre[L]["ns_per_token"] / ref
    Bt = 64
    W = I.WORKLOADS[4]
    p = I.make_fwd_inputs_torch(4, Bt * W.seqlen, D, dev)
    A, Dv, bias = p["A"], p["D"], p["dt_bias"]
    _, st2048 = S.scan_fwd(*(p[n].view(Bt, W.seqlen, -1) for n in ("x", "dt", "z", "B", "C")), A, Dv, bias)
    del p
    rg = I.make_step_ring_torch(4, 16, Bt, D, dev)
    ys = torch.empty(Bt, D, dtype=torch.bfloat16, device=dev)
    dec = {}
    for name, st in (("after_0_tokens", torch.zeros(Bt, D, 16, device=dev)), ("after_2048_tokens", st2048)):
        i = [0]

        def step():
            r = i[0] % 16
            i[0] += 1
            S.scan_step(st, rg["x"][r], rg["dt"][r], rg["z"][r], rg["B"][r], rg["C"][r], A, Dv, bias, y=ys)

        for _ in range(32):
            step()
        torch.cuda.synchronize()
        dec[name] = {"us_per_step": _timed(step, 400, stream) * 1e3}
    dec["ratio"] = dec["after_2048_tokens"]["us_per_step"] / dec["after_0_tokens"]["us_per_step"]
    return {"prefill_time_vs_L": {str(k): v for k, v in pre.items()}, "decode_step_vs_prior_tokens": dec,
            "note": "per-token prefill time flat in L means linear time; decode step time independent of the "
                    "tokens already consumed means a constant-size state (page 1, 推理效率)"}


def bench_decode_states(nstates: int = 24, rounds: int = 100):
    """Decode over `nstates` independent batch-64 states (16 MiB each, 384 MiB together, more than the
    256 MB last-level cache), step k on state k % nstates, as one token through a stack of layers: every
    step's state comes from HBM, unlike the single in-place state of the streaming-decode leg."""
    import torch
    from selective_state_space_05_amd import inputs as I
    from selective_state_space_05_amd import scan as S
    dev = torch.device("cuda:0")
    Bt, D = 64, 4096
    p = I.make_params(4, D)
    A, Dv, bias = (torch.from_numpy(p[k]).to(dev) for k in ("A", "D", "dt_bias"))
    states = [torch.zeros(Bt, D, 16, device=dev) for _ in range(nstates)]
    rg = I.make_step_ring_torch(4, nstates, Bt, D, dev)
    ys = torch.empty(nstates, Bt, D, dtype=torch.bfloat16, device=dev)
    lib = S.load_library()
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    args = [S.step_args(states[k], rg["x"][k], rg["dt"][k], rg["z"][k], rg["B"][k], rg["C"][k], A, Dv, bias,
                        y=ys[k]) for k in range(nstates)]
    refs = [ctypes.byref(a) for a in args]

    def one_round():
        for r in refs:
            if lib.samba_scan_step(r, sh) != 0:
                raise RuntimeError("samba_scan_step failed")

    for _ in range(3):
        one_round()
    torch.cuda.synchronize()
    us = _timed(one_round, rounds, stream) * 1e3 / nstates
    gbs = decode_bytes(Bt, D) / (us * 1e-6) / 1e9

    # reference at the same size: a device copy of each 16 MiB state into a second ring of 24 (16 MiB read
    # from HBM and 16 MiB written per copy, as a step reads and writes its state), timed the same way
    dst = [torch.empty_like(t) for t in states]

    def copy_round():
        for k in range(nstates):
            dst[k].copy_(states[k])

    for _ in range(3):
        copy_round()
    torch.cuda.synchronize()
    copy_us = _timed(copy_round, rounds, stream) * 1e3 / nstates
    copy_gbs = 2 * states[0].numel() * 4 / (copy_us * 1e-6) / 1e9
    del dst
    return {"states": nstates, "state_mib_total": nstates * Bt * D * 16 * 4 / 2 ** 20, "us_per_step": us,
            "steps_per_s": 1e6 / us, "gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "same_size_copy": {"us": copy_us, "gbs": copy_gbs,
                               "note": "device copy of one 16 MiB state into another buffer, rotating over "
                                       "%d states like the steps" % nstates},
            "frac_of_same_size_copy": gbs / copy_gbs,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                         "kernel": "scan_step_kernel<bf16,bf16>"}}


def cpu_baseline_cfg1():
    """The oracle on the whole B1 L4096 D2048 call (all host cores)."""
    from oracle import oracle as O
    from selective_state_space_05_amd import inputs as I
    W = I.WORKLOADS[1]
    L, D = W.seqlen, W.dim
    lib = O.load()
    inp = I.make_fwd_inputs_torch(1, L, D, "cpu")
    P = I.make_params(1, D)
    arr = [inp[k].double().numpy() for k in ("x", "dt", "z", "B", "C")]
    t0 = time.perf_counter()
    O.scan_fwd(*arr, P["A"], P["D"], P["dt_bias"], lib=lib)
    dt_s = time.perf_counter() - t0
    return {"value": prefill_bytes(L, D, h0=False) / dt_s / 1e9, "unit": "GB/s", "cores": O.max_threads(lib),
            "kind": "oracle", "tokens_channels_per_s": L * D / dt_s,
            "sample": "the whole call (4096 tokens x 2048 channels), %.2f s" % dt_s}


def cpu_baseline_cfg2(channels: int = 512):
    """The oracle on every sequence of the packed stream, over `channels` of the 4096 channels (rate per
    (token, channel) extrapolates to the whole)."""
    import numpy as np
    from oracle import oracle as O
    from selective_state_space_05_amd import inputs as I
    W = I.WORKLOADS[2]
    T, D = W.varlen_total, W.dim
    lib = O.load()
    lens = I.varlen_lengths(2, T)
    ss = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    inp = I.make_fwd_inputs_torch(2, T, D, "cpu")
    P = I.make_params(2, D)
    x, dt, z = (inp[k][:, :channels].double().numpy().copy() for k in ("x", "dt", "z"))
    Bm, Cm = (inp[k].double().numpy() for k in ("B", "C"))
    t0 = time.perf_counter()
    O.scan_fwd(x, dt, z, Bm, Cm, P["A"][:channels], P["D"][:channels], P["dt_bias"][:channels], seq_start=ss, lib=lib)
    dt_s = time.perf_counter() - t0
    td_s = T * channels / dt_s
    per_td = (prefill_bytes(T, D, h0=False, h_last=False) + len(lens) * D * 64) / (T * D)
    return {"value": td_s * per_td / 1e9, "unit": "GB/s", "cores": O.max_threads(lib), "kind": "oracle",
            "tokens_channels_per_s": td_s,
            "sample": "all %d sequences (32768 tokens), %d of 4096 channels, %.2f s" % (len(lens), channels, dt_s)}


PMC_RUN = ("python3 <repo>/bench.py --steps 1 --warmup 0 --decode-steps 256 --no-cpu --bwd-steps 1 "
           "--proj-steps 1 --copy-probe")


def pmc_summary(fetch_dir: str, write_dir: str, out: str):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; CSV output) of PMC_RUN into the per-launch HBM
    byte summary bench.py reports as `traffic`: the prefill kernel, the decode step, the three kernels of
    one backward call, and the projection GEMM.

    Each counter is scaled by what it reads for the plain 512 MiB copy of the same run (expected 512 MiB
    fetched and 512 MiB written per dispatch); values are the median over each kernel's dispatches."""
    import csv
    import glob
    import statistics

    def per_kernel(d, counter):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
        vals = {}
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    def pick(vals, *parts):
        keys = [k for k in vals if all(p in k for p in parts)]
        assert len(keys) == 1, (parts, keys)
        return keys[0]

    # (the inference launches run the copy instantiated with kNoCkpt: names end in "false, true>"; the
    # checkpoint pass is the kCkpt variant: "true, false>")
    sel = {"fwd": ("scan_fwd_kernel", "16, 1, 8, false, true>"),
           "step": ("scan_step_kernel<unsigned short, unsigned short",),
           "cfg1": ("scan_split8_kernel<unsigned short, unsigned short, 16>",),
           "cfg2": ("scan_fwd_kernel", "unsigned short, 1, 4, 16, false, true>"),
           "ckpt": ("scan_fwd_kernel", ", true, false>"), "bwd": ("scan_bwd_kernel<",), "finish": ("scan_bwd_finish_kernel",),
           "proj": ("proj_dma_kernel<unsigned short",)}
    got = {k: {} for k in sel}
    scales = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = per_kernel(d, counter)
        copy = [v for k, vs in vals.items() if "copyBuffer" in k for v in vs]
        # the 512 MiB probe: the smallest of the large copies (a run may also hold small copies)
        big = min(v for v in copy if v > 0.25 * max(copy))
        scale = (512 << 20) / 1024.0 / big
        scales[counter] = {"copy_raw_kib_per_dispatch": big, "scale": scale}
        for name, parts in sel.items():
            key = pick(vals, *parts)
            kib = statistics.median(vals[key])
            got[name][counter] = {"kernel": key[:120], "raw_kib_per_dispatch": kib, "bytes": kib * scale * 1024.0}

    def entry(name, algorithmic):
        f, w = got[name]["FETCH_SIZE"]["bytes"], got[name]["WRITE_SIZE"]["bytes"]
        return {"kernel": got[name]["FETCH_SIZE"]["kernel"], "fetch_bytes": f, "write_bytes": w,
                "bytes_per_launch": f + w, "algorithmic_bytes_per_launch": algorithmic}

    out_d = {"kernel_source_sha256_16": kernel_hash(), "unit": "bytes per launch", "calibration": scales,
             "forward": entry("fwd", prefill_bytes(16384, 4096)),
             "decode_step": entry("step", decode_bytes(64, 4096)),
             "backward": {"kernels": {n: entry(n, None) for n in ("ckpt", "bwd", "finish")},
                          "algorithmic_bytes_per_call": bwd_bytes(4 * 4096, 4096, 4)},
             "projections": entry("proj", (16384 * 4096 + 4128 * 4096 + 16384 * 4128) * 2),
             "cfg1": entry("cfg1", prefill_bytes(4096, 2048, h0=False)),
             "cfg2": entry("cfg2", None)}
    out_d["backward"]["bytes_per_call"] = sum(v["bytes_per_launch"] for v in out_d["backward"]["kernels"].values())
    out_d["command"] = [
        f"cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d <repo>/{fetch_dir} -o p -- {PMC_RUN}",
        f"cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d <repo>/{write_dir} -o p -- {PMC_RUN}",
        f"python bench.py --pmc-summary {fetch_dir} {write_dir} {out}",
    ]
    out_d["note"] = ("FETCH_SIZE and WRITE_SIZE are KiB per dispatch (median over each kernel's dispatches), each "
                     "scaled by the ratio of the known size of the plain 512 MiB device copy in the same run to what "
                     "the counter reports for it (FETCH_SIZE reads half, WRITE_SIZE exact).")
    Path(out).write_text(json.dumps(out_d, indent=1) + "\n")
    print(json.dumps(out_d))


SWA_PMC_RUN = "python3 <repo>/bench.py --swa-only --swa-steps 2 --swa-decode-steps 2 --warmup 1 --copy-probe"
GROUPS_PMC_RUN = "python3 <repo>/bench.py --groups-only --groups-steps 2 --warmup 1 --copy-probe"
SSD_PMC_RUN = "python3 <repo>/bench.py --ssd-only --ssd-steps 2 --warmup 1 --copy-probe"
RETENTION_PMC_RUN = "python3 <repo>/bench.py --retention-only --ssd-steps 2 --warmup 1 --copy-probe"
GLA_PMC_RUN = "python3 <repo>/bench.py --gla-only --gla-steps 2 --warmup 1 --copy-probe"  # 2 + 1 prefill calls, 220 steps


VALU_PMC_RUN = ("python3 <repo>/bench.py --steps 1 --warmup 0 --no-decode --no-cpu --no-bwd --no-proj --no-swa "
                "--no-groups --no-ssd --no-gla --no-cfg --no-alu --copy-probe")
VALU_PASSES = ("SQ_WAVES SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 SQ_ACTIVE_INST_VALU SQ_WAVE_CYCLES SQ_INSTS_LDS "
               "SQ_INSTS_SALU SQ_BUSY_CYCLES",
               "SQ_WAIT_INST_ANY SQ_WAIT_ANY SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_LDS SQ_WAIT_INST_LDS "
               "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_ACTIVE_INST_VALU2")


def valu_summary(dir_a: str, dir_b: str, out: str):
    """Turn the two SQ counter passes (VALU_PASSES, each a rocprofv3 --pmc run of VALU_RUN) into per
    (token, channel) executed instruction counts of the long-prompt prefill kernel and its wave-time split.
    Values are medians over that kernel's dispatches; instruction counts are wave-wide (x 64 lanes)."""
    import csv
    import glob
    import statistics

    vals = {}
    for d in (dir_a, dir_b):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
        per = {}
        for r in csv.DictReader(open(f)):
            k = r["Kernel_Name"]
            if "scan_fwd_kernel" in k and "16, 1, 8, false, true>" in k:
                per.setdefault((r["Dispatch_Id"], r["Counter_Name"]), 0.0)
                per[(r["Dispatch_Id"], r["Counter_Name"])] += float(r["Counter_Value"])
                kernel = k
        for (disp, c), v in per.items():
            vals.setdefault(c, []).append(v)
    med = {c: statistics.median(v) for c, v in vals.items()}
    td = 16384 * 4096
    valu = med["SQ_INSTS_VALU"] * 64 / td
    trans = med["SQ_INSTS_VALU_TRANS_F32"] * 64 / td
    wc = med["SQ_WAVE_CYCLES"]
    fw = {"forward": {
        "kernel": kernel[:120], "dispatches": len(vals["SQ_INSTS_VALU"]), "tokens_channels_per_launch": td,
        "valu_lane_ops_per_td": round(valu, 2), "trans_lane_ops_per_td": round(trans, 2),
        "executed_slots_per_td": round(valu - trans + TRANS_SLOTS * trans, 1),
        "algorithmic_slots_per_td": SLOTS_PER_TD,
        "lds_wave_instructions_per_td": round(med["SQ_INSTS_LDS"] / td, 4),
        "salu_wave_instructions_per_td": round(med["SQ_INSTS_SALU"] / td, 4),
        "wave_time": {"waiting_on_dependencies": round(med["SQ_WAIT_ANY"] / wc, 3),
                      "issuing": round(med["SQ_ACTIVE_INST_ANY"] / wc, 3),
                      "waiting_for_issue": round(med["SQ_WAIT_INST_ANY"] / wc, 3),
                      "valu_active": round(med["SQ_ACTIVE_INST_VALU"] / wc, 3)},
        "lds_bank_conflict_cycles_over_lds_active": round(med["SQ_LDS_BANK_CONFLICT"] / max(med["SQ_LDS_IDX_ACTIVE"], 1.0),
                                                          4),
        "raw_medians": med}}
    out_d = {"kernel_source_sha256_16": kernel_hash(), **fw}
    out_d["command"] = [
        f"cd /tmp && rocprofv3 --pmc {VALU_PASSES[0]} --output-format csv -d <repo>/{dir_a} -o p -- {VALU_PMC_RUN}",
        f"cd /tmp && rocprofv3 --pmc {VALU_PASSES[1]} --output-format csv -d <repo>/{dir_b} -o p -- {VALU_PMC_RUN}",
        f"python bench.py --valu-summary {dir_a} {dir_b} {out}"]
    out_d["note"] = ("SQ_INSTS_VALU counts every VALU instruction (transcendentals included); executed slots count a "
                     "transcendental as %d, as the algorithmic count does. wave_time fractions are the SQ wave-cycle "
                     "counters over SQ_WAVE_CYCLES (quad-cycle units cancel)." % TRANS_SLOTS)
    Path(out).write_text(json.dumps(out_d, indent=1) + "\n")
    print(json.dumps(out_d))


def _counter_summary(fetch_dir: str, write_dir: str, out: str, which: str):
    """HBM bytes per launch of the attention kernels (which = "swa"), the grouped prefill ("groups"), the SSD
    prefill ("ssd") or gated linear attention ("gla") from
    two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE), each calibrated by the 512 MiB copy of the same run (as
    pmc_summary does for the scan)."""
    import csv
    import glob
    import statistics

    def per_kernel(d, counter):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
        vals = {}
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                vals.setdefault((r["Kernel_Name"], int(r.get("Grid_Size", r.get("Grid_Size_X", 0)) or 0)),
                                []).append(float(r["Counter_Value"]))
        return vals

    def pick(vals, part):
        parts = part if isinstance(part, tuple) else (part,)   # every piece must be in the kernel's name
        keys = [k for k in vals if all(q in k[0] for q in parts)]
        assert keys, part
        return sorted(keys, key=lambda k: k[1])[-1]   # the largest launch of that kernel

    from selective_state_space_05_amd import inputs as I
    if which == "swa":
        wl6, wl7 = I.WORKLOADS[6], I.WORKLOADS[7]
        B, L, H, hd, w = wl6.batch, wl6.seqlen, wl6.extra["heads"], wl6.extra["head_dim"], wl6.extra["window"]
        Bd, Hd, hdd, wd = wl7.batch, wl7.extra["heads"], wl7.extra["head_dim"], wl7.extra["window"]
        sel = {"prefill": ("swa_fwd_kernel<unsigned short>", 4 * B * L * H * hd * 2),
               "rope_prefill": ("rope_kernel<true, true>", 4 * B * L * H * hd * 2 + L * hd * 4),
               "decode": ("swa_decode_kernel<unsigned short>", swa_decode_bytes(Bd, Hd, hdd, wd))}
        src_hash, run, flag = swa_hash(), SWA_PMC_RUN, "--pmc-summary-swa"
        note = ("Algorithmic bytes: prefill q, k, v read once and o written once (the window's re-reads of K and V "
                "are meant to hit L2); RoPE q, k read and written plus the tables; decode the window's cached K "
                "and V, the new q, k, v, the cache write and o.")
    elif which == "gla":
        wl = I.WORKLOADS[10]
        Bt, L, H, N, P = wl.batch, wl.seqlen, wl.extra["heads"], wl.dstate, wl.extra["head_dim"]
        T = Bt * L
        sel = {"gla_prep": ("gla_prep_kernel<256>", T * H * 3 * N * 2),
               "gla_chunk": ("gla_chunk_kernel<unsigned short, 256>", gla_bytes(Bt, L, H, N, P) - T * H * 3 * N * 2)}
        src_hash, run, flag = gla_hash(), GLA_PMC_RUN, "--pmc-summary-gla"
        note = ("Algorithmic bytes: q, k, gk (the prep kernel) and v read and o written once (bf16), h_last out "
                "(the chunk kernel). The workspace the prep kernel writes and the chunk kernel reads (145 KiB per "
                "(chunk, head), 152 MB here) is not counted in the algorithmic bytes.")
    elif which == "ssd":
        wl = I.WORKLOADS[9]
        Bt, L, H, P, N, G = (wl.batch, wl.seqlen, wl.extra["heads"], wl.extra["head_dim"], wl.dstate,
                             wl.extra["ngroups"])
        # (the default form: C B^T inside the prefill kernel, the last template argument)
        sel = {"ssd": ("ssd_fwd_kernel<unsigned short, 128, true, false, true>", ssd_bytes(Bt, L, H, P, G, N))}
        src_hash, run, flag = ssd_hash(), SSD_PMC_RUN, "--pmc-summary-ssd"
        note = ("Algorithmic bytes: x, z read and y written once (bf16), dt, B and C once, parameters, h_last "
                "out. C B^T is formed inside the prefill kernel (no workspace).")
    elif which == "retention":
        wl = I.WORKLOADS[11]
        Bt, L, H, P, N, G = (wl.batch, wl.seqlen, wl.extra["heads"], wl.extra["head_dim"], wl.dstate,
                             wl.extra["ngroups"])
        # the retention leg runs the unsplit or split prefill depending on the CU count: match either, in the
        # default form (C B^T inside the prefill kernel: the last template argument)
        sel = {"ssd": (("ssd_fwd_kernel<unsigned short, 128, false, ", ", true>("),
                       ssd_bytes(Bt, L, H, P, G, N, gated=False))}
        src_hash, run, flag = ssd_hash(), RETENTION_PMC_RUN, "--pmc-summary-retention"
        note = ("Algorithmic bytes: B, C (k, q) and x (v) read and y written once (bf16), parameters, h_last out. "
                "C B^T is formed inside the prefill kernel: one launch per call, no workspace.")
    else:
        wl = I.WORKLOADS[8]
        Bt, L, D, N, G = wl.batch, wl.seqlen, wl.dim, wl.dstate, wl.extra["ngroups"]
        sel = {"groups": ("scan_groups_kernel<unsigned short, unsigned short, 64>", groups_bytes(Bt, L, D, G, N)),
               "decode": ("step_groups_kernel<unsigned short, unsigned short, 64>",
                          64 * D * N * 8 + 64 * D * 8 + 64 * G * N * 4 + D * N * 4 + D * 8)}
        src_hash, run, flag = groups_hash(), GROUPS_PMC_RUN, "--pmc-summary-groups"
        note = ("Algorithmic bytes: prefill x, dt, z read and y written once (bf16), B and C once, parameters, "
                "h_last out; decode step the state read and written, x, dt, z in and y out, B, C, parameters.")
    got = {k: {} for k in sel}
    scales = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = per_kernel(d, counter)
        copy = [v for k, vs in vals.items() if "copyBuffer" in k[0] for v in vs]
        big = min(v for v in copy if v > 0.25 * max(copy))
        scale = (512 << 20) / 1024.0 / big
        scales[counter] = {"copy_raw_kib_per_dispatch": big, "scale": scale}
        for name, (part, _) in sel.items():
            key = pick(vals, part)
            kib = statistics.median(vals[key])
            got[name][counter] = {"kernel": key[0][:120], "grid": key[1], "raw_kib_per_dispatch": kib,
                                  "bytes": kib * scale * 1024.0}
    out_d = {"kernel_source_sha256_16": src_hash, "unit": "bytes per launch", "calibration": scales}
    for name, (_, algorithmic) in sel.items():
        f, wr = got[name]["FETCH_SIZE"]["bytes"], got[name]["WRITE_SIZE"]["bytes"]
        out_d[name] = {"kernel": got[name]["FETCH_SIZE"]["kernel"], "grid": got[name]["FETCH_SIZE"]["grid"],
                       "fetch_bytes": f, "write_bytes": wr, "bytes_per_launch": f + wr,
                       "algorithmic_bytes_per_launch": algorithmic}
    if which in ("gla", "retention"):
        out_d[which + "_call"] = {"bytes_per_call": sum(out_d[k]["bytes_per_launch"] for k in sel),
                                  "algorithmic_bytes_per_call": sum(out_d[k]["algorithmic_bytes_per_launch"]
                                                                    for k in sel)}
    out_d["command"] = [
        f"cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d <repo>/{fetch_dir} -o p -- {run}",
        f"cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d <repo>/{write_dir} -o p -- {run}",
        f"python bench.py {flag} {fetch_dir} {write_dir} {out}",
    ]
    out_d["note"] = note
    Path(out).write_text(json.dumps(out_d, indent=1) + "\n")
    print(json.dumps(out_d))


def kernel_name(plan) -> str:
    """The prefill kernel a launch plan runs (bf16 in, bf16 out)."""
    if plan["lanes_per_channel"] == 8:
        return "scan_split8_kernel<bf16,bf16,W=%d> (8 lanes per channel)" % plan["time_slices"]
    return "scan_fwd_kernel<bf16,bf16,W=%d> (4 lanes per channel)" % plan["time_slices"]


def copy_ceiling(nbytes: int = 1 << 30, reps: int = 10) -> float:
    """Measured device-to-device copy rate (bytes read + bytes written per second, GB/s): the practical HBM
    ceiling the algorithmic rates are also compared with."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        b.copy_(a)
    e1.record(stream)
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return gbs


def copy_probe(nbytes: int = 512 << 20, reps: int = 3):
    """A plain device-to-device copy of known size; its FETCH_SIZE / WRITE_SIZE per dispatch calibrate the counters."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").uniform_()
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(max_oracle_s: float = 30.0):
    """The fp64 oracle on the same long-prompt workload: the 8 chained 16384-token
    calls (h0 -> h_last carried between calls) over all 4096 channels, with
    seeded CPU-generated inputs of the same distribution.  Only the oracle calls
    are timed; if they would exceed ~max_oracle_s the run stops after the calls
    done so far and the sample says how many."""
    import numpy as np
    from oracle import oracle as O
    from selective_state_space_05_amd import inputs as I

    W = I.WORKLOADS[3]
    cl, D, n = W.seqlen // W.chunks, W.dim, W.chunks
    P = I.make_params(3, D)
    lib = O.load()
    cores = O.max_threads(lib)
    h = np.zeros((1, D, 16))
    spent, done = 0.0, 0
    for i in range(n):
        inp = I.make_fwd_inputs_torch(3, cl, D, "cpu", tensor_offset=i)
        x, dt, z, Bm, Cm = (inp[k].double().numpy() for k in ("x", "dt", "z", "B", "C"))
        t0 = time.perf_counter()
        _, h = O.scan_fwd(x, dt, z, Bm, Cm, P["A"], P["D"], P["dt_bias"], h0=h, lib=lib)
        spent += time.perf_counter() - t0
        done += 1
        del x, dt, z, Bm, Cm, inp
        if spent * (done + 1) / done > max_oracle_s:
            break
    gbs = done * prefill_bytes(cl, D) / spent / 1e9
    # the same oracle on one core, over the first call's first 256 channels
    inp = I.make_fwd_inputs_torch(3, cl, D, "cpu", tensor_offset=0)
    c1 = 256
    x, dt, z = (inp[k][:, :c1].double().numpy().copy() for k in ("x", "dt", "z"))
    Bm, Cm = (inp[k].double().numpy() for k in ("B", "C"))
    t0 = time.perf_counter()
    O.scan_fwd(x, dt, z, Bm, Cm, P["A"][:c1], P["D"][:c1], P["dt_bias"][:c1], nthreads=1, lib=lib)
    one = time.perf_counter() - t0
    return {"value": gbs, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": "%d of the 8 chained 16384-token calls of the 131072-token prompt, all 4096 channels, "
                      "fp64 oracle (OpenMP over channels), %.1f s of oracle time" % (done, spent),
            "tokens_channels_per_s": done * cl * D / spent,
            "one_core": {"tokens_channels_per_s": cl * c1 / one,
                         "sample": "first 16384-token call, 256 channels, 1 thread, %.2f s" % one},
            "nproc": os.cpu_count(), "cpu_model": _cpu_model()}


def cpu_baseline_backward(max_oracle_s: float = 30.0):
    """The fp64 oracle's gradients on the same training-shape backward (all 4 sequences, all channels)."""
    import numpy as np
    from oracle import oracle as O
    from selective_state_space_05_amd import inputs as I

    W = I.WORKLOADS[5]
    Bt, L, D = W.batch, W.seqlen, W.dim
    P = I.make_params(5, D)
    lib = O.load()
    inp = I.make_fwd_inputs_torch(5, Bt * L, D, "cpu")
    ex = I.make_bwd_extra_torch(5, Bt * L, D, Bt, "cpu")
    arrs = [inp[k].double().numpy() for k in ("x", "dt", "z", "B", "C")]
    dy = ex["dy"].double().numpy()
    ss = np.arange(Bt + 1, dtype=np.int64) * L
    # one sequence first: stop there if the whole would exceed the time budget
    t0 = time.perf_counter()
    O.scan_bwd(*(a[:L] for a in arrs), P["A"], P["D"], P["dt_bias"], dy[:L], seq_start=ss[:2], lib=lib)
    one = time.perf_counter() - t0
    if one * Bt <= max_oracle_s:
        t0 = time.perf_counter()
        O.scan_bwd(*arrs, P["A"], P["D"], P["dt_bias"], dy, seq_start=ss, lib=lib)
        spent, nseq = time.perf_counter() - t0, Bt
    else:
        spent, nseq = one, 1
    return {"value": nseq * L * D / spent, "unit": "tokens*channels/s", "cores": O.max_threads(lib),
            "kind": "oracle", "sample": "%d of the 4 sequences (4096 tokens, all 4096 channels), fp64 oracle "
                                        "gradients, %.1f s" % (nseq, spent)}


def cpu_baseline_decode(steps: int = 1024, max_oracle_s: float = 15.0):
    """The fp64 oracle's decode step on the full batch-64, D-4096 state, chained over the first `steps`
    steps of the input ring (stopping early past ~max_oracle_s); steps/s is extrapolated from that sample."""
    import numpy as np
    from oracle import oracle as O
    from selective_state_space_05_amd import inputs as I

    W = I.WORKLOADS[4]
    Bt, D, R = W.batch, W.dim, W.decode_ring
    P = I.make_params(4, D)
    lib = O.load()
    state = np.zeros((Bt, D, 16))
    ring = [I.make_step_inputs_np(4, r, Bt, D) for r in range(min(R, 16))]
    spent, done = 0.0, 0
    for k in range(steps):
        s = ring[k % len(ring)]
        t0 = time.perf_counter()
        _, state = O.scan_step(state, s["x_f32"], s["dt_f32"], s["z_f32"], s["B_f32"], s["C_f32"], P["A"], P["D"],
                               P["dt_bias"], lib=lib)
        spent += time.perf_counter() - t0
        done += 1
        if spent > max_oracle_s:
            break
    return {"value": done / spent, "unit": "steps/s", "cores": O.max_threads(lib), "kind": "oracle",
            "sample": "first %d of the 65536 steps (batch 64, D 4096, fp64 state), extrapolated to steps/s; "
                      "%.1f s of oracle time" % (done, spent)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=65536)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward leg")
    ap.add_argument("--bwd-steps", type=int, default=10)
    ap.add_argument("--no-proj", action="store_true", help="skip the selection-projection leg")
    ap.add_argument("--proj-steps", type=int, default=20)
    ap.add_argument("--no-swa", action="store_true", help="skip the sliding-window attention legs")
    ap.add_argument("--swa-steps", type=int, default=20)
    ap.add_argument("--swa-decode-steps", type=int, default=200)
    ap.add_argument("--no-groups", action="store_true", help="skip the grouped-prefill leg")
    ap.add_argument("--groups-steps", type=int, default=10)
    ap.add_argument("--groups-only", action="store_true", help="run only the grouped-prefill leg")
    ap.add_argument("--no-ssd", action="store_true", help="skip the state-space duality leg")
    ap.add_argument("--ssd-steps", type=int, default=20)
    ap.add_argument("--ssd-only", action="store_true", help="run only the state-space duality leg")
    ap.add_argument("--retention-only", action="store_true",
                    help="run only the multi-scale retention leg (the duality entry point)")
    ap.add_argument("--no-gla", action="store_true", help="skip the gated linear attention leg")
    ap.add_argument("--gla-steps", type=int, default=5)
    ap.add_argument("--gla-only", action="store_true", help="run only the gated linear attention leg")
    ap.add_argument("--swa-only", action="store_true",
                    help="run only the attention legs (and the copy probe with --copy-probe): counter runs")
    ap.add_argument("--time-slices", type=int, default=0, help="force the prefill's waves per time chunk (0 = auto)")
    ap.add_argument("--no-cfg", action="store_true",
                    help="skip the B1 L4096 D2048 and packed T=32768 prefill legs and the complexity checks")
    ap.add_argument("--no-alu", action="store_true", help="skip the ALU issue-rate probes")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 512 MiB device copy (untimed), the reference kernel for HBM byte counters")
    ap.add_argument("--pmc-summary", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT"),
                    help="summarise two rocprofv3 counter runs into OUT (host only; no GPU work)")
    ap.add_argument("--pmc-summary-swa", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT"),
                    help="the same for the attention kernels (counter runs of the --swa-only legs)")
    ap.add_argument("--pmc-summary-groups", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT"),
                    help="the same for the grouped prefill (counter runs of the --groups-only leg)")
    ap.add_argument("--pmc-summary-ssd", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT"),
                    help="the same for the SSD prefill (counter runs of the --ssd-only leg)")
    ap.add_argument("--valu-summary", nargs=3, metavar=("PASS_A_DIR", "PASS_B_DIR", "OUT"),
                    help="per-(token, channel) VALU counters of the prefill kernel from the two SQ passes")
    ap.add_argument("--pmc-summary-retention", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT"),
                    help="the same for the retention configuration (counter runs of the --retention-only leg)")
    ap.add_argument("--pmc-summary-gla", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT"),
                    help="the same for gated linear attention (counter runs of the --gla-only leg)")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.valu_summary:
        valu_summary(*args.valu_summary)
        return
    if args.pmc_summary_swa:
        _counter_summary(*args.pmc_summary_swa, which="swa")
        return
    if args.pmc_summary_groups:
        _counter_summary(*args.pmc_summary_groups, which="groups")
        return
    if args.pmc_summary_ssd:
        _counter_summary(*args.pmc_summary_ssd, which="ssd")
        return
    if args.pmc_summary_gla:
        _counter_summary(*args.pmc_summary_gla, which="gla")
        return
    if args.pmc_summary_retention:
        _counter_summary(*args.pmc_summary_retention, which="retention")
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only (the library has no multi-GPU path); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    if args.groups_only:
        out = {"groups": bench_groups(args.groups_steps, min(args.warmup, 3)), "groups_decode": bench_groups_step()}
        if args.copy_probe:
            copy_probe()
        print(json.dumps(out), flush=True)
        return
    if args.gla_only:
        out = {"gla": bench_gla(args.gla_steps, min(args.warmup, 2))}
        if args.copy_probe:
            copy_probe()
        print(json.dumps(out), flush=True)
        return
    if args.retention_only:
        out = {"retention": bench_retention(args.ssd_steps, min(args.warmup, 5))}
        if args.copy_probe:
            copy_probe()
        print(json.dumps(out), flush=True)
        return
    if args.ssd_only:
        out = {"ssd": bench_ssd(args.ssd_steps, min(args.warmup, 5))}
        if args.copy_probe:
            copy_probe()
        print(json.dumps(out), flush=True)
        return
    if args.swa_only:
        out = {"attention": bench_swa(args.swa_steps, min(args.warmup, 5)),
               "attention_decode": bench_swa_decode(args.swa_decode_steps, min(args.warmup, 20))}
        if args.copy_probe:
            copy_probe()
        print(json.dumps(out), flush=True)
        return

    pf = bench_prefill(args.steps, args.warmup, args.time_slices)
    # (counter runs skip the ceiling measurement: its 1 GiB copies are not needed there)
    ceiling = None if args.copy_probe else copy_ceiling()
    if args.copy_probe:
        copy_probe()
    achieved = SLOTS_PER_TD * pf["launch_td"] / (pf["launch_ms"] * 1e-3) / 1e12
    traffic = read_traffic()
    # (counter runs skip the ALU probes and the complexity checks: their launches would mix into the medians)
    alu = None if (args.no_alu or args.copy_probe) else alu_ceiling()
    valu = read_valu_counters()
    line = {
        "metric": METRIC,
        "value": round(pf["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pf["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "long-prompt prefill L=131072 D=4096 N=16 as 8 chained calls of 16384 "
                               "(h0 -> h_last), bf16 I/O, fp32 state", "seq_len": 131072, "dim": 4096,
                   "dstate": 16, "chunks": 8, "io": "bf16"},
        "tokens_channels_per_s": pf["tokens_channels_per_s"],
        "hbm_frac": pf["gbs"] / HBM_PEAK_GBS,
        "copy_ceiling_gbs": round(ceiling, 1) if ceiling else None,
        "copy_frac": pf["gbs"] / ceiling if ceiling else None,
        "plan": pf["plan"],
        "call_us": pf["call_us"],
        "roofline": {"bound": "alu", "achieved": round(achieved, 3), "peak": round(VALU_PEAK_TSLOT, 2),
                     "unit": "Tslot/s", "frac": round(achieved / VALU_PEAK_TSLOT, 4),
                     "traffic": traffic, "kernel": kernel_name(pf["plan"]),
                     "launch_us": round(pf["launch_ms"] * 1e3, 2), "slots_per_token_channel": SLOTS_PER_TD,
                     "algorithmic_bytes_per_launch": pf["bytes_per_launch"]},
    }
    rf = line["roofline"]
    launch_td_s = pf["launch_td"] / (pf["launch_ms"] * 1e-3)
    rf["hbm_frac_of_launch"] = round(pf["bytes_per_launch"] / (pf["launch_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    if alu:
        rf["measured_ceiling_td_per_s"] = alu["prefill_ceiling_td_per_s"]
        rf["frac_of_measured_ceiling"] = round(launch_td_s / alu["prefill_ceiling_td_per_s"], 4)
        line["alu_ceiling"] = alu
    if valu:
        rf["executed_per_td"] = {k: valu[k] for k in ("valu_lane_ops_per_td", "trans_lane_ops_per_td",
                                                       "executed_slots_per_td") if k in valu}
        rf["executed_over_algorithmic_slots"] = round(valu["executed_slots_per_td"] / SLOTS_PER_TD, 3)
    if not args.no_decode:
        dec = bench_decode(args.decode_steps)
        dec["roofline"] = {"bound": "hbm", "achieved": round(dec["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(dec["gbs"] / HBM_PEAK_GBS, 4), "traffic": read_traffic("decode_step"),
                           "kernel": "scan_step_kernel<bf16,bf16>"}
        dec["copy_frac"] = dec["gbs"] / ceiling if ceiling else None
        dec["note"] = ("one 16 MiB state read and written in place by every step: it stays in the 256 MB last-level "
                       "cache, so these bytes are cache-assisted; decode_many_states is the HBM-bound variant")
        line["decode"] = dec
    if not args.no_decode and not args.copy_probe:
        line["decode_many_states"] = bench_decode_states()
    if not args.no_cfg:
        line["cfg1"] = bench_cfg1()
        line["cfg1"]["roofline"]["traffic"] = read_traffic("cfg1")
        line["cfg2"] = bench_cfg2()
        line["cfg2"]["roofline"]["traffic"] = read_traffic("cfg2")
        if not args.copy_probe:
            line["complexity"] = bench_complexity()
    if not args.no_proj:
        line["projections"] = bench_proj(args.proj_steps)
        line["projections"]["roofline"]["traffic"] = read_traffic("projections")
    if not args.no_bwd:
        line["backward"] = bench_backward(args.bwd_steps)
        line["backward"]["roofline"]["traffic"] = read_traffic("backward")
    if not args.no_groups:
        line["groups"] = bench_groups(args.groups_steps)
        line["groups_decode"] = bench_groups_step()
    if not args.no_ssd:
        line["ssd"] = bench_ssd(args.ssd_steps)
        line["retention"] = bench_retention(args.ssd_steps)
    if not args.no_gla:
        line["gla"] = bench_gla(args.gla_steps)
    if not args.no_swa:
        line["attention"] = bench_swa(args.swa_steps)
        line["attention_decode"] = bench_swa_decode(args.swa_decode_steps)
        line["attention_decode"]["copy_frac"] = line["attention_decode"]["gbs"] / ceiling if ceiling else None
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline()
        if not args.no_decode:
            line["cpu_baseline"]["decode"] = cpu_baseline_decode()
        if not args.no_cfg:
            line["cpu_baseline"]["cfg1"] = cpu_baseline_cfg1()
            line["cpu_baseline"]["cfg2"] = cpu_baseline_cfg2()
        if not args.no_bwd:
            line["cpu_baseline"]["backward"] = cpu_baseline_backward()
        if not args.no_proj:
            line["cpu_baseline"]["projections"] = cpu_baseline_proj()
        if not args.no_groups:
            line["cpu_baseline"]["groups"] = cpu_baseline_groups()
        if not args.no_ssd:
            line["cpu_baseline"]["ssd"] = cpu_baseline_ssd()
        if not args.no_gla:
            line["cpu_baseline"]["gla"] = cpu_baseline_gla()
        if not args.no_swa:
            line["cpu_baseline"]["attention"] = cpu_baseline_swa()
            line["cpu_baseline"]["attention_decode"] = cpu_baseline_swa_decode()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
