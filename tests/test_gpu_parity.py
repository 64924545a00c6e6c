"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Host-sized cases run the oracle over every output; the full-size workloads
(long prompt, packed variable lengths, streaming decode) compare sampled
channels that the oracle computes one by one, in the same launch
configuration the benchmark times.  Tolerances: tests/parity.py.
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as O
from selective_state_space_05_amd import inputs as I
from selective_state_space_05_amd import scan as S
from tests.parity import check_bf16_y, check_fp32, norm_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_in(arr, in_dtype):
    """Host array (bf16 bit patterns or fp32) -> device tensor of the matching dtype."""
    if in_dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(DEV)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_case(batch, L, D, in_dtype="bf16", y_dtype="f32", ts=0, h0_scale=0.0, cfg=0, dt_override=None, lanes=0):
    """Build a seeded host-sized case, run GPU and oracle, return both."""
    rows = batch * L
    inp = I.make_fwd_inputs_np(cfg, rows, D, in_dtype=in_dtype)
    if dt_override is not None:
        v = np.full((rows, D), dt_override, dtype=np.float32)
        inp["dt"] = I.bf16_bits_from_f32(v) if in_dtype == "bf16" else v
        inp["dt_f32"] = I.f32_from_bf16_bits(inp["dt"]) if in_dtype == "bf16" else v
    h0 = I.make_h0(cfg, batch, D, scale=h0_scale) if h0_scale else None
    shp = (batch, L, D)
    x, dt, z = (dev_in(inp[k], in_dtype).reshape(shp) for k in ("x", "dt", "z"))
    B, C = (dev_in(inp[k], in_dtype).reshape(batch, L, 16) for k in ("B", "C"))
    A, Dv, bias = (torch.from_numpy(inp[k]).to(DEV) for k in ("A", "D", "dt_bias"))
    h0_t = torch.from_numpy(h0).to(DEV) if h0 is not None else None
    ydt = torch.float32 if y_dtype == "f32" else torch.bfloat16
    y, hl = S.scan_fwd(x, dt, z, B, C, A, Dv, bias, h0=h0_t, y_dtype=ydt, time_slices=ts, lanes_per_channel=lanes)
    torch.cuda.synchronize()
    yo, ho = O.scan_fwd(inp["x_f32"].reshape(shp), inp["dt_f32"].reshape(shp), inp["z_f32"].reshape(shp),
                        inp["B_f32"].reshape(batch, L, 16), inp["C_f32"].reshape(batch, L, 16), inp["A"], inp["D"],
                        inp["dt_bias"], h0=h0)
    return dict(y=host(y), h=host(hl), yo=yo, ho=ho, inp=inp, h0=h0)


def check_case(r, batch, L, y_dtype, what):
    bounds = np.arange(batch + 1) * L
    y = r["y"].reshape(batch * L, -1)
    yo = r["yo"].reshape(batch * L, -1)
    if y_dtype == "f32":
        e = check_fp32(y, yo, what + " y", bounds)
    else:
        e = check_bf16_y(y, yo, what + " y", bounds)
    eh = check_fp32(r["h"].reshape(batch, -1), r["ho"].reshape(batch, -1), what + " h_last")
    say("%s: y err %.3e  h_last err %.3e" % (what, e, eh))


# --------------------------------------------------------------------------- #
# host-sized cases, whole-output comparison
# --------------------------------------------------------------------------- #
SMALL = [
    # batch, L, D, in, y, time_slices, h0 scale
    (1, 256, 64, "f32", "f32", 0, 0.0),     # the fp32 reference workload
    (1, 256, 64, "f32", "bf16", 0, 0.0),
    (1, 256, 64, "bf16", "f32", 8, 1.0),
    (2, 1, 16, "bf16", "f32", 0, 1.0),      # single token
    (3, 5, 40, "bf16", "f32", 1, 0.5),      # ragged tokens (< 4) and channels (not a multiple of 16)
    (1, 130, 33, "bf16", "f32", 8, 1.0),    # ragged last chunk with 8 slices
    (1, 300, 33, "bf16", "f32", 16, 1.0),   # 16 slices of 8 tokens, ragged
    (3, 1000, 48, "bf16", "f32", 16, 1.0),
    (2, 1000, 48, "bf16", "f32", 1, 1.0),
    (2, 1000, 48, "bf16", "f32", 2, 1.0),
    (2, 1000, 48, "bf16", "f32", 4, 1.0),
    (2, 1000, 48, "bf16", "bf16", 8, 1.0),
    (1, 777, 1, "bf16", "f32", 4, 1.0),     # one channel
    (4, 63, 20, "f32", "f32", 2, 2.0),
]


@pytest.mark.parametrize("lanes", [4, 8])
@pytest.mark.parametrize("batch,L,D,ind,yd,ts,h0s", SMALL)
def test_small(batch, L, D, ind, yd, ts, h0s, lanes):
    """Every case through the 4-lane kernel and, where time is split, the 8-lane kernel (8-channel tiles)."""
    if lanes == 8 and ts == 1:
        pytest.skip("the 8-lane kernel only splits time (a sequential plan has 4 lanes per channel)")
    say("case batch=%d L=%d D=%d in=%s y=%s slices=%d h0=%g lanes=%d" % (batch, L, D, ind, yd, ts, h0s, lanes))
    r = run_case(batch, L, D, ind, yd, ts, h0s, lanes=lanes if ts != 1 else 0)
    check_case(r, batch, L, yd, "B%d L%d D%d" % (batch, L, D))


def test_empty_sequence_copies_carry():
    D = 48
    h0 = torch.randn(2, D, 16, device=DEV)
    p = I.make_params(0, D)
    A, Dv, bias = (torch.from_numpy(p[k]).to(DEV) for k in ("A", "D", "dt_bias"))
    e = torch.empty(2, 0, D, device=DEV, dtype=torch.bfloat16)
    eB = torch.empty(2, 0, 16, device=DEV, dtype=torch.bfloat16)
    y, hl = S.scan_fwd(e, e, e, eB, eB, A, Dv, bias, h0=h0)
    torch.cuda.synchronize()
    assert y.shape == (2, 0, D) and torch.equal(hl, h0)
    y, hl = S.scan_fwd(e, e, e, eB, eB, A, Dv, bias)
    torch.cuda.synchronize()
    assert torch.count_nonzero(hl) == 0


def test_time_slices_agree():
    """Every slicing of the time axis, with 4 or 8 lanes per channel, gives the same result to fp32 rounding."""
    outs = {}
    outs[(1, 4)] = run_case(1, 2000, 64, "bf16", "f32", 1, 1.0, cfg=1)
    for ts in (2, 4, 8, 16):
        for lanes in (4, 8):
            outs[(ts, lanes)] = run_case(1, 2000, 64, "bf16", "f32", ts, 1.0, cfg=1, lanes=lanes)
    for key, r in outs.items():
        assert norm_err(r["y"], outs[(1, 4)]["y"]) < 1e-5, key
        assert norm_err(r["h"], outs[(1, 4)]["h"]) < 1e-5, key


@pytest.mark.parametrize("ts", [1, 4, 8, 16])
@pytest.mark.parametrize("in_dtype,y_dtype", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "bf16"), ("f32", "f32")])
def test_scheduled_copies_agree(ts, in_dtype, y_dtype):
    """At 1, 4, 8 and 16 time slices a call without h_ckpt runs the prefill kernel's separately scheduled copy,
    the same call with h_ckpt the library's other copy: y and h_last must be bitwise the same, and match
    the oracle (several tiles, a ragged channel tile and a ragged last chunk)."""
    batch, L, D, cfg = 2, 333, 72, 2
    say("case: scheduled copies, W=%d %s -> %s" % (ts, in_dtype, y_dtype))
    rows = batch * L
    inp = I.make_fwd_inputs_np(cfg, rows, D, in_dtype=in_dtype)
    h0 = I.make_h0(cfg, batch, D, scale=1.0)
    shp = (batch, L, D)
    x, dt, z = (dev_in(inp[k], in_dtype).reshape(shp) for k in ("x", "dt", "z"))
    B, C = (dev_in(inp[k], in_dtype).reshape(batch, L, 16) for k in ("B", "C"))
    A, Dv, bias = (torch.from_numpy(inp[k]).to(DEV) for k in ("A", "D", "dt_bias"))
    h0_t = torch.from_numpy(h0).to(DEV)
    ydt = torch.float32 if y_dtype == "f32" else torch.bfloat16
    y1, hl1 = S.scan_fwd(x, dt, z, B, C, A, Dv, bias, h0=h0_t, y_dtype=ydt, time_slices=ts, lanes_per_channel=4)
    ck = S.alloc_ckpt(x, None)
    y2, hl2 = S.scan_fwd(x, dt, z, B, C, A, Dv, bias, h0=h0_t, y_dtype=ydt, time_slices=ts, lanes_per_channel=4,
                         h_ckpt=ck)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(hl1, hl2)
    yo, ho = O.scan_fwd(inp["x_f32"].reshape(shp), inp["dt_f32"].reshape(shp), inp["z_f32"].reshape(shp),
                        inp["B_f32"].reshape(batch, L, 16), inp["C_f32"].reshape(batch, L, 16), inp["A"], inp["D"],
                        inp["dt_bias"], h0=h0)
    bounds = np.arange(batch + 1, dtype=np.int64) * L
    if y_dtype == "f32":
        check_fp32(host(y1).reshape(rows, D), yo.reshape(rows, D), "y", bounds)
    else:
        check_bf16_y(host(y1).reshape(rows, D), yo.reshape(rows, D), "y", bounds)
    check_fp32(host(hl1).reshape(batch, -1), ho.reshape(batch, -1), "h_last")


def test_delta_to_zero_carry_pin():
    """dt_raw = -40 makes Δ ~ 1e-18: h_last must equal h0 and y_t = (C_t.h0 + D x_t) silu(z_t).
    Away from the first token only a correct carry (across slices, chunks and waves) gives this."""
    for ts, lanes in ((1, 0), (8, 4), (16, 4), (2, 8), (8, 8), (16, 8)):
        r = run_case(2, 1000, 32, "bf16", "f32", ts, 1.0, dt_override=-40.0, lanes=lanes)
        inp, h0 = r["inp"], r["h0"]
        C = inp["C_f32"].reshape(2, 1000, 16).astype(np.float64)
        x = inp["x_f32"].reshape(2, 1000, 32).astype(np.float64)
        z = inp["z_f32"].reshape(2, 1000, 32).astype(np.float64)
        closed = (np.einsum("btn,bdn->btd", C, h0) + inp["D"][None, None, :] * x) * z / (1 + np.exp(-z))
        assert norm_err(r["y"], closed) < 1e-5
        assert np.max(np.abs(r["h"] - h0)) < 1e-6
        check_case(r, 2, 1000, "f32", "dt->0 slices=%d" % ts)


@pytest.mark.parametrize("lanes", [4, 8])
def test_slow_decay_chained_calls(lanes):
    """Long memory (Δ = 1e-3, A = -1): 4 chained calls of 1024 tokens == one call == oracle."""
    D, L, parts = 64, 4096, 4
    inp = I.make_fwd_inputs_np(3, L, D)
    inp["dt"] = I.bf16_bits_from_f32(np.zeros((L, D), np.float32))
    inp["dt_f32"] = I.f32_from_bf16_bits(inp["dt"])
    bias = np.full(D, math.log(math.expm1(1e-3)), np.float32)
    A = -np.ones((D, 16), np.float32)
    x, dt, z = (dev_in(inp[k], "bf16").reshape(1, L, D) for k in ("x", "dt", "z"))
    B, C = (dev_in(inp[k], "bf16").reshape(1, L, 16) for k in ("B", "C"))
    A_t, D_t, b_t = torch.from_numpy(A).to(DEV), torch.from_numpy(inp["D"]).to(DEV), torch.from_numpy(bias).to(DEV)
    y1, h1 = S.scan_fwd(x, dt, z, B, C, A_t, D_t, b_t, y_dtype=torch.float32, time_slices=8, lanes_per_channel=lanes)
    h = None
    ys = []
    n = L // parts
    for i in range(parts):
        sl = slice(i * n, (i + 1) * n)
        yi, h = S.scan_fwd(x[:, sl].contiguous(), dt[:, sl].contiguous(), z[:, sl].contiguous(),
                           B[:, sl].contiguous(), C[:, sl].contiguous(), A_t, D_t, b_t, h0=h,
                           y_dtype=torch.float32, time_slices=8, lanes_per_channel=lanes)
        ys.append(yi)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(ys, 1), y1) and torch.equal(h, h1)
    yo, ho = O.scan_fwd(inp["x_f32"][None], inp["dt_f32"][None], inp["z_f32"][None], inp["B_f32"][None],
                        inp["C_f32"][None], A, inp["D"], bias)
    check_fp32(host(y1)[0], yo[0], "slow decay y")
    check_fp32(host(h1), ho, "slow decay h_last")


def test_deterministic_and_in_place_carry():
    inp = I.make_fwd_inputs_np(1, 3000, 96)
    x, dt, z = (dev_in(inp[k], "bf16").reshape(1, 3000, 96) for k in ("x", "dt", "z"))
    B, C = (dev_in(inp[k], "bf16").reshape(1, 3000, 16) for k in ("B", "C"))
    A, Dv, bias = (torch.from_numpy(inp[k]).to(DEV) for k in ("A", "D", "dt_bias"))
    h0 = torch.randn(1, 96, 16, device=DEV)
    y1, h1 = S.scan_fwd(x, dt, z, B, C, A, Dv, bias, h0=h0)
    y2, h2 = S.scan_fwd(x, dt, z, B, C, A, Dv, bias, h0=h0)
    hbuf = h0.clone()
    y3, h3 = S.scan_fwd(x, dt, z, B, C, A, Dv, bias, h0=hbuf, h_last=hbuf)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    assert torch.equal(y1, y3) and torch.equal(h1, h3) and h3.data_ptr() == hbuf.data_ptr()


def test_varlen_small_with_empty_sequences():
    lens = [0, 37, 1, 300, 0, 129, 64]
    T, D = sum(lens), 40
    cu = I.cu_from_lengths(lens)
    inp = I.make_fwd_inputs_np(2, T, D)
    h0 = I.make_h0(2, len(lens), D, scale=1.0)
    x, dt, z = (dev_in(inp[k], "bf16") for k in ("x", "dt", "z"))
    B, C = (dev_in(inp[k], "bf16") for k in ("B", "C"))
    A, Dv, bias = (torch.from_numpy(inp[k]).to(DEV) for k in ("A", "D", "dt_bias"))
    for ts, lanes in ((0, 0), (1, 0), (4, 4), (16, 4), (4, 8), (16, 8)):
        y, hl = S.scan_fwd(x, dt, z, B, C, A, Dv, bias, h0=torch.from_numpy(h0).to(DEV),
                           cu_seqlens=torch.from_numpy(cu).to(DEV), y_dtype=torch.float32, time_slices=ts,
                           lanes_per_channel=lanes)
        torch.cuda.synchronize()
        yo, ho = O.scan_fwd(inp["x_f32"], inp["dt_f32"], inp["z_f32"], inp["B_f32"], inp["C_f32"], inp["A"],
                            inp["D"], inp["dt_bias"], h0=h0, seq_start=cu.astype(np.int64))
        check_fp32(host(y), yo, "varlen y ts=%d lanes=%d" % (ts, lanes), cu)
        check_fp32(host(hl).reshape(len(lens), -1), ho.reshape(len(lens), -1),
                   "varlen h_last ts=%d lanes=%d" % (ts, lanes))
        assert np.array_equal(host(hl)[0], h0[0]) and np.array_equal(host(hl)[4], h0[4])


def test_step_matches_oracle_and_fwd():
    """Decode steps == oracle steps, and a step loop == one prefill over the same tokens."""
    Bt, D, L = 6, 80, 40
    inp = I.make_fwd_inputs_np(4, Bt * L, D)
    h0 = I.make_h0(4, Bt, D, scale=1.0)
    sh = (Bt, L, D)
    x, dt, z = (dev_in(inp[k], "bf16").reshape(sh) for k in ("x", "dt", "z"))
    B, C = (dev_in(inp[k], "bf16").reshape(Bt, L, 16) for k in ("B", "C"))
    A, Dv, bias = (torch.from_numpy(inp[k]).to(DEV) for k in ("A", "D", "dt_bias"))
    yf, hf = S.scan_fwd(x, dt, z, B, C, A, Dv, bias, h0=torch.from_numpy(h0).to(DEV), y_dtype=torch.float32)
    st = torch.from_numpy(h0).to(DEV).contiguous()
    ys = []
    for t in range(L):
        ys.append(S.scan_step(st, x[:, t].contiguous(), dt[:, t].contiguous(), z[:, t].contiguous(),
                              B[:, t].contiguous(), C[:, t].contiguous(), A, Dv, bias, y_dtype=torch.float32))
    torch.cuda.synchronize()
    ys = torch.stack(ys, 1)
    assert norm_err(host(ys), host(yf)) < 1e-5 and norm_err(host(st), host(hf)) < 1e-5
    yo, ho = O.scan_fwd(inp["x_f32"].reshape(sh), inp["dt_f32"].reshape(sh), inp["z_f32"].reshape(sh),
                        inp["B_f32"].reshape(Bt, L, 16), inp["C_f32"].reshape(Bt, L, 16), inp["A"], inp["D"],
                        inp["dt_bias"], h0=h0)
    check_fp32(host(ys).reshape(Bt * L, D), yo.reshape(Bt * L, D), "step y", np.arange(Bt + 1) * L)
    check_fp32(host(st).reshape(Bt, -1), ho.reshape(Bt, -1), "step state")


def test_step_many_sequences_ragged():
    """A batch large enough for several sequences per thread, with ragged batch and channel counts."""
    Bt, D = 130, 2000
    g = np.random.default_rng(7)
    p = I.make_params(1, D)
    st0 = (0.5 * g.standard_normal((Bt, D, 16))).astype(np.float32)
    s = I.make_step_inputs_np(1, 0, Bt, D)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    bf = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)
    st = T(st0)
    y = S.scan_step(st, bf(s["x"]), bf(s["dt"]), bf(s["z"]), bf(s["B"]), bf(s["C"]), T(p["A"]), T(p["D"]),
                    T(p["dt_bias"]), y_dtype=torch.float32)
    torch.cuda.synchronize()
    yo, so = O.scan_step(st0, s["x_f32"], s["dt_f32"], s["z_f32"], s["B_f32"], s["C_f32"], p["A"], p["D"], p["dt_bias"])
    check_fp32(host(y), yo, "step ragged y", np.arange(Bt + 1))
    check_fp32(host(st).reshape(Bt, -1), so.reshape(Bt, -1), "step ragged state")


def test_step_fp32_io_and_ragged_dim():
    Bt, D = 3, 37
    g = np.random.default_rng(5)
    p = I.make_params(0, D)
    st0 = g.standard_normal((Bt, D, 16)).astype(np.float32)
    x, dt, z = (g.standard_normal((Bt, D)).astype(np.float32) for _ in range(3))
    Bv, Cv = (g.standard_normal((Bt, 16)).astype(np.float32) for _ in range(2))
    st = torch.from_numpy(st0).to(DEV)
    T = lambda a: torch.from_numpy(a).to(DEV)
    y = S.scan_step(st, T(x), T(dt), T(z), T(Bv), T(Cv), T(p["A"]), T(p["D"]), T(p["dt_bias"]))
    torch.cuda.synchronize()
    yo, so = O.scan_step(st0, x, dt, z, Bv, Cv, p["A"], p["D"], p["dt_bias"])
    check_fp32(host(y), yo, "step fp32 y")
    check_fp32(host(st).reshape(Bt, -1), so.reshape(Bt, -1), "step fp32 state")


# --------------------------------------------------------------------------- #
# full-size workloads (launch configuration of the benchmark), sampled channels
# --------------------------------------------------------------------------- #
def sample_channels(D, k, seed):
    g = np.random.default_rng(seed)
    fixed = [0, 1, 15, 16, 17, D // 2, D - 17, D - 16, D - 1]
    rest = g.choice(D, size=k - len(fixed), replace=False)
    return np.unique(np.concatenate([fixed, rest]))


def oracle_on_channels(x, dt, z, B, C, P, sel, h0=None, seq_start=None):
    """x, dt, z: device [tokens][D]; B, C: device [tokens][16]; P: host params dict."""
    st = torch.from_numpy(sel).to(DEV)
    xs, ds, zs = (host(t.index_select(1, st)) for t in (x, dt, z))
    return O.scan_fwd(xs, ds, zs, host(B), host(C), P["A"][sel], P["D"][sel], P["dt_bias"][sel],
                      h0=None if h0 is None else h0[:, sel], seq_start=seq_start)


def test_full_cfg1_b1_l4096_d2048():
    W = I.WORKLOADS[1]
    inp = I.make_fwd_inputs_np(1, W.seqlen, W.dim)
    x, dt, z = (dev_in(inp[k], "bf16").reshape(1, W.seqlen, W.dim) for k in ("x", "dt", "z"))
    B, C = (dev_in(inp[k], "bf16").reshape(1, W.seqlen, 16) for k in ("B", "C"))
    A, Dv, bias = (torch.from_numpy(inp[k]).to(DEV) for k in ("A", "D", "dt_bias"))
    yb, hl = S.scan_fwd(x, dt, z, B, C, A, Dv, bias)
    yf, hf = S.scan_fwd(x, dt, z, B, C, A, Dv, bias, y_dtype=torch.float32)
    torch.cuda.synchronize()
    yo, ho = O.scan_fwd(inp["x_f32"], inp["dt_f32"], inp["z_f32"], inp["B_f32"], inp["C_f32"], inp["A"], inp["D"],
                        inp["dt_bias"])
    e1 = check_bf16_y(host(yb)[0], yo, "cfg1 bf16 y")
    e2 = check_fp32(host(yf)[0], yo, "cfg1 fp32 y")
    e3 = check_fp32(host(hl), ho, "cfg1 h_last")
    assert torch.equal(hl, hf)
    say("cfg1: bf16 ratio %.3f fp32 y %.3e h_last %.3e plan %s" % (e1, e2, e3, S.fwd_plan(
        x, dt, z, B, C, A, Dv, bias, y=yb)))


def test_full_cfg2_varlen_t32768_d4096():
    W = I.WORKLOADS[2]
    lens = I.varlen_lengths(2, W.varlen_total)
    cu = I.cu_from_lengths(lens)
    inp = I.make_fwd_inputs_torch(2, W.varlen_total, W.dim, DEV)
    P = I.make_params(2, W.dim)
    h0 = I.make_h0(2, len(lens), W.dim, scale=1.0)
    cu_t = torch.from_numpy(cu).to(DEV)
    args = [inp[k] for k in ("x", "dt", "z", "B", "C", "A", "D", "dt_bias")]
    yb, hl = S.scan_fwd(*args, h0=torch.from_numpy(h0).to(DEV), cu_seqlens=cu_t)
    yf, _ = S.scan_fwd(*args, h0=torch.from_numpy(h0).to(DEV), cu_seqlens=cu_t, y_dtype=torch.float32)
    torch.cuda.synchronize()
    sel = sample_channels(W.dim, 64, 22)
    yo, ho = oracle_on_channels(inp["x"], inp["dt"], inp["z"], inp["B"], inp["C"], P, sel, h0=h0,
                                seq_start=cu.astype(np.int64))
    st = torch.from_numpy(sel).to(DEV)
    e1 = check_bf16_y(host(yb.index_select(1, st)), yo, "cfg2 bf16 y", cu)
    e2 = check_fp32(host(yf.index_select(1, st)), yo, "cfg2 fp32 y", cu)
    e3 = check_fp32(host(hl)[:, sel].reshape(len(lens), -1), ho.reshape(len(lens), -1), "cfg2 h_last")
    say("cfg2: %d seqs, bf16 ratio %.3f fp32 y %.3e h_last %.3e" % (len(lens), e1, e2, e3))


def test_full_cfg3_chained_128k():
    """L = 131072, D = 4096 as 8 chained calls of 16384 == one call == oracle (sampled channels)."""
    W = I.WORKLOADS[3]
    L, D, n = W.seqlen, W.dim, W.chunks
    inp = I.make_fwd_inputs_torch(3, L, D, DEV)
    P = I.make_params(3, D)
    A, Dv, bias = inp["A"], inp["D"], inp["dt_bias"]
    cl = L // n
    yc = torch.empty(L, D, dtype=torch.bfloat16, device=DEV)
    hbufs = [torch.empty(1, D, 16, device=DEV) for _ in range(2)]
    h = None
    for i in range(n):
        sl = slice(i * cl, (i + 1) * cl)
        S.scan_fwd(*(inp[k][sl].view(1, cl, -1) for k in ("x", "dt", "z", "B", "C")), A, Dv, bias, h0=h,
                   h_last=hbufs[i % 2], y=yc[sl].view(1, cl, D))
        h = hbufs[i % 2]
    y1, h1 = S.scan_fwd(*(inp[k].view(1, L, -1) for k in ("x", "dt", "z", "B", "C")), A, Dv, bias,
                        y_dtype=torch.float32)
    torch.cuda.synchronize()
    sel = sample_channels(D, 48, 33)
    yo, ho = oracle_on_channels(inp["x"], inp["dt"], inp["z"], inp["B"], inp["C"], P, sel)
    st = torch.from_numpy(sel).to(DEV)
    e1 = check_bf16_y(host(yc.index_select(1, st)), yo, "cfg3 chained bf16 y")
    e2 = check_fp32(host(y1[0].index_select(1, st)), yo, "cfg3 single-pass fp32 y")
    e3 = check_fp32(host(h)[:, sel].reshape(1, -1), ho.reshape(1, -1), "cfg3 chained h_last")
    # chained vs single pass: same kernel, chunk boundaries aligned -> identical state
    assert torch.equal(h, h1), "chained h_last differs from single pass"
    d = norm_err(host(yc), host(y1[0].to(torch.bfloat16)))
    assert d == 0.0, "chained y differs from single pass by %.3e" % d
    say("cfg3: bf16 ratio %.3f fp32 y %.3e h_last %.3e chained==single" % (e1, e2, e3))


def test_full_cfg4_decode_65536_steps():
    """B = 64, D = 4096: prefill 2048 tokens, then 65536 steps over a ring of 256 input sets.

    Checked: the full state [64][4096][16] after 1024 steps, and, on all 64
    sequences x 64 sampled channels, the state after all 65536 steps and the y
    of the last 256 steps.  The oracle side runs the step tokens through its
    chained forward scan (its step loop equals its forward scan: pinned in the
    oracle tests), in sequence groups and time chunks that bound host memory."""
    W = I.WORKLOADS[4]
    Bt, L, D, steps, R = W.batch, W.seqlen, W.dim, W.decode_steps, W.decode_ring
    early = 1024
    pre = I.make_fwd_inputs_torch(4, Bt * L, D, DEV)
    P = I.make_params(4, D)
    A, Dv, bias = pre["A"], pre["D"], pre["dt_bias"]
    _, state = S.scan_fwd(*(pre[k].view(Bt, L, -1) for k in ("x", "dt", "z", "B", "C")), A, Dv, bias)
    ring = I.make_step_ring_torch(4, R, Bt, D, DEV)
    ys = torch.empty(R, Bt, D, dtype=torch.bfloat16, device=DEV)
    state_early = None
    for k in range(steps):
        r = k % R
        S.scan_step(state, ring["x"][r], ring["dt"][r], ring["z"][r], ring["B"][r], ring["C"][r], A, Dv, bias,
                    y=ys[r])
        if k == early - 1:
            state_early = state.clone()
    torch.cuda.synchronize()
    say("cfg4: GPU steps done")

    def ring_tokens(t, first, count, bsl, dsl=None):
        """Step inputs of steps first..first+count-1 as a token axis: [sequences][count][cols]."""
        v = t[:, bsl] if dsl is None else t[:, bsl][:, :, dsl]
        idx = torch.arange(first, first + count, device=DEV) % R
        return host(v.index_select(0, idx).transpose(0, 1).contiguous())

    # full state after `early` steps: oracle prefill + `early` step tokens, 8 sequences at a time
    lib = O.load()
    so_pre = np.empty((Bt, D, 16))
    worst = 0.0
    for g0 in range(0, Bt, 8):
        bs = slice(g0, g0 + 8)
        sub = {k: pre[k].view(Bt, L, -1)[bs] for k in ("x", "dt", "z", "B", "C")}
        _, hp = O.scan_fwd(*(host(sub[k]) for k in ("x", "dt", "z", "B", "C")), P["A"], P["D"], P["dt_bias"],
                           lib=lib)
        so_pre[bs] = hp
        _, he = O.scan_fwd(*(ring_tokens(ring[k], 0, early, bs) for k in ("x", "dt", "z", "B", "C")), P["A"],
                           P["D"], P["dt_bias"], h0=hp, lib=lib)
        ge = host(state_early[bs])
        worst = max(worst, check_fp32(ge.reshape(8, -1), he.reshape(8, -1), "cfg4 full state after %d steps" % early,
                                      np.arange(9)))
    say("cfg4: full state after %d steps err %.3e" % (early, worst))

    # 64 sequences x 64 sampled channels through all steps
    dsel = sample_channels(D, 64, 44)
    dtt = torch.from_numpy(dsel).to(DEV)
    bs = slice(0, Bt)
    so = so_pre[:, dsel]
    chunk = 4096
    yo_last = None
    for c0 in range(0, steps, chunk):
        toks = [ring_tokens(ring[k], c0, chunk, bs, dtt) for k in ("x", "dt", "z")]
        toks += [ring_tokens(ring[k], c0, chunk, bs) for k in ("B", "C")]
        yk, so = O.scan_fwd(*toks, P["A"][dsel], P["D"][dsel], P["dt_bias"][dsel], h0=so, lib=lib)
        if c0 + chunk == steps:
            yo_last = yk[:, chunk - R:]  # [seq][last R steps][ch]; step k uses ring slot k % R
    yg = host(ys.index_select(2, dtt)).transpose(1, 0, 2)  # [seq][ring slot][ch]
    e1 = check_bf16_y(yg.reshape(Bt * R, -1), yo_last.reshape(Bt * R, -1), "cfg4 last-256-steps bf16 y",
                      np.arange(Bt + 1) * R)
    sg = host(state.index_select(1, dtt))
    e2 = check_fp32(sg.reshape(Bt, -1), so.reshape(Bt, -1), "cfg4 state after 65536 steps", np.arange(Bt + 1))
    say("cfg4: bf16 ratio %.3f state err %.3e" % (e1, e2))
