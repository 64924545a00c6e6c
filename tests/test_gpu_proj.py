"""GPU parity of the selection projections (samba_proj through the C ABI) against the fp64 oracle.

The oracle (oracle_proj, pinned in tests/test_oracle_proj_pins.py) multiplies the exact bf16 input
values in fp64.  The GPU accumulates bf16 products in fp32 on the matrix cores.  Tolerance: for fp32
outputs, per output tensor max|g - o| / max|o| <= 2e-3 (the contract) with a tripwire of 1e-5 (an fp32
sum of dim products carries a few ulp of the partial sums, measured near 1e-6); bf16 outputs get one
bf16 rounding on top (tests/parity.py), per output column.  Cases: ragged tokens and features (tiles of
128), a K tail (dim not a multiple of 64), both output dtypes, the full 16384 x 4096 shape on sampled
rows, and projections feeding the scan.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as O
from selective_state_space_05_amd import inputs as I
from selective_state_space_05_amd import scan as S
from tests.parity import check_bf16_y, check_fp32

pytestmark = pytest.mark.gpu
DEV = "cuda"
PROJ_TRIP = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("T,dim,out", [(300, 200, "f32"), (300, 200, "bf16"), (128, 64, "f32"), (1, 8, "f32"),
                                       (257, 384, "bf16")])
def test_proj_small(T, dim, out):
    say("case: proj T%d dim%d out %s" % (T, dim, out))
    inp = I.make_fwd_inputs_np(0, T, dim, in_dtype="bf16")
    w = I.make_proj_weight_np(0, dim)
    od = torch.float32 if out == "f32" else torch.bfloat16
    dt, B, C = S.proj(bf16_dev(inp["x"]).reshape(T, dim), bf16_dev(w["W"]).reshape(-1, dim), out_dtype=od)
    torch.cuda.synchronize()
    odt, oB, oC = O.proj(inp["x_f32"].reshape(T, dim), w["W_f32"])
    for name, g, o in (("dt", dt, odt), ("B", B, oB), ("C", C, oC)):
        if out == "f32":
            e = check_fp32(host(g), o, "proj " + name, trip=PROJ_TRIP)
        else:
            e = check_bf16_y(host(g), o, "proj " + name)
        say("  %s: %.2e" % (name, e))


@pytest.mark.parametrize("T,dim,N,out,shift", [(300, 296, 16, "bf16", 0), (130, 304, 8, "bf16", 0),
                                               (200, 136, 5, "bf16", 1), (70, 64, 3, "f32", 1),
                                               (513, 520, 16, "bf16", 1)])
def test_proj_ragged_columns_and_layouts(T, dim, N, out, shift):
    """Last column tile 72 and 64 wide (a wave computes 3 or 2 of its 4 column blocks), a state size that
    is not a multiple of 8 and outputs that start one element past a 16-byte boundary (element-wise
    result stores)."""
    say("case: proj T%d dim%d N%d out %s shift %d" % (T, dim, N, out, shift))
    inp = I.make_fwd_inputs_np(2, T, dim, in_dtype="bf16")
    w = I.make_proj_weight_np(2, dim, dstate=N)
    od = torch.float32 if out == "f32" else torch.bfloat16

    def buf(n):
        return torch.full((n + shift,), float("nan"), dtype=od, device=DEV)[shift:]

    dt, B, C = buf(T * dim).view(T, dim), buf(T * N).view(T, N), buf(T * N).view(T, N)
    S.proj(bf16_dev(inp["x"]).reshape(T, dim), bf16_dev(w["W"]).reshape(-1, dim), dt=dt, B=B, C=C)
    torch.cuda.synchronize()
    odt, oB, oC = O.proj(inp["x_f32"].reshape(T, dim), w["W_f32"], dstate=N)
    for name, g, o in (("dt", dt, odt), ("B", B, oB), ("C", C, oC)):
        if out == "f32":
            e = check_fp32(host(g), o, "proj " + name, trip=PROJ_TRIP)
        else:
            e = check_bf16_y(host(g), o, "proj " + name)
        say("  %s: %.2e" % (name, e))


def test_proj_full_shape_sampled_rows():
    """16384 tokens x 4096 channels (the long-prompt chunk), every output feature of 96 sampled tokens."""
    T, dim = 16384, 4096
    say("case: proj full T%d dim%d" % (T, dim))
    inp = I.make_fwd_inputs_torch(3, T, dim, DEV)
    W = I.make_proj_weight_torch(3, dim, DEV)
    dt, B, C = S.proj(inp["x"], W)
    torch.cuda.synchronize()
    g = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, 127, 128, T - 1], g.choice(T, 92, replace=False)]))
    ridx = torch.from_numpy(rows).to(DEV)
    odt, oB, oC = O.proj(host(inp["x"].index_select(0, ridx)), host(W))
    for name, gt, o in (("dt", dt, odt), ("B", B, oB), ("C", C, oC)):
        e = check_bf16_y(host(gt.index_select(0, ridx)), o, "proj full " + name)
        say("  %s: %.3f of the bound" % (name, e))


def test_proj_feeds_the_scan():
    """samba_proj -> samba_scan_fwd equals oracle_proj -> oracle_scan_fwd (fp32 projections)."""
    T, dim = 200, 64
    say("case: proj -> scan T%d dim%d" % (T, dim))
    inp = I.make_fwd_inputs_np(1, T, dim, in_dtype="bf16")
    w = I.make_proj_weight_np(1, dim)
    dt, B, C = S.proj(bf16_dev(inp["x"]).reshape(T, dim), bf16_dev(w["W"]).reshape(-1, dim), out_dtype=torch.float32)
    x32 = torch.from_numpy(inp["x_f32"].reshape(T, dim)).to(DEV)
    z32 = torch.from_numpy(inp["z_f32"].reshape(T, dim)).to(DEV)
    A, Dv, bias = (torch.from_numpy(inp[k]).to(DEV) for k in ("A", "D", "dt_bias"))
    y, hl = S.scan_fwd(x32.view(1, T, dim), dt.view(1, T, dim), z32.view(1, T, dim), B.view(1, T, 16),
                       C.view(1, T, 16), A, Dv, bias, y_dtype=torch.float32)
    torch.cuda.synchronize()
    odt, oB, oC = O.proj(inp["x_f32"].reshape(T, dim), w["W_f32"])
    yo, ho = O.scan_fwd(inp["x_f32"].reshape(T, dim), odt, inp["z_f32"].reshape(T, dim), oB, oC, inp["A"], inp["D"],
                        inp["dt_bias"])
    e1 = check_fp32(host(y).reshape(T, dim), yo, "proj -> scan y")
    e2 = check_fp32(host(hl).reshape(1, -1), ho.reshape(1, -1), "proj -> scan h_last")
    say("  y %.2e h_last %.2e" % (e1, e2))
