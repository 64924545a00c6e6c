"""GPU parity of the grouped prefill (samba_scan_fwd_groups through the C ABI) against the fp64 oracle
(oracle_scan_fwd_groups, pinned in tests/test_oracle_groups_pins.py).

Same tolerance reading as the ungrouped prefill (tests/parity.py): fp32 outputs per sequence within the
2e-3 contract and the 1e-4 tripwire, bf16 y one bf16 rounding on top per (sequence, channel).  Cases: every
state size (16, 32, 64, 128, 256) with several groups, fp32 and bf16 inputs and outputs, h0 given and
h_last written in place over it, packed sequences with empty ones, a ragged last chunk, one group equal to
the ungrouped kernel's result within rounding, and the benchmark's shape (B4 L4096 D4096 G4 N64) on sampled
channel blocks of every group.
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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


CASES = [
    # lengths, dim, G, N, in, out, h0
    ((100, 100), 64, 2, 32, "bf16", "bf16", False),
    ((100, 100), 64, 2, 32, "bf16", "f32", True),
    ((37,), 48, 3, 64, "f32", "f32", True),
    ((70, 9), 64, 2, 16, "bf16", "f32", True),
    ((33,), 16, 4, 128, "bf16", "f32", True),
    ((20, 3), 8, 2, 256, "f32", "f32", True),
    ((0, 41, 1, 0, 64), 32, 4, 32, "bf16", "f32", True),   # packed, with empty sequences
]


def run_case(lengths, dim, G, N, din, dout, with_h0, cfg=8, varlen=None):
    T = sum(lengths)
    nseq = len(lengths)
    inp = I.make_groups_inputs_np(cfg, T, dim, G, N, in_dtype=din)
    h0 = I.make_h0(cfg, nseq, dim, N, scale=0.5) if with_h0 else None
    packed = varlen if varlen is not None else len(set(lengths)) > 1 or 0 in lengths
    x, dt, z = (dev(inp[k], din).reshape(T, dim) for k in ("x", "dt", "z"))
    B, C = (dev(inp[k], din).reshape(T, G, N) for k in ("B", "C"))
    A, D, bias = (torch.from_numpy(inp[k]).to(DEV) for k in ("A", "D", "dt_bias"))
    od = torch.float32 if dout == "f32" else torch.bfloat16
    h0d = None if h0 is None else torch.from_numpy(h0).to(DEV)
    cu = torch.from_numpy(I.cu_from_lengths(lengths)).to(DEV) if packed else None
    if not packed:
        x, dt, z = (t.reshape(nseq, lengths[0], dim) for t in (x, dt, z))
        B, C = (t.reshape(nseq, lengths[0], G, N) for t in (B, C))
    # h_last written in place over h0 when h0 is given
    y, hl = S.scan_fwd_groups(x, dt, z, B, C, A, D, bias, h0=h0d, h_last=h0d, y_dtype=od, cu_seqlens=cu)
    torch.cuda.synchronize()
    bounds = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    yo, ho = O.scan_fwd_groups(inp["x_f32"], inp["dt_f32"], inp["z_f32"], inp["B_f32"], inp["C_f32"], inp["A"],
                               inp["D"], inp["dt_bias"], h0=h0, seq_start=bounds)
    return host(y).reshape(T, dim), yo, host(hl), ho, bounds


@pytest.mark.parametrize("lengths,dim,G,N,din,dout,with_h0", CASES)
def test_groups_matches_oracle(lengths, dim, G, N, din, dout, with_h0):
    say("case: groups", lengths, "dim", dim, "G", G, "N", N, din, dout, "h0" if with_h0 else "")
    y, yo, hl, ho, b = run_case(lengths, dim, G, N, din, dout, with_h0)
    ey = check_fp32(y, yo, "y", b) if dout == "f32" else check_bf16_y(y, yo, "y", b)
    eh = 0.0
    for s in range(len(lengths)):
        eh = max(eh, check_fp32(hl[s], ho[s], "h_last"))
    say("  y %.2e h_last %.2e" % (ey, eh))


def test_one_group_matches_ungrouped_kernel():
    """G = 1, N = 16 is the pages' selection: both kernels agree within fp32 rounding."""
    L, dim = 300, 128
    inp = I.make_groups_inputs_np(9, L, dim, 1, 16)
    x, dt, z = (dev(inp[k], "bf16").reshape(1, L, dim) for k in ("x", "dt", "z"))
    B, C = (dev(inp[k], "bf16").reshape(1, L, 1, 16) for k in ("B", "C"))
    A, D, bias = (torch.from_numpy(inp[k]).to(DEV) for k in ("A", "D", "dt_bias"))
    yg, hg = S.scan_fwd_groups(x, dt, z, B, C, A, D, bias, y_dtype=torch.float32)
    yu, hu = S.scan_fwd(x, dt, z, B.reshape(1, L, 16), C.reshape(1, L, 16), A, D, bias, y_dtype=torch.float32)
    torch.cuda.synchronize()
    check_fp32(host(yg), host(yu), "y vs ungrouped")
    check_fp32(host(hg), host(hu), "h_last vs ungrouped")


def test_groups_deterministic():
    L, dim, G, N = 200, 64, 2, 64
    inp = I.make_groups_inputs_np(10, L, dim, G, N)
    x, dt, z = (dev(inp[k], "bf16").reshape(1, L, dim) for k in ("x", "dt", "z"))
    B, C = (dev(inp[k], "bf16").reshape(1, L, G, N) for k in ("B", "C"))
    A, D, bias = (torch.from_numpy(inp[k]).to(DEV) for k in ("A", "D", "dt_bias"))
    y1, h1 = S.scan_fwd_groups(x, dt, z, B, C, A, D, bias)
    y2, h2 = S.scan_fwd_groups(x, dt, z, B, C, A, D, bias)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)) and torch.equal(h1, h2)


def test_groups_full_shape_sampled():
    """B4 L4096 D4096 G4 N64 (the benchmark's launch): a block of 8 channels from each group of each
    sequence against the oracle (channels are independent; a block's group is the same)."""
    wl = I.WORKLOADS[8]
    Bt, L, dim, N, G = wl.batch, wl.seqlen, wl.dim, wl.dstate, wl.extra["ngroups"]
    say("case: groups full shape B%d L%d D%d G%d N%d" % (Bt, L, dim, G, N))
    t = I.make_groups_inputs_torch(8, Bt * L, dim, G, N, DEV)
    x, dt, z = (t[k].view(Bt, L, dim) for k in ("x", "dt", "z"))
    B, C = (t[k].view(Bt, L, G, N) for k in ("B", "C"))
    y, hl = S.scan_fwd_groups(x, dt, z, B, C, t["A"], t["D"], t["dt_bias"])
    torch.cuda.synchronize()
    per = dim // G
    for s in (0, 3):
        for g in range(G):
            c0 = g * per + (37 * (g + 1)) % (per - 8)
            sl = slice(c0, c0 + 8)
            yo, ho = O.scan_fwd(host(x[s, :, sl]), host(dt[s, :, sl]), host(z[s, :, sl]), host(B[s, :, g]),
                                host(C[s, :, g]), host(t["A"][sl]), host(t["D"][sl]), host(t["dt_bias"][sl]))
            check_bf16_y(host(y[s, :, sl]), yo, "y s%d g%d" % (s, g))
            check_fp32(host(hl[s, sl]), ho[0], "h_last s%d g%d" % (s, g))
    say("  ok")


@pytest.mark.parametrize("N,G,din,dout", [(16, 2, "bf16", "f32"), (64, 4, "bf16", "bf16"), (256, 1, "f32", "f32")])
def test_step_groups_continues_prefill(N, G, din, dout):
    """Prefill 30 tokens, then 5 grouped decode steps from its h_last: each step against the oracle's grouped
    prefill over the whole sequence (its row for that token; the final state against its h_last)."""
    say("case: step groups N%d G%d %s %s" % (N, G, din, dout))
    Bt, L, steps, dim = 3, 30, 5, 64
    n = L + steps
    inp = I.make_groups_inputs_np(12, Bt * n, dim, G, N, in_dtype=din)
    view = lambda k, shape: dev(inp[k], din).reshape(shape)
    x, dt, z = (view(k, (Bt, n, dim)) for k in ("x", "dt", "z"))
    B, C = (view(k, (Bt, n, G, N)) for k in ("B", "C"))
    A, D, bias = (torch.from_numpy(inp[k]).to(DEV) for k in ("A", "D", "dt_bias"))
    _, state = S.scan_fwd_groups(x[:, :L].contiguous(), dt[:, :L].contiguous(), z[:, :L].contiguous(),
                                 B[:, :L].contiguous(), C[:, :L].contiguous(), A, D, bias)
    od = torch.float32 if dout == "f32" else torch.bfloat16
    ys = []
    for t in range(L, n):
        ys.append(S.scan_step_groups(state, x[:, t].contiguous(), dt[:, t].contiguous(), z[:, t].contiguous(),
                                     B[:, t].contiguous(), C[:, t].contiguous(), A, D, bias, y_dtype=od))
    torch.cuda.synchronize()
    f = lambda k, shape: inp[k + "_f32"].reshape(shape)
    yo, ho = O.scan_fwd_groups(f("x", (Bt, n, dim)), f("dt", (Bt, n, dim)), f("z", (Bt, n, dim)),
                               f("B", (Bt, n, G, N)), f("C", (Bt, n, G, N)), inp["A"], inp["D"], inp["dt_bias"])
    g = np.stack([host(y) for y in ys], axis=1)            # [Bt][steps][dim]
    for b in range(Bt):
        if dout == "f32":
            check_fp32(g[b], yo[b, L:], "step y b%d" % b)
        else:
            check_bf16_y(g[b], yo[b, L:], "step y b%d" % b)
        check_fp32(host(state[b]), ho[b], "state b%d" % b)
