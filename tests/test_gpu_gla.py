"""GPU parity of gated linear attention (samba_gla_fwd through the C ABI) against the fp64 oracle (oracle_gla,
pinned in tests/test_oracle_gla_pins.py).

Tolerance reading as for the selective scan (tests/parity.py): the recurrence runs in fp32 (no bf16
products), and the chunked form feeds the matrix cores bf16 hi + lo pairs (16 significant bits) for every
operand that is not an input, so fp32 outputs per sequence meet the 2e-3 contract and the 1e-4 tripwire;
bf16 o gets one bf16 rounding on top per (sequence, column).  Cases: every key size (16 .. 256), fp32 and bf16 inputs and
outputs, h0 given and h_last written in place over it, packed sequences with empty ones, ragged chunks,
strongly decaying gates, a chained call, determinism, and the benchmark's shape (B4 L4096, 4 heads, keys
256, values 512) on sampled value columns of every head; each in the recurrent and the chunked form.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as O
from selective_state_space_05_amd import gla as G
from selective_state_space_05_amd import inputs as I
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
    # lengths, heads, N (keys), P (values), in, out, h0
    ((100,), 2, 16, 64, "bf16", "f32", True),
    ((77, 77), 2, 64, 16, "bf16", "bf16", False),
    ((0, 41, 1, 0, 64), 2, 32, 32, "bf16", "f32", True),
    ((50,), 1, 256, 16, "f32", "f32", True),
    ((33, 33, 33), 3, 128, 16, "bf16", "f32", True),
    ((130,), 2, 256, 32, "bf16", "bf16", True),
    # the chunked form (bf16 inputs, 128 or 256 keys, values a multiple of 32): 64-token chunks
    ((64, 0, 129, 1, 200), 2, 128, 32, "bf16", "f32", True),
    ((65,), 3, 256, 64, "bf16", "f32", True),
    ((300,), 1, 128, 96, "bf16", "bf16", False),
    ((128, 128), 2, 256, 32, "bf16", "f32", False),
]


def run_case(lengths, H, N, P, din, dout, with_h0, cfg=10, gk_scale=1.0):
    T = sum(lengths)
    nseq = len(lengths)
    inp = I.make_gla_inputs_np(cfg, T, H, N, P, in_dtype=din)
    if not np.all(np.asarray(gk_scale) == 1.0):
        g = (inp["gk_f32"] * np.asarray(gk_scale, dtype=np.float32)).astype(np.float32)
        inp["gk"] = I.bf16_bits_from_f32(g) if din == "bf16" else g
        inp["gk_f32"] = I.f32_from_bf16_bits(inp["gk"]) if din == "bf16" else g
    h0 = (0.5 * np.random.default_rng(cfg).standard_normal((nseq, H, P, N))).astype(np.float32) if with_h0 else None
    packed = len(set(lengths)) > 1 or 0 in lengths
    q, k, gk, v = (dev(inp[n], din) for n in ("q", "k", "gk", "v"))
    od = torch.float32 if dout == "f32" else torch.bfloat16
    h0d = None if h0 is None else torch.from_numpy(h0).to(DEV)
    cu = torch.from_numpy(I.cu_from_lengths(lengths)).to(DEV) if packed else None
    if not packed:
        L = lengths[0]
        q, k, gk = (t.reshape(nseq, L, H, N) for t in (q, k, gk))
        v = v.reshape(nseq, L, H, P)
    o, hl = G.gla_fwd(q, k, v, gk, h0=h0d, h_last=h0d, y_dtype=od, cu_seqlens=cu)
    torch.cuda.synchronize()
    bounds = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    oo, ho = O.gla(inp["q_f32"], inp["k_f32"], inp["v_f32"], inp["gk_f32"], h0=h0, seq_start=bounds)
    return host(o).reshape(T, H * P), oo.reshape(T, H * P), host(hl), ho, bounds


def check(o, oo, hl, ho, b, dout):
    eo = check_fp32(o, oo, "o", b) if dout == "f32" else check_bf16_y(o, oo, "o", b)
    eh = 0.0
    for s in range(len(b) - 1):
        eh = max(eh, check_fp32(hl[s], ho[s], "h_last s%d" % s))
    say("  o %.2e h_last %.2e" % (eo, eh))


@pytest.mark.parametrize("lengths,H,N,P,din,dout,with_h0", CASES)
def test_gla_matches_oracle(lengths, H, N, P, din, dout, with_h0):
    say("case: gla", lengths, "heads", H, "N", N, "P", P, din, dout, "h0" if with_h0 else "")
    check(*run_case(lengths, H, N, P, din, dout, with_h0), dout)


@pytest.mark.parametrize("N,P,scale", [(64, 16, 16.0), (256, 32, 16.0), (128, 32, 120.0), (256, 32, 120.0)])
def test_gla_strong_decay(N, P, scale):
    """Gates 16x the recipe's (decays down to ~e^-3 per token): the state forgets within a few tokens, and in
    the chunked form the decay across a 64-token chunk spans tens of e-folds.  At 120x a 32-token half spans
    more than the 64 e-folds across which the intra-chunk matrix is formed from factored decays, so those
    blocks take the exact term-by-term form."""
    say("case: gla strong decay N%d P%d x%g" % (N, P, scale))
    o, oo, hl, ho, b = run_case((150,), 2, N, P, "bf16", "f32", True, gk_scale=scale)
    check(o, oo, hl, ho, b, "f32")


@pytest.mark.parametrize("wide", ["first", "second"])
def test_gla_strong_decay_in_one_key_pass(wide):
    """Keys 256 in the chunked form go through in two passes of 128; gates 120x the recipe's on one pass's keys
    only, so that pass takes the exact form of the diagonal blocks of A and the other the factored one."""
    say("case: gla strong decay on the %s 128 keys" % wide)
    scale = np.ones(256, dtype=np.float32)
    scale[slice(0, 128) if wide == "first" else slice(128, 256)] = 120.0
    o, oo, hl, ho, b = run_case((150,), 2, 256, 32, "bf16", "f32", True, gk_scale=scale)
    check(o, oo, hl, ho, b, "f32")


@pytest.mark.parametrize("N,P,L1,L2", [(128, 16, 45, 38), (256, 32, 70, 60)])
def test_gla_chained_and_deterministic(N, P, L1, L2):
    say("case: gla chained N%d P%d" % (N, P))
    H = 2
    inp = I.make_gla_inputs_np(11, L1 + L2, H, N, P)
    q, k, gk, v = (dev(inp[n], "bf16") for n in ("q", "k", "gk", "v"))
    o, hl = G.gla_fwd(q, k, v, gk, y_dtype=torch.float32)
    o1, h1 = G.gla_fwd(q[:L1], k[:L1], v[:L1], gk[:L1], y_dtype=torch.float32)
    o2, h2 = G.gla_fwd(q[L1:], k[L1:], v[L1:], gk[L1:], h0=h1, y_dtype=torch.float32)
    o3, h3 = G.gla_fwd(q, k, v, gk, y_dtype=torch.float32)
    torch.cuda.synchronize()
    oo, ho = O.gla(inp["q_f32"], inp["k_f32"], inp["v_f32"], inp["gk_f32"])
    T = L1 + L2
    check_fp32(host(torch.cat([o1, o2])).reshape(T, -1), oo.reshape(T, -1), "chained o")
    check_fp32(host(h2), ho, "chained h_last")
    check_fp32(host(o).reshape(T, -1), oo.reshape(T, -1), "one-pass o")
    assert torch.equal(o, o3) and torch.equal(hl, h3)


def test_gla_full_shape_sampled():
    """B4 L4096, 4 heads, keys 256, values 512 (the benchmark's launch): 8 value columns of every head of two
    sequences against the oracle (value columns are independent recurrences)."""
    wl = I.WORKLOADS[10]
    Bt, L, H, N, P = wl.batch, wl.seqlen, wl.extra["heads"], wl.dstate, wl.extra["head_dim"]
    say("case: gla full shape B%d L%d H%d N%d P%d" % (Bt, L, H, N, P))
    t = I.make_gla_inputs_torch(10, Bt * L, H, N, P, DEV)
    q, k, gk = (t[n].view(Bt, L, H, N) for n in ("q", "k", "gk"))
    v = t["v"].view(Bt, L, H, P)
    o, hl = G.gla_fwd(q, k, v, gk)
    torch.cuda.synchronize()
    for s in (0, 3):
        for h in range(H):
            c0 = (97 * (h + 1) + 13 * s) % (P - 8)
            cols = slice(c0, c0 + 8)
            oo, ho = O.gla(host(q[s, :, h:h + 1]), host(k[s, :, h:h + 1]), host(v[s, :, h:h + 1, cols]),
                           host(gk[s, :, h:h + 1]))
            check_bf16_y(host(o[s, :, h, cols]), oo[:, 0], "o s%d h%d" % (s, h))
            check_fp32(host(hl[s, h, cols]), ho[0, 0], "h_last s%d h%d" % (s, h))
    say("  ok")


@pytest.mark.parametrize("N,P", [(64, 16), (128, 32)])
def test_gla_no_tokens_carries_h0(N, P):
    say("case: gla no tokens N%d P%d" % (N, P))
    H = 2
    h0 = torch.from_numpy((0.5 * np.random.default_rng(13).standard_normal((3, H, P, N))).astype(np.float32)).to(DEV)
    q = torch.zeros(3, 0, H, N, dtype=torch.bfloat16, device=DEV)
    v = torch.zeros(3, 0, H, P, dtype=torch.bfloat16, device=DEV)
    _, hl = G.gla_fwd(q, q, v, q, h0=h0)
    torch.cuda.synchronize()
    assert torch.equal(hl, h0)


def test_gla_one_past_a_chunk():
    """17 and 33 tokens at 256 keys (16-token chunks) and 9 at 32 keys (8-token chunks) in the recurrence;
    65 and 1 tokens in the chunked form (64-token chunks)."""
    for L, N, P in ((17, 256, 16), (33, 256, 16), (9, 32, 32), (65, 256, 32), (1, 128, 32)):
        say("case: gla L%d N%d" % (L, N))
        check(*run_case((L,), 2, N, P, "bf16", "f32", True), "f32")
