"""GPU parity of the sliding-window attention layer (samba_rope, samba_swa_fwd, samba_swa_decode through the
C ABI) against the fp64 oracle (oracle_swa / oracle_rope, pinned in tests/test_oracle_swa_pins.py).

Both sides take the same bf16 q, k, v and the same RoPE table (fp64 for the oracle, its fp32 rounding for the
library).  The oracle rotates and attends in fp64; the library rotates in fp32, rounds the rotated q and k to
bf16 (samba_rope's output), forms scores from bf16 products with fp32 accumulation, scales them in fp32, and
feeds bf16 probabilities to the P.V product (the denominator sums those same bf16 values).

Tolerances:
  * RoPE: one bf16 rounding of the rotated value plus the fp32 roundings of the table and the products,
    |g - o| <= 2^-8 |o| + 2^-22 (|x[c]| + |x[c + hd/2]|);
  * attention entry points alone (q and k given in bf16, no RoPE): per (sequence, head)
    max|g - o| / max|o| <= CORE_TOL = 2e-3.  The only rounding left in the prefill is that of the bf16
    probabilities (relative 2^-9 each; the output is a convex combination of the values with weights perturbed
    by at most 2^-8 relative), measured 0.7-1.3e-3 with N(0, 1) inputs and scores four times larger; the
    decode keeps fp32 probabilities (error ~1e-7);
  * RoPE then attention, fp32 output: per (sequence, head) max|g - o| / max|o| <= ATT_TOL = 5e-3 for scores
    of unit size.  On top of the above, the bf16 rotated q and k (a relative 2^-9 per element each, i.e. a
    score error of about 2^-9 |q||k| / sqrt(d), random over the keys) move the output by sum_j p_j ds_j
    (v_j - o) to first order: the errors grow with the scores' size.  Measured 1.7-3.5e-3 with N(0, 1)
    inputs; scores four times larger get four times the tolerance (measured 8e-3).  A single decoded row
    over a 24-key window, normalised by its own largest element, averages over few keys: ROW_TOL = 1e-2
    there (measured up to 7.3e-3);
  * attention, bf16 output: one more bf16 rounding, |g - o| <= 2^-8 |o| + tol max|o|;
  * tripwires with exact arithmetic on the device: q = 0 (every visible key weighs exactly 1, so o is an
    fp32 mean of bf16 values: error ~1e-6) pins the window's edges and the sequence boundaries, and hard
    attention (one key scores ~300 above the rest) returns that key's value exactly.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as O
from selective_state_space_05_amd import inputs as I
from selective_state_space_05_amd import swa as W

pytestmark = pytest.mark.gpu
DEV = "cuda"
HD = 128
ATT_TOL = 5e-3
ROW_TOL = 1e-2
CORE_TOL = 2e-3
EXACT_TOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def tables(npos):
    c, s = I.rope_tables(npos, HD)
    return c, s, torch.from_numpy(c.astype(np.float32)).to(DEV), torch.from_numpy(s.astype(np.float32)).to(DEV)


def seq_bounds(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)


def check_att(g, o, bounds, what, out="f32", tol=ATT_TOL):
    """g, o [T][H][hd]; per (sequence, head) normalised error; bf16 adds one rounding per element."""
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    assert np.all(np.isfinite(g)), what + ": non-finite GPU output"
    worst = 0.0
    for a, b in zip(bounds[:-1], bounds[1:]):
        if b <= a:
            continue
        for h in range(o.shape[1]):
            oo, gg = o[a:b, h], g[a:b, h]
            scale = float(np.max(np.abs(oo)))
            if out == "f32":
                r = float(np.max(np.abs(gg - oo))) / max(scale, 1e-300) / tol
            else:
                r = float(np.max(np.abs(gg - oo) / (2.0 ** -8 * np.abs(oo) + tol * scale + 1e-300)))
            worst = max(worst, r)
    assert worst <= 1.0, "%s: error ratio %.3f over the tolerance" % (what, worst)
    return worst


def rope_bound(x, o):
    """One bf16 rounding of the rotated value, plus the fp32 rounding of the table and of the products
    (2^-23 relative to each term): |g - o| <= 2^-8 |o| + 2^-22 (|x[c]| + |x[c + hd/2]|)."""
    a = np.abs(np.asarray(x, np.float64))
    half = a.shape[-1] // 2
    pair = a[..., :half] + a[..., half:]
    return 2.0 ** -8 * np.abs(o) + 2.0 ** -22 * np.concatenate([pair, pair], axis=-1)


def run_rope(q, k, ct, st, lengths=None, pos0=None, in_place=False):
    cu = None if lengths is None else torch.from_numpy(I.cu_from_lengths(lengths)).to(DEV)
    return W.rope(q, k, ct, st, cu_seqlens=cu, pos0=pos0, in_place=in_place)


# --------------------------------------------------------------------------- #
# RoPE
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("lengths", [(300,), (1, 0, 129, 64, 7)])
def test_rope_matches_oracle(lengths):
    say("case: rope lengths", lengths)
    T, H = sum(lengths), 3
    inp = I.make_swa_inputs_np(6, T, H, HD)
    c, s, ct, st = tables(max(lengths))
    q, k = bf16_dev(inp["q"]), bf16_dev(inp["k"])
    qr, kr = run_rope(q, k, ct, st, lengths=list(lengths) if len(lengths) > 1 else None)
    torch.cuda.synchronize()
    b = seq_bounds(lengths)
    pos = np.concatenate([np.arange(b[i + 1] - b[i]) for i in range(len(lengths))]).astype(np.int64)
    for name, g in (("q", qr), ("k", kr)):
        o = O.rope(inp[name + "_f32"], c, s, pos)
        ratio = np.abs(host(g) - o) / rope_bound(inp[name + "_f32"], o)
        assert np.all(ratio <= 1.0), "rope %s: worst ratio %.3f" % (name, float(ratio.max()))
    # in place gives the same bits
    q2, k2 = q.clone(), k.clone()
    run_rope(q2, k2, ct, st, lengths=list(lengths) if len(lengths) > 1 else None, in_place=True)
    torch.cuda.synchronize()
    assert torch.equal(q2.view(torch.int16), qr.view(torch.int16)) and torch.equal(k2.view(torch.int16),
                                                                                   kr.view(torch.int16))


@pytest.mark.parametrize("H,hd", [(40, 64), (1, 16), (2, 1024)])
def test_rope_other_shapes(H, hd):
    """Head sizes other than 128 (RoPE accepts any multiple of 16) and more heads than one pass covers."""
    say("case: rope H%d hd%d" % (H, hd))
    T = 77
    g = np.random.default_rng(12)
    v = g.standard_normal((2, T, H, hd)).astype(np.float32)
    bits = [I.bf16_bits_from_f32(x) for x in v]
    c, s = I.rope_tables(T, hd)
    ct, st = (torch.from_numpy(x.astype(np.float32)).to(DEV) for x in (c, s))
    q, k = (bf16_dev(b).reshape(1, T, H, hd) for b in bits)
    qr, kr = W.rope(q, k, ct, st)
    torch.cuda.synchronize()
    for g_, b in ((qr, bits[0]), (kr, bits[1])):
        x = I.f32_from_bf16_bits(b)
        o = O.rope(x, c, s, np.arange(T))
        ratio = np.abs(host(g_).reshape(T, H, hd) - o) / rope_bound(x, o)
        assert np.all(ratio <= 1.0), "worst ratio %.3f" % float(ratio.max())


def test_rope_positions_offset():
    """A decode batch: one-token sequences at positions pos0[b] (and k only)."""
    B, H = 9, 4
    inp = I.make_swa_inputs_np(7, B, H, HD)
    pos = I.make_positions_np(7, B, 0, 5000)
    c, s, ct, st = tables(5001)
    k = bf16_dev(inp["k"]).reshape(B, 1, H, HD)
    _, kr = W.rope(None, k, ct, st, pos0=torch.from_numpy(pos).to(DEV))
    torch.cuda.synchronize()
    o = O.rope(inp["k_f32"], c, s, pos.astype(np.int64))
    ratio = np.abs(host(kr).reshape(B, H, HD) - o) / rope_bound(inp["k_f32"], o)
    assert np.all(ratio <= 1.0), "worst ratio %.3f" % float(ratio.max())


# --------------------------------------------------------------------------- #
# prefill attention
# --------------------------------------------------------------------------- #
PREFILL_CASES = [
    # (lengths or (batch, seqlen), heads, window, out)
    ("batch", (2, 300), 3, 64, "f32"),
    ("batch", (2, 300), 3, 64, "bf16"),
    ("batch", (1, 1000), 2, 2048, "f32"),     # window beyond the sequence: full causal attention
    ("batch", (1, 700), 2, 0, "f32"),         # each token sees itself only
    ("batch", (3, 129), 2, 100, "f32"),       # window not a multiple of the tile, ragged blocks
    ("varlen", (1, 0, 200, 128, 77, 513), 2, 130, "f32"),
    ("varlen", (640, 1, 255), 1, 127, "bf16"),
]


def prefill(case_kind, shape, H, window, out, q_scale=1.0, zero_q=False, cfg=6):
    if case_kind == "batch":
        batch, L = shape
        lengths = [L] * batch
    else:
        lengths = list(shape)
    T = sum(lengths)
    inp = I.make_swa_inputs_np(cfg, T, H, HD, q_scale=q_scale)
    if zero_q:
        inp["q"] = np.zeros_like(inp["q"])
        inp["q_f32"] = np.zeros_like(inp["q_f32"])
    c, s, ct, st = tables(max(max(lengths), 1))
    q, k, v = (bf16_dev(inp[n]) for n in ("q", "k", "v"))
    od = torch.float32 if out == "f32" else torch.bfloat16
    if case_kind == "batch":
        q, k, v = (t.reshape(batch, L, H, HD) for t in (q, k, v))
        o = W.attention(q, k, v, window, ct, st, out_dtype=od)
    else:
        cu = torch.from_numpy(I.cu_from_lengths(lengths)).to(DEV)
        o = W.attention(q, k, v, window, ct, st, cu_seqlens=cu, out_dtype=od)
    torch.cuda.synchronize()
    b = seq_bounds(lengths)
    oo = O.swa(inp["q_f32"], inp["k_f32"], inp["v_f32"], window, c, s, seq_start=b)
    return host(o).reshape(T, H, HD), oo, b


@pytest.mark.parametrize("kind,shape,H,window,out", PREFILL_CASES)
def test_swa_fwd_matches_oracle(kind, shape, H, window, out):
    say("case: swa_fwd", kind, shape, "H", H, "w", window, out)
    g, o, b = prefill(kind, shape, H, window, out)
    r = check_att(g, o, b, "swa_fwd", out=out)
    say("  error ratio %.3f" % r)


def prefill_core(case_kind, shape, H, window, out, q_scale=1.0):
    """samba_swa_fwd alone on bf16 q, k, v taken as already rotated, against the oracle's attention without
    RoPE on the same values."""
    if case_kind == "batch":
        batch, L = shape
        lengths = [L] * batch
    else:
        lengths = list(shape)
    T = sum(lengths)
    inp = I.make_swa_inputs_np(13, T, H, HD, q_scale=q_scale)
    q, k, v = (bf16_dev(inp[n]) for n in ("q", "k", "v"))
    od = torch.float32 if out == "f32" else torch.bfloat16
    if case_kind == "batch":
        q, k, v = (t.reshape(batch, L, H, HD) for t in (q, k, v))
        o = W.swa_fwd(q, k, v, window, out_dtype=od)
    else:
        cu = torch.from_numpy(I.cu_from_lengths(lengths)).to(DEV)
        o = W.swa_fwd(q, k, v, window, cu_seqlens=cu, out_dtype=od)
    torch.cuda.synchronize()
    b = seq_bounds(lengths)
    oo = O.swa(inp["q_f32"], inp["k_f32"], inp["v_f32"], window, seq_start=b)
    return host(o).reshape(T, H, HD), oo, b


@pytest.mark.parametrize("kind,shape,H,window,out", PREFILL_CASES)
def test_swa_fwd_core_matches_oracle(kind, shape, H, window, out):
    """The attention entry point on its own: q and k enter in bf16 as given, so the only roundings left are
    the bf16 probabilities of the P.V product and fp32 accumulation; held to CORE_TOL."""
    say("case: swa_fwd core", kind, shape, "H", H, "w", window, out)
    g, o, b = prefill_core(kind, shape, H, window, out)
    say("  error ratio %.3f" % check_att(g, o, b, "swa_fwd core", out=out, tol=CORE_TOL))


def test_swa_fwd_core_sharp_softmax():
    say("case: swa_fwd core sharp softmax")
    g, o, b = prefill_core("batch", (1, 600), 2, 200, "f32", q_scale=4.0)
    say("  error ratio %.3f" % check_att(g, o, b, "swa_fwd core sharp", tol=CORE_TOL))


def test_swa_fwd_sharp_softmax():
    """Scores ~N(0, 16): the maximum moves often and the probabilities span many orders of magnitude.  The
    rounding errors of the bf16 operands perturb each score in proportion to its size (to first order the
    output moves by sum_j p_j ds_j (v_j - o)), so scores four times larger get four times the tolerance."""
    say("case: swa_fwd sharp softmax")
    g, o, b = prefill("batch", (1, 600), 2, 200, "f32", q_scale=4.0)
    say("  error ratio %.3f" % check_att(g, o, b, "swa_fwd sharp", tol=4 * ATT_TOL))


@pytest.mark.parametrize("kind,shape,window", [("batch", (2, 333), 70), ("varlen", (5, 0, 260, 1, 130), 64),
                                               ("batch", (1, 300), 0)])
def test_swa_fwd_uniform_exact(kind, shape, window):
    """q = 0: every visible key has probability exactly 1 before normalisation; o is an fp32 mean."""
    say("case: swa_fwd uniform", kind, shape, window)
    g, o, b = prefill(kind, shape, 2, window, "f32", zero_q=True)
    r = check_att(g, o, b, "swa_fwd uniform", tol=EXACT_TOL)
    say("  error ratio %.3f" % r)


def test_swa_fwd_hard_attention_exact():
    """Query i carries 24 x (key j(i)), j(i) the oldest visible key: that key scores ~300 above the others."""
    say("case: swa_fwd hard attention")
    L, H, window = 400, 1, 90
    inp = I.make_swa_inputs_np(8, L, H, HD)
    k = inp["k_f32"].copy()
    q = np.zeros_like(k)
    tgt = np.maximum(np.arange(L) - window, 0)
    q[:, 0] = 24.0 * k[tgt, 0]
    qb = I.bf16_bits_from_f32(q.astype(np.float32))
    ident_c, ident_s = np.ones((L, HD // 2)), np.zeros((L, HD // 2))
    ct = torch.ones(L, HD // 2, device=DEV)
    st = torch.zeros(L, HD // 2, device=DEV)
    qd, kd, vd = bf16_dev(qb).reshape(1, L, H, HD), bf16_dev(inp["k"]).reshape(1, L, H, HD), bf16_dev(
        inp["v"]).reshape(1, L, H, HD)
    o = W.attention(qd, kd, vd, window, ct, st, out_dtype=torch.float32)
    torch.cuda.synchronize()
    oo = O.swa(I.f32_from_bf16_bits(qb), inp["k_f32"], inp["v_f32"], window, ident_c, ident_s)
    np.testing.assert_allclose(oo[:, 0], inp["v_f32"][tgt, 0], rtol=0, atol=1e-9)   # the oracle picks the key
    g = host(o).reshape(L, H, HD)
    r = check_att(g, oo, seq_bounds([L]), "swa_fwd hard", tol=EXACT_TOL)
    say("  error ratio %.3f" % r)


def test_swa_fwd_deterministic():
    L, H = 1000, 2
    inp = I.make_swa_inputs_np(9, L, H, HD)
    c, s, ct, st = tables(L)
    q, k, v = (bf16_dev(inp[n]).reshape(1, L, H, HD) for n in ("q", "k", "v"))
    o1 = W.attention(q, k, v, 300, ct, st)
    o2 = W.attention(q, k, v, 300, ct, st)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_swa_fwd_full_shape_sampled():
    """Samba-3.8B's attention on the training shape (4 x 4096 tokens, 24 heads of 128, window 2048), the
    launch the benchmark times; the oracle checks every head of sampled query rows (edges of tiles, blocks
    and of the window included)."""
    wl = I.WORKLOADS[6]
    B, L, H, w = wl.batch, wl.seqlen, wl.extra["heads"], wl.extra["window"]
    say("case: swa_fwd full shape B%d L%d H%d w%d" % (B, L, H, w))
    t = I.make_swa_inputs_torch(6, B * L, H, HD, DEV)
    c, s, ct, st = tables(L)
    q, k, v = (t[n].reshape(B, L, H, HD) for n in ("q", "k", "v"))
    o = W.attention(q, k, v, w, ct, st)
    torch.cuda.synchronize()
    rows_in_seq = [0, 1, 63, 64, 127, 128, 2047, 2048, 2049, 2111, 3000, 4095]
    for bi in range(B):
        qs, ks, vs = (host(x[bi]) for x in (q, k, v))
        oo = O.swa(qs, ks, vs, w, c, s, rows=rows_in_seq)
        g = host(o[bi])
        for r in rows_in_seq:
            scale = np.max(np.abs(oo[r]), axis=-1, keepdims=True)
            bound = 2.0 ** -8 * np.abs(oo[r]) + ATT_TOL * scale
            assert np.all(np.abs(g[r] - oo[r]) <= bound), "row %d of sequence %d" % (r, bi)
    say("  ok")


# --------------------------------------------------------------------------- #
# decode step
# --------------------------------------------------------------------------- #
def fill_cache(kr_seq, v_seq, pos, cache_len, kc, vc, b):
    """Ring slots p % cache_len of sequence b for positions max(0, pos - cache_len + 1) .. pos - 1."""
    for p in range(max(0, pos - cache_len + 1), pos):
        kc[b, :, p % cache_len] = kr_seq[p]
        vc[b, :, p % cache_len] = v_seq[p]


@pytest.mark.parametrize("window,cache_len,out", [(40, 41, "f32"), (40, 57, "bf16"), (0, 1, "f32"),
                                                  (300, 301, "f32")])
def test_swa_decode_matches_oracle(window, cache_len, out):
    say("case: swa_decode w%d cache %d %s" % (window, cache_len, out))
    H = 2
    pos = np.array([0, 5, 40, 41, 100, 333], dtype=np.int32)
    B = len(pos)
    od = torch.float32 if out == "f32" else torch.bfloat16
    c, s, ct, st = tables(int(pos.max()) + 1)
    kc = torch.zeros(B, H, cache_len, HD, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    qn, kn, vn, want = [], [], [], []
    for b in range(B):
        n = int(pos[b]) + 1
        inp = I.make_swa_inputs_np(100 + b, n, H, HD)
        qd, kd, vd = (bf16_dev(inp[x]).reshape(1, n, H, HD) for x in ("q", "k", "v"))
        qr, kr = W.rope(qd, kd, ct, st)
        fill_cache(kr[0], vd[0], n - 1, cache_len, kc, vc, b)
        qn.append(qr[0, n - 1])
        kn.append(kr[0, n - 1])
        vn.append(vd[0, n - 1])
        oo = O.swa(inp["q_f32"], inp["k_f32"], inp["v_f32"], window, c, s, rows=[n - 1])
        want.append(oo[n - 1])
    qn, kn, vn = (torch.stack(x).contiguous() for x in (qn, kn, vn))
    o = W.swa_decode(qn, kn, vn, kc, vc, torch.from_numpy(pos).to(DEV), window, out_dtype=od)
    torch.cuda.synchronize()
    want = np.stack(want)
    r = check_att(host(o).reshape(B, H, HD), want, np.arange(B + 1), "swa_decode", out=out)
    say("  error ratio %.3f" % r)
    # the new token went into its ring slot
    for b in range(B):
        slot = int(pos[b]) % cache_len
        assert torch.equal(kc[b, :, slot].view(torch.int16), kn[b].view(torch.int16))
        assert torch.equal(vc[b, :, slot].view(torch.int16), vn[b].view(torch.int16))


def test_swa_decode_core_matches_oracle():
    """The decode entry point on its own: q, k and the cache hold bf16 values taken as already rotated; the
    probabilities stay fp32, so only fp32 rounding is left."""
    say("case: swa_decode core")
    H, window, cache_len = 2, 40, 57
    pos = np.array([0, 5, 40, 41, 100, 333], dtype=np.int32)
    B = len(pos)
    kc = torch.zeros(B, H, cache_len, HD, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    qn, kn, vn, want = [], [], [], []
    for b in range(B):
        n = int(pos[b]) + 1
        inp = I.make_swa_inputs_np(200 + b, n, H, HD)
        qd, kd, vd = (bf16_dev(inp[x]).reshape(n, H, HD) for x in ("q", "k", "v"))
        fill_cache(kd, vd, n - 1, cache_len, kc, vc, b)
        qn.append(qd[n - 1])
        kn.append(kd[n - 1])
        vn.append(vd[n - 1])
        want.append(O.swa(inp["q_f32"], inp["k_f32"], inp["v_f32"], window, rows=[n - 1])[n - 1])
    qn, kn, vn = (torch.stack(x).contiguous() for x in (qn, kn, vn))
    o = W.swa_decode(qn, kn, vn, kc, vc, torch.from_numpy(pos).to(DEV), window, out_dtype=torch.float32)
    torch.cuda.synchronize()
    r = check_att(host(o).reshape(B, H, HD), np.stack(want), np.arange(B + 1), "swa_decode core", tol=CORE_TOL)
    say("  error ratio %.3f" % r)


def test_swa_decode_steps_continue_prefill():
    """Prefill 50 tokens, fill the ring from the prefill's rotated keys, then 12 decode steps; every step's
    output against the oracle's row of the whole sequence (the ring wraps during the steps)."""
    H, window, cache_len, P, steps = 2, 24, 25, 50, 12
    n = P + steps
    inp = I.make_swa_inputs_np(11, n, H, HD)
    c, s, ct, st = tables(n)
    q, k, v = (bf16_dev(inp[x]).reshape(1, n, H, HD) for x in ("q", "k", "v"))
    qr, kr = W.rope(q, k, ct, st)
    kc = torch.zeros(1, H, cache_len, HD, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    fill_cache(kr[0], v[0], P, cache_len, kc, vc, 0)
    oo = O.swa(inp["q_f32"], inp["k_f32"], inp["v_f32"], window, c, s, rows=list(range(P, n)))
    for t in range(P, n):
        pos = torch.tensor([t], dtype=torch.int32, device=DEV)
        o = W.swa_decode(qr[0, t:t + 1].contiguous(), kr[0, t:t + 1].contiguous(), v[0, t:t + 1].contiguous(), kc,
                         vc, pos, window, out_dtype=torch.float32)
        torch.cuda.synchronize()
        check_att(host(o).reshape(1, H, HD), oo[t:t + 1], np.array([0, 1]), "decode step %d" % t, tol=ROW_TOL)


def test_swa_decode_full_shape_sampled():
    """64 sequences x 24 heads at position 4096 with a full 2049-slot ring (the benchmark's launch);
    sampled sequences checked against the oracle's last row of their window."""
    wl = I.WORKLOADS[7]
    B, H, w, cl, P = wl.batch, wl.extra["heads"], wl.extra["window"], wl.extra["cache_len"], wl.extra["pos"]
    say("case: swa_decode full shape B%d H%d w%d" % (B, H, w))
    c, s, ct, st = tables(P + 1)
    n = w + 1                                   # the window's tokens, positions P - w .. P
    t = I.make_swa_inputs_torch(7, B * n, H, HD, DEV)
    q, k, v = (t[x].reshape(B, n, H, HD) for x in ("q", "k", "v"))
    pos0 = torch.full((B,), P - w, dtype=torch.int32, device=DEV)
    qr, kr = W.rope(q, k, ct, st, pos0=pos0)
    kc = torch.empty(B, H, cl, HD, dtype=torch.bfloat16, device=DEV)
    vc = torch.empty_like(kc)
    slots = torch.arange(P - w, P, device=DEV) % cl
    kc[:, :, slots] = kr[:, :n - 1].permute(0, 2, 1, 3)
    vc[:, :, slots] = v[:, :n - 1].permute(0, 2, 1, 3)
    pos = torch.full((B,), P, dtype=torch.int32, device=DEV)
    o = W.swa_decode(qr[:, n - 1].contiguous(), kr[:, n - 1].contiguous(), v[:, n - 1].contiguous(), kc, vc, pos, w)
    torch.cuda.synchronize()
    cs, sn = c[P - w:], s[P - w:]               # table rows of positions P - w .. P
    for bi in (0, 17, 63):
        oo = O.swa(host(q[bi]), host(k[bi]), host(v[bi]), w, cs, sn, rows=[n - 1])[n - 1]
        g = host(o[bi])
        scale = np.max(np.abs(oo), axis=-1, keepdims=True)
        assert np.all(np.abs(g - oo) <= 2.0 ** -8 * np.abs(oo) + ATT_TOL * scale), "sequence %d" % bi
    say("  ok")
