"""Pins of the oracle's state-space duality layer (oracle_ssd): the Mamba-2 form that the pages compare Samba
with (page "SAMBA混合注意力状态空间模型", 与其他混合架构对比: SSD and its duality, no formula given).

The oracle writes the layer as its recurrence (a scalar decay per head, a P x N state per head).  Pins:
  * the dual, quadratic form (an independent formulation: one masked L x L matrix per head,
    M[t][s] = exp(A (S_t - S_s)) (C_t . B_s) Δ_s for s <= t, with S the running sum of Δ, applied to x);
  * when every state of a channel shares the head's A and Δ, the layer is the grouped selective scan over
    dim = heads * P channels, each head's P channels reading its group's (B, C);
  * carrying h_last into h0 over a split, packed sequences against separate calls, batched rows against
    packed ones;
  * planted mistakes in the recurrence and its indexing are rejected by the quadratic form;
  * with a unit step (Δ = 1) and A = ln γ per head the layer is multi-scale retention, checked against the
    retention's parallel form.
"""
import shutil

import numpy as np
import pytest
from scipy.special import expit

from oracle import oracle as O
from tests.test_oracle_pins import rel_err


def ssd_case(seed, L, H, P, G, N, h0_scale=0.0, gate=True):
    g = np.random.default_rng(seed)
    x = g.standard_normal((L, H, P))
    z = g.standard_normal((L, H, P)) if gate else None
    dt = g.standard_normal((L, H))
    B, C = g.standard_normal((L, G, N)), g.standard_normal((L, G, N))
    bias = np.log(np.expm1(g.uniform(1e-3, 1e-1, H)))
    A = -np.exp(g.uniform(0, np.log(16), H))
    Dv = g.uniform(0, 1, H)
    h0 = h0_scale * g.standard_normal((H, P, N)) if h0_scale else None
    return dict(x=x, dt=dt, z=z, B=B, C=C, A=A, Dv=Dv, bias=bias, h0=h0)


def run(c, lib=None, seq_start=None):
    h0 = None if c["h0"] is None else c["h0"][None]
    return O.ssd(c["x"], c["dt"], c["B"], c["C"], c["A"], c["Dv"], c["bias"], z=c["z"], h0=h0,
                 seq_start=seq_start, lib=lib)


def quadratic_form(c):
    """y = silu(z) * (M x + exp(A S_t) C_t H0^T + D x) per head, with the L x L matrix M above."""
    x, dt, B, C = c["x"], c["dt"], c["B"], c["C"]
    L, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    y = np.zeros((L, H, P))
    h_last = np.zeros((H, P, N))
    for h in range(H):
        g = h // (H // G)
        delta = np.logaddexp(0.0, dt[:, h] + c["bias"][h])
        S = np.cumsum(delta)                                         # S_t = sum_{r<=t} Δ_r
        seg = S[:, None] - S[None, :]                                # S_t - S_s
        mask = np.tril(np.ones((L, L), dtype=bool))
        decay = np.where(mask, np.exp(np.where(mask, c["A"][h] * seg, 0.0)), 0.0)
        M = decay * (C[:, g] @ B[:, g].T) * delta[None, :]
        yh = M @ x[:, h] + c["Dv"][h] * x[:, h]
        w = np.exp(c["A"][h] * (S[-1] - S)) * delta                  # weight of token s in the final state
        h_last[h] = (x[:, h] * w[:, None]).T @ B[:, g]
        if c["h0"] is not None:
            yh += np.exp(c["A"][h] * S)[:, None] * (C[:, g] @ c["h0"][h].T)
            h_last[h] += np.exp(c["A"][h] * S[-1]) * c["h0"][h]
        y[:, h] = yh * (c["z"][:, h] * expit(c["z"][:, h]) if c["z"] is not None else 1.0)
    return y, h_last


@pytest.mark.parametrize("seed,L,H,P,G,N,h0s,gate", [(1, 23, 2, 3, 1, 4, 0.0, True), (2, 31, 4, 2, 2, 8, 1.0, True),
                                                     (3, 17, 3, 5, 3, 16, 0.5, False), (4, 12, 2, 4, 1, 64, 1.0, True),
                                                     (5, 40, 6, 2, 2, 3, 2.0, False)])
def test_quadratic_form(oracle_lib, seed, L, H, P, G, N, h0s, gate):
    c = ssd_case(seed, L, H, P, G, N, h0s, gate)
    y, hl = run(c, oracle_lib)
    yq, hq = quadratic_form(c)
    assert rel_err(y, yq) < 1e-11
    assert rel_err(hl[0], hq) < 1e-11


def test_hand_worked_scalar(oracle_lib):
    """One head, P = N = 1, Δ = softplus(0 + log(e - 1)) = 1, A = -log 2 so a = 1/2, B = C = 1, D = 0, no gate:
    h_t = h_{t-1} / 2 + x_t and y_t = h_t.  x = (1, 0, 2, 0) gives h = (1, 1/2, 9/4, 9/8)."""
    c = dict(x=np.array([1.0, 0, 2, 0]).reshape(4, 1, 1), dt=np.zeros((4, 1)), z=None,
             B=np.ones((4, 1, 1)), C=np.ones((4, 1, 1)), A=np.array([-np.log(2.0)]), Dv=np.zeros(1),
             bias=np.array([np.log(np.e - 1.0)]), h0=None)
    y, hl = run(c, oracle_lib)
    np.testing.assert_allclose(y.ravel(), [1.0, 0.5, 2.25, 1.125], rtol=1e-14)
    np.testing.assert_allclose(hl.ravel(), [1.125], rtol=1e-14)


def test_equals_grouped_scan_with_shared_decay(oracle_lib):
    L, H, P, G, N = 29, 4, 3, 2, 16
    c = ssd_case(6, L, H, P, G, N, 1.0)
    y, hl = run(c, oracle_lib)
    dim = H * P
    yg, hg = O.scan_fwd_groups(c["x"].reshape(L, dim), np.repeat(c["dt"], P, axis=1), c["z"].reshape(L, dim),
                               c["B"], c["C"], np.repeat(c["A"], P)[:, None] * np.ones((1, N)),
                               np.repeat(c["Dv"], P), np.repeat(c["bias"], P),
                               h0=c["h0"].reshape(1, dim, N), lib=oracle_lib)
    assert rel_err(y.reshape(L, dim), yg) < 1e-13
    assert rel_err(hl.reshape(dim, N), hg[0]) < 1e-13


def test_split_carries_state(oracle_lib):
    c = ssd_case(7, 37, 2, 4, 1, 8, 1.0)
    y, hl = run(c, oracle_lib)
    k = 15
    first = {key: (v[:k] if key in ("x", "dt", "z", "B", "C") else v) for key, v in c.items()}
    second = {key: (v[k:] if key in ("x", "dt", "z", "B", "C") else v) for key, v in c.items()}
    y1, h1 = run(first, oracle_lib)
    second["h0"] = h1[0]
    y2, h2 = run(second, oracle_lib)
    assert rel_err(np.concatenate([y1, y2]), y) < 1e-13
    assert rel_err(h2, hl) < 1e-13


def test_packed_equals_separate_and_batched(oracle_lib):
    lens = [9, 1, 14, 6]
    H, P, G, N = 4, 2, 2, 8
    parts = [ssd_case(20 + i, n, H, P, G, N, 1.0) for i, n in enumerate(lens)]
    cat = {k: np.concatenate([p[k] for p in parts]) for k in ("x", "dt", "z", "B", "C")}
    packed = dict(parts[0], **cat)
    seq_start = np.concatenate([[0], np.cumsum(lens)])
    h0 = np.stack([p["h0"] for p in parts])
    for p in parts[1:]:
        p.update(A=parts[0]["A"], Dv=parts[0]["Dv"], bias=parts[0]["bias"])
    y, hl = O.ssd(packed["x"], packed["dt"], packed["B"], packed["C"], packed["A"], packed["Dv"], packed["bias"],
                  z=packed["z"], h0=h0, seq_start=seq_start, lib=oracle_lib)
    for i, p in enumerate(parts):
        yi, hi = run(p, oracle_lib)
        np.testing.assert_array_equal(y[seq_start[i]:seq_start[i + 1]], yi)
        np.testing.assert_array_equal(hl[i], hi[0])
    # equal-length rows given as [batch][L][H][P] are the same packed sequences
    eq = [ssd_case(40 + i, 7, H, P, G, N, 1.0) for i in range(3)]
    for p in eq[1:]:
        p.update(A=eq[0]["A"], Dv=eq[0]["Dv"], bias=eq[0]["bias"])
    st = lambda k: np.stack([p[k] for p in eq])
    yb, hb = O.ssd(st("x"), st("dt"), st("B"), st("C"), eq[0]["A"], eq[0]["Dv"], eq[0]["bias"], z=st("z"),
                   h0=st("h0"), lib=oracle_lib)
    for i, p in enumerate(eq):
        yi, hi = run(p, oracle_lib)
        np.testing.assert_array_equal(yb[i], yi)
        np.testing.assert_array_equal(hb[i], hi[0])


def test_rejects_heads_not_multiple_of_groups(oracle_lib):
    c = ssd_case(8, 4, 3, 2, 2, 4)
    with pytest.raises(Exception):
        run(c, oracle_lib)


SSD_MUTANTS = {
    "interleaved_groups": ("const int64_t g = h / (H / G);", "const int64_t g = h % G;"),
    "no_delta_on_input": ("a * st[p * N + n] + delta * xt[p] * Bt[n];", "a * st[p * N + n] + xt[p] * Bt[n];"),
    "readout_before_update": ("st[p * N + n] = a * st[p * N + n] + delta * xt[p] * Bt[n];\n            acc += st[p * N + n] * Ct[n];",
                              "acc += st[p * N + n] * Ct[n];\n            st[p * N + n] = a * st[p * N + n] + delta * xt[p] * Bt[n];"),
    "transposed_state": ("st[p * N + n] = a * st[p * N + n]", "st[p * N + n] = a * st[(n * P + p) % (P * N)]"),
    "h0_of_first_sequence": ("st[k] = h0 ? h0[(s * H + h) * P * N + k] : 0.0;",
                             "st[k] = h0 ? h0[(0 * H + h) * P * N + k] : 0.0;"),
    "skip_from_other_head": ("D[h] * xt[p]", "D[(h + 1) % H] * xt[p]"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(SSD_MUTANTS))
def test_ssd_mutant_is_caught(tmp_path, name):
    src = O.SRC.read_text()
    old, new = SSD_MUTANTS[name]
    assert src.count(old) == 1, "mutation anchor missing or ambiguous in oracle.c: " + name
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / ("lib_%s.so" % name)
    O.build(force=True, src=path, out=so)
    lib = O.load(so)
    lens = [9, 5]
    parts = [ssd_case(50 + i, n, 4, 3, 2, 5, 1.0) for i, n in enumerate(lens)]
    c = dict(parts[0], **{k: np.concatenate([p[k] for p in parts]) for k in ("x", "dt", "z", "B", "C")})
    seq_start = np.array([0, 9, 14])
    h0 = np.stack([p["h0"] for p in parts])
    y, hl = O.ssd(c["x"], c["dt"], c["B"], c["C"], c["A"], c["Dv"], c["bias"], z=c["z"], h0=h0,
                  seq_start=seq_start, lib=lib)
    bad = False
    for i, p in enumerate(parts):
        p.update(A=c["A"], Dv=c["Dv"], bias=c["bias"])
        yq, hq = quadratic_form(p)
        bad |= rel_err(y[seq_start[i]:seq_start[i + 1]], yq) > 1e-6 or rel_err(hl[i], hq) > 1e-6
    assert bad, "quadratic form did not reject mutant " + name


def retention_parallel(q, k, v, gammas):
    """Multi-scale retention in its parallel form (the hackernoon page "Microsoft's Samba Model Redefines
    Long-Context Learning for AI", §2, names Multi-Scale Retention and GLA as substitutes for the Mamba
    layer; the form is the retention paper's): per head, O = (Q Kᵀ ∘ Γ) V with Γ[t][s] = γ^(t - s), s <= t."""
    L, H, _ = v.shape
    o = np.zeros_like(v)
    idx = np.arange(L)
    for h in range(H):
        gam = np.where(idx[:, None] >= idx[None, :], gammas[h] ** (idx[:, None] - idx[None, :]).astype(float), 0.0)
        o[:, h] = ((q[:, h] @ k[:, h].T) * gam) @ v[:, h]
    return o


def test_retention_is_ssd_with_unit_step():
    """Δ = softplus(0 + ln(e - 1)) = 1 and A = ln γ make the layer multi-scale retention: state S_t =
    γ S_{t-1} + k_t v_tᵀ read out by q_t (B = k, C = q per head, x = v, no skip, no gate), with RetNet's
    decays γ_h = 1 - 2^(-5-h)."""
    g = np.random.default_rng(60)
    L, H, P, N = 45, 4, 3, 5
    q, k = g.standard_normal((L, H, N)), g.standard_normal((L, H, N))
    v = g.standard_normal((L, H, P))
    gammas = 1.0 - 2.0 ** (-5.0 - np.arange(H))
    y, _ = O.ssd(v, np.zeros((L, H)), k, q, np.log(gammas), np.zeros(H), np.full(H, np.log(np.e - 1.0)))
    assert rel_err(y, retention_parallel(q, k, v, gammas)) < 1e-12


def test_golden_regression_ssd_and_gla(oracle_lib):
    """Regression fixture written by tests/golden/make_golden.py from oracle/ only (catches accidental changes
    to the oracle; the pins above are what tie it to the definitions)."""
    import json
    from pathlib import Path
    data = json.loads((Path(__file__).resolve().parent / "golden" / "oracle_variants_small.json").read_text())
    ss = np.array(data["seq_start"], dtype=np.int64)
    a = {k: np.array(v, dtype=np.float64) for k, v in data["ssd"]["inputs"].items()}
    y, h = O.ssd(a["x"], a["dt"], a["B"], a["C"], a["A"], a["D"], a["dt_bias"], z=a["z"], h0=a["h0"], seq_start=ss,
                 lib=oracle_lib)
    assert rel_err(y, np.array(data["ssd"]["y"])) < 1e-13 and rel_err(h, np.array(data["ssd"]["h_last"])) < 1e-13
    g = {k: np.array(v, dtype=np.float64) for k, v in data["gla"]["inputs"].items()}
    o, hg = O.gla(g["q"], g["k"], g["v"], g["gk"], h0=g["h0"], seq_start=ss, lib=oracle_lib)
    assert rel_err(o, np.array(data["gla"]["o"])) < 1e-13 and rel_err(hg, np.array(data["gla"]["h_last"])) < 1e-13
