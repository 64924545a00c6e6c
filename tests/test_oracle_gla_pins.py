"""Pins of the oracle's gated linear attention (oracle_gla): the hackernoon page "Microsoft's Samba Model
Redefines Long-Context Learning for AI", §2, names GLA (with Multi-Scale Retention) as a substitute for the
Mamba layer; the recurrence is the GLA paper's, S_t = diag(exp(gk_t)) S_{t-1} + k_tᵀ v_t, o_t = q_t S_t.

Pins:
  * the parallel form (an independent formulation): o_t = sum_{s<=t} (q_t ∘ exp(G_t - G_s)) · k_s v_s with G
    the running sum of gk per key dimension, plus the carried state's term;
  * constant gates are retention: gk = ln γ per head equals oracle_ssd's retention configuration;
  * gates that depend on the key dimension only are the grouped selective scan with a unit step (A = gk,
    B = k, C = q, x = v; the scan's silu gate divided out);
  * split with h_last -> h0, packed = separate, batched rows = packed;
  * planted mistakes in the recurrence and its indexing are rejected by the parallel form.
"""
import shutil

import numpy as np
import pytest
from scipy.special import expit

from oracle import oracle as O
from tests.test_oracle_pins import rel_err


def gla_case(seed, L, H, P, N, h0_scale=0.0):
    g = np.random.default_rng(seed)
    q, k = g.standard_normal((L, H, N)), g.standard_normal((L, H, N))
    v = g.standard_normal((L, H, P))
    gk = np.log(expit(g.standard_normal((L, H, N)) + 3.0))      # decays in (0, 1), mostly close to 1
    h0 = h0_scale * g.standard_normal((H, P, N)) if h0_scale else None
    return dict(q=q, k=k, v=v, gk=gk, h0=h0)


def run(c, lib=None, seq_start=None):
    h0 = None if c["h0"] is None else c["h0"][None]
    return O.gla(c["q"], c["k"], c["v"], c["gk"], h0=h0, seq_start=seq_start, lib=lib)


def parallel_form(c):
    q, k, v, gk = c["q"], c["k"], c["v"], c["gk"]
    L, H, P = v.shape
    G = np.cumsum(gk, axis=0)                                   # G_t = sum_{r<=t} gk_r
    o = np.zeros((L, H, P))
    hl = np.zeros((H, P, k.shape[2]))
    for h in range(H):
        for t in range(L):
            w = q[t, h][None, :] * np.exp(G[t, h][None, :] - G[: t + 1, h])   # [s][n]
            o[t, h] = ((w * k[: t + 1, h]).sum(axis=1)) @ v[: t + 1, h]
            if c["h0"] is not None:
                o[t, h] += c["h0"][h] @ (q[t, h] * np.exp(G[t, h]))
        dec = np.exp(G[-1, h][None, :] - G[:, h])                              # [s][n]
        hl[h] = v[:, h].T @ (dec * k[:, h])
        if c["h0"] is not None:
            hl[h] += c["h0"][h] * np.exp(G[-1, h])[None, :]
    return o, hl


@pytest.mark.parametrize("seed,L,H,P,N,h0s", [(1, 20, 2, 3, 4, 0.0), (2, 33, 3, 2, 8, 1.0), (3, 9, 1, 5, 16, 0.5)])
def test_parallel_form(oracle_lib, seed, L, H, P, N, h0s):
    c = gla_case(seed, L, H, P, N, h0s)
    o, hl = run(c, oracle_lib)
    op, hp = parallel_form(c)
    assert rel_err(o, op) < 1e-11
    assert rel_err(hl[0], hp) < 1e-11


def test_constant_gates_are_retention(oracle_lib):
    L, H, P, N = 40, 3, 4, 6
    c = gla_case(4, L, H, P, N)
    gam = 1.0 - 2.0 ** (-5.0 - np.arange(H))
    c["gk"] = np.broadcast_to(np.log(gam)[None, :, None], (L, H, N)).copy()
    o, hl = run(c, oracle_lib)
    y, hs = O.ssd(c["v"], np.zeros((L, H)), c["k"], c["q"], np.log(gam), np.zeros(H),
                  np.full(H, np.log(np.e - 1.0)), lib=oracle_lib)
    assert rel_err(o, y) < 1e-12
    assert rel_err(hl, hs) < 1e-12


def test_key_gates_are_grouped_scan_with_unit_step(oracle_lib):
    L, H, P, N = 30, 2, 3, 8
    c = gla_case(5, L, H, P, N, 1.0)
    gk_n = -np.exp(np.random.default_rng(6).uniform(-3, 0, (H, N)))
    c["gk"] = np.broadcast_to(gk_n[None], (L, H, N)).copy()
    o, hl = run(c, oracle_lib)
    dim = H * P
    z = np.full((L, dim), 2.0)
    y, hs = O.scan_fwd_groups(c["v"].reshape(L, dim), np.zeros((L, dim)), z, c["k"], c["q"],
                              np.repeat(gk_n, P, axis=0), np.zeros(dim), np.full(dim, np.log(np.e - 1.0)),
                              h0=c["h0"].reshape(1, dim, N), lib=oracle_lib)
    assert rel_err(o.reshape(L, dim), y / (z * expit(z))) < 1e-12
    assert rel_err(hl.reshape(dim, N), hs[0]) < 1e-12


def test_split_packed_batched(oracle_lib):
    L, H, P, N = 37, 2, 3, 5
    c = gla_case(7, L, H, P, N, 1.0)
    o, hl = run(c, oracle_lib)
    k = 16
    first = {key: (val[:k] if key != "h0" else val) for key, val in c.items()}
    second = {key: (val[k:] if key != "h0" else val) for key, val in c.items()}
    o1, h1 = run(first, oracle_lib)
    second["h0"] = h1[0]
    o2, h2 = run(second, oracle_lib)
    assert rel_err(np.concatenate([o1, o2]), o) < 1e-13 and rel_err(h2, hl) < 1e-13
    parts = [gla_case(10 + i, n, H, P, N, 1.0) for i, n in enumerate((5, 1, 12))]
    cat = {key: np.concatenate([p_[key] for p_ in parts]) for key in ("q", "k", "v", "gk")}
    ss = np.array([0, 5, 6, 18])
    op, hp = O.gla(cat["q"], cat["k"], cat["v"], cat["gk"], h0=np.stack([p_["h0"] for p_ in parts]), seq_start=ss,
                   lib=oracle_lib)
    for i, p_ in enumerate(parts):
        oi, hi = run(p_, oracle_lib)
        np.testing.assert_array_equal(op[ss[i]:ss[i + 1]], oi)
        np.testing.assert_array_equal(hp[i], hi[0])
    eq = [gla_case(20 + i, 6, H, P, N, 1.0) for i in range(2)]
    st = lambda key: np.stack([p_[key] for p_ in eq])
    ob, hb = O.gla(st("q"), st("k"), st("v"), st("gk"), h0=st("h0"), lib=oracle_lib)
    for i, p_ in enumerate(eq):
        oi, hi = run(p_, oracle_lib)
        np.testing.assert_array_equal(ob[i], oi)
        np.testing.assert_array_equal(hb[i], hi[0])


GLA_MUTANTS = {
    "readout_before_update": ("st[p * N + n] = exp(gt[n]) * st[p * N + n] + kt[n] * vp;\n            acc += qt[n] * st[p * N + n];",
                              "acc += qt[n] * st[p * N + n];\n            st[p * N + n] = exp(gt[n]) * st[p * N + n] + kt[n] * vp;"),
    "gate_on_input": ("exp(gt[n]) * st[p * N + n] + kt[n] * vp;", "st[p * N + n] + exp(gt[n]) * kt[n] * vp;"),
    "q_and_k_swapped": ("acc += qt[n] * st[p * N + n];", "acc += kt[n] * st[p * N + n];"),
    "gate_of_other_head": ("const double* gt = gk + (t * H + h) * N;", "const double* gt = gk + (t * H + (h + 1) % H) * N;"),
    "no_h0_offset": ("st[i] = h0 ? h0[(s * H + h) * P * N + i] : 0.0;", "st[i] = h0 ? h0[h * P * N + i] : 0.0;"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(GLA_MUTANTS))
def test_gla_mutant_is_caught(tmp_path, name):
    src = O.SRC.read_text()
    old, new = GLA_MUTANTS[name]
    assert src.count(old) == 1, "mutation anchor missing or ambiguous in oracle.c: " + name
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / ("lib_%s.so" % name)
    O.build(force=True, src=path, out=so)
    lib = O.load(so)
    parts = [gla_case(30 + i, n, 3, 2, 4, 1.0) for i, n in enumerate((7, 5))]
    cat = {key: np.concatenate([p_[key] for p_ in parts]) for key in ("q", "k", "v", "gk")}
    ss = np.array([0, 7, 12])
    o, hl = O.gla(cat["q"], cat["k"], cat["v"], cat["gk"], h0=np.stack([p_["h0"] for p_ in parts]), seq_start=ss,
                  lib=lib)
    bad = False
    for i, p_ in enumerate(parts):
        op, hp = parallel_form(p_)
        bad |= rel_err(o[ss[i]:ss[i + 1]], op) > 1e-6 or rel_err(hl[i], hp) > 1e-6
    assert bad, "parallel form did not reject mutant " + name
