"""Pins of the oracle's gradients (oracle_scan_bwd) against facts that do not come from that function.

The gradients are the derivative of the prefill the oracle computes (page
"SAMBA混合注意力状态空间模型", 数学框架 -> Mamba层, with the Mamba reading of Ā,
B̄, Δ, skip and gate), taken for the loss sum(dy * y) + sum(dh_last * h_last):
  * central finite differences of the oracle's own forward, on every input
    element (x, dt, z, B, C, A, D, dt_bias, h0), including the regions where
    softplus is linear (v > 20) and vanishing (v << 0);
  * reverse-mode autodiff (torch, float64 on the CPU) of an independent loop
    written here;
  * a closed form: with dy = 0 the adjoint of h_t is the future decay
    exp(A * sum of later Δ) times dh_last, which fixes dh0, dx and dB;
  * structural identities: chained calls (dh0 of the later call fed as dh_last
    of the earlier one) == one call; packed sequences == separate calls;
    linearity in (dy, dh_last).
A mutation test plants mistakes in copies of the backward and checks that the
finite-difference pin rejects every one.
"""
import math
import shutil

import numpy as np
import pytest

from oracle import oracle as O

GRAD_KEYS = ("dx", "ddt", "dz", "dB", "dC", "dA", "dD", "ddt_bias", "dh0")


def make_case(seed, lengths, D, N, h0_scale=1.0, extreme=False):
    g = np.random.default_rng(seed)
    T = int(sum(lengths))
    nseq = len(lengths)
    c = dict(
        x=g.standard_normal((T, D)), dt=g.standard_normal((T, D)), z=g.standard_normal((T, D)),
        B=g.standard_normal((T, N)), C=g.standard_normal((T, N)),
        A=-np.exp(g.uniform(0, math.log(16), (D, N))), D=g.uniform(0, 1, D),
        bias=np.log(np.expm1(g.uniform(1e-3, 1e-1, D))),
        h0=h0_scale * g.standard_normal((nseq, D, N)),
        dy=g.standard_normal((T, D)), dh_last=g.standard_normal((nseq, D, N)),
        seq_start=np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64),
    )
    if extreme and T >= 3:
        c["dt"][0, 0] = 27.0     # softplus linear: Δ = v
        c["dt"][1, 0] = -30.0    # Δ ~ 1e-13
        c["dt"][2, -1] = 3.0     # a large step: strong decay
    return c


def fwd(c, lib, **over):
    v = {**c, **over}
    return O.scan_fwd(v["x"], v["dt"], v["z"], v["B"], v["C"], v["A"], v["D"], v["bias"], h0=v["h0"],
                      seq_start=v["seq_start"], lib=lib)


def bwd(c, lib, **over):
    v = {**c, **over}
    return O.scan_bwd(v["x"], v["dt"], v["z"], v["B"], v["C"], v["A"], v["D"], v["bias"], v["dy"], h0=v["h0"],
                      dh_last=v["dh_last"], seq_start=v["seq_start"], lib=lib)


def loss(c, lib, **over):
    y, hl = fwd(c, lib, **over)
    return float(np.sum(y * c["dy"]) + np.sum(hl * c["dh_last"]))


# the oracle's name of each input's gradient
FD_MAP = {"x": "dx", "dt": "ddt", "z": "dz", "B": "dB", "C": "dC", "A": "dA", "D": "dD", "bias": "ddt_bias",
          "h0": "dh0"}


def fd_errors(c, lib, grads):
    """max |finite difference - analytic| / max(1, max |analytic|), per input."""
    errs = {}
    for name, gk in FD_MAP.items():
        base = c[name]
        an = grads[gk]
        fd = np.empty_like(base)
        for idx in np.ndindex(base.shape):
            eps = 1e-6 * max(1.0, abs(base[idx]))
            p = base.copy()
            p[idx] = base[idx] + eps
            lp = loss(c, lib, **{name: p})
            p[idx] = base[idx] - eps
            lm = loss(c, lib, **{name: p})
            fd[idx] = (lp - lm) / (2 * eps)
        errs[name] = float(np.max(np.abs(fd - an))) / max(1.0, float(np.max(np.abs(an))))
    return errs


@pytest.mark.parametrize("seed,lengths,D,N", [(11, [5, 0, 7], 3, 16), (12, [9], 2, 16), (13, [3, 4], 2, 3)])
def test_finite_differences(oracle_lib, seed, lengths, D, N):
    c = make_case(seed, lengths, D, N, extreme=True)
    errs = fd_errors(c, oracle_lib, bwd(c, oracle_lib))
    assert max(errs.values()) < 2e-6, errs


def test_torch_autograd(oracle_lib):
    torch = pytest.importorskip("torch")
    c = make_case(21, [6, 4], 3, 16, extreme=True)
    t = {k: torch.tensor(c[k], dtype=torch.float64, requires_grad=True)
         for k in ("x", "dt", "z", "B", "C", "A", "D", "bias", "h0")}
    total = torch.zeros((), dtype=torch.float64)
    dy = torch.tensor(c["dy"], dtype=torch.float64)
    dhl = torch.tensor(c["dh_last"], dtype=torch.float64)
    ss = c["seq_start"]
    for s in range(len(ss) - 1):
        h = t["h0"][s]                                       # [D][N]
        for r in range(ss[s], ss[s + 1]):
            delta = torch.logaddexp(torch.zeros(()), t["dt"][r] + t["bias"])   # [D]
            h = torch.exp(delta[:, None] * t["A"]) * h + (delta * t["x"][r])[:, None] * t["B"][r][None, :]
            pre = (h * t["C"][r][None, :]).sum(dim=1) + t["D"] * t["x"][r]
            y = pre * t["z"][r] * torch.sigmoid(t["z"][r])
            total = total + (y * dy[r]).sum()
        total = total + (h * dhl[s]).sum()
    total.backward()
    ref = {FD_MAP[k]: t[k].grad.numpy() for k in FD_MAP}
    got = bwd(c, oracle_lib)
    for k in GRAD_KEYS:
        scale = max(1.0, float(np.max(np.abs(ref[k]))))
        assert float(np.max(np.abs(got[k] - ref[k]))) / scale < 1e-12, k


def test_adjoint_closed_form_without_dy(oracle_lib):
    """dy = 0: g_t = exp(A * sum_{r>t} Δ_r) dh_last; dh0 = exp(A * sum Δ) dh_last,
    dx_t = Δ_t sum_n g_t B_t, dB_t = sum_d g_t Δ_t x_t; dz, dC, dD vanish."""
    c = make_case(31, [10], 2, 16)
    c["dy"] = np.zeros_like(c["dy"])
    got = bwd(c, oracle_lib)
    delta = np.logaddexp(0.0, c["dt"] + c["bias"][None, :])      # [T][D]
    later = np.cumsum(delta[::-1], axis=0)[::-1] - delta          # sum_{r>t} Δ_r
    g = np.exp(later[:, :, None] * c["A"][None]) * c["dh_last"][0][None]   # [T][D][N]
    np.testing.assert_allclose(got["dh0"][0], np.exp(delta.sum(0)[:, None] * c["A"]) * c["dh_last"][0],
                               rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(got["dx"], delta * np.einsum("tdn,tn->td", g, c["B"]), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(got["dB"], np.einsum("tdn,td->tn", g, delta * c["x"]), rtol=1e-11, atol=1e-13)
    for k in ("dz", "dC", "dD"):
        assert np.all(got[k] == 0.0), k


def test_chained_calls_equal_one_call(oracle_lib):
    c = make_case(41, [30], 3, 16)
    one = bwd(c, oracle_lib)
    cut = 12
    part = lambda a, sl: a[sl]
    c1 = {**c, **{k: part(c[k], slice(0, cut)) for k in ("x", "dt", "z", "B", "C", "dy")},
          "seq_start": np.array([0, cut], dtype=np.int64)}
    c2 = {**c, **{k: part(c[k], slice(cut, 30)) for k in ("x", "dt", "z", "B", "C", "dy")},
          "seq_start": np.array([0, 30 - cut], dtype=np.int64)}
    _, hmid = fwd({**c1, "dh_last": None}, oracle_lib)
    g2 = bwd(c2, oracle_lib, h0=hmid)
    g1 = bwd(c1, oracle_lib, dh_last=g2["dh0"])
    for k in ("dx", "ddt", "dz", "dB", "dC"):
        np.testing.assert_allclose(np.concatenate([g1[k], g2[k]]), one[k], rtol=1e-12, atol=1e-13, err_msg=k)
    for k in ("dA", "dD", "ddt_bias"):
        np.testing.assert_allclose(g1[k] + g2[k], one[k], rtol=1e-12, atol=1e-13, err_msg=k)
    np.testing.assert_allclose(g1["dh0"], one["dh0"], rtol=1e-12, atol=1e-14)


def test_packed_equals_separate(oracle_lib):
    lengths = [7, 0, 5, 9]
    c = make_case(51, lengths, 3, 16)
    packed = bwd(c, oracle_lib)
    ss = c["seq_start"]
    sums = {k: 0.0 for k in ("dA", "dD", "ddt_bias")}
    for s in range(len(lengths)):
        sl = slice(ss[s], ss[s + 1])
        cs = {**c, **{k: c[k][sl] for k in ("x", "dt", "z", "B", "C", "dy")}, "h0": c["h0"][s:s + 1],
              "dh_last": c["dh_last"][s:s + 1], "seq_start": np.array([0, lengths[s]], dtype=np.int64)}
        gs = bwd(cs, oracle_lib)
        for k in ("dx", "ddt", "dz", "dB", "dC"):
            np.testing.assert_allclose(packed[k][sl], gs[k], rtol=1e-13, atol=1e-15, err_msg=k)
        np.testing.assert_allclose(packed["dh0"][s], gs["dh0"][0], rtol=1e-13, atol=1e-15)
        for k in sums:
            sums[k] = sums[k] + gs[k]
    for k in sums:
        np.testing.assert_allclose(packed[k], sums[k], rtol=1e-12, atol=1e-14, err_msg=k)


def test_linear_in_upstream_gradients(oracle_lib):
    c = make_case(61, [8, 6], 2, 16)
    g = np.random.default_rng(5)
    dy2, dh2 = g.standard_normal(c["dy"].shape), g.standard_normal(c["dh_last"].shape)
    a = bwd(c, oracle_lib)
    b = bwd(c, oracle_lib, dy=dy2, dh_last=dh2)
    ab = bwd(c, oracle_lib, dy=2.0 * c["dy"] - 3.0 * dy2, dh_last=2.0 * c["dh_last"] - 3.0 * dh2)
    for k in GRAD_KEYS:
        np.testing.assert_allclose(ab[k], 2.0 * a[k] - 3.0 * b[k], rtol=1e-10, atol=1e-11, err_msg=k)
    z = bwd(c, oracle_lib, dy=0.0 * c["dy"], dh_last=None)
    for k in GRAD_KEYS:
        assert np.all(z[k] == 0.0), k


# --------------------------------------------------------------------------- #
# Mutation test of the backward: the finite-difference pin must reject each
# --------------------------------------------------------------------------- #
BWD_MUTANTS = {
    "readout_adjoint_dropped": ("const double gt = g[n] + dr * C[t * dstate + n];", "const double gt = g[n];"),
    "softplus_derivative_dropped": ("ddt[t * dim + d] = ddelta * sigmoid(v);", "ddt[t * dim + d] = ddelta;"),
    "post_state_in_ddelta": ("ddelta += gt * (Arow[n] * abar * hprev[n]", "ddelta += gt * (Arow[n] * abar * hcur[n]"),
    "silu_derivative_wrong": ("sz * (1.0 + zv * (1.0 - sz))", "sz"),
    "dh_last_ignored": ("g[n] = dh_last ? dh_last[(s * dim + d) * dstate + n] : 0.0;", "g[n] = 0.0;"),
    "carry_without_decay": ("g[n] = abar * gt;", "g[n] = gt;"),
    "dC_with_previous_state": ("acc[T * dstate + t * dstate + n] += dr * hcur[n];",
                               "acc[T * dstate + t * dstate + n] += dr * hprev[n];"),
    "dA_without_delta": ("dA[d * dstate + n] += gt * delta * abar * hprev[n];",
                         "dA[d * dstate + n] += gt * abar * hprev[n];"),
    "dx_skip_dropped": ("double dxv = dr * Dskip[d], ddelta = 0.0;", "double dxv = 0.0, ddelta = 0.0;"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_bwd_mutant_is_caught(tmp_path, name):
    src = O.SRC.read_text()
    old, new = BWD_MUTANTS[name]
    assert src.count(old) == 1, "mutation anchor missing or ambiguous in oracle.c: " + name
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / ("lib_%s.so" % name)
    O.build(force=True, src=path, out=so)
    lib = O.load(so)
    c = make_case(71, [4, 3], 2, 16, extreme=True)
    grads = bwd(c, lib)
    bad = any(not np.all(np.isfinite(grads[k])) for k in GRAD_KEYS)
    if not bad:
        errs = fd_errors(c, lib, grads)
        bad = max(errs.values()) > 1e-4
    assert bad, "finite differences did not reject mutant " + name
