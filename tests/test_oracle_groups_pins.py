"""Pins of the oracle's grouped prefill (oracle_scan_fwd_groups): several (B, C) groups per token and state
sizes beyond 16.

The recurrence is that of page "SAMBA混合注意力状态空间模型", 数学框架 -> Mamba层, with the Mamba reading of Ā,
B̄, Δ, skip and gate.  Groups generalise the pages' single selection vector: channel d reads the (B, C) of
group d // (dim // G) (contiguous channel blocks per group).  Pins:
  * the O(L^2) unrolled-sum brute force (an independent formulation: products of Ā as exp(A * sum of Δ)),
    applied to each group's block of channels with that group's B and C, for state sizes 16, 32, 64, 128;
  * G = 1 is exactly the ungrouped prefill; G = dim is one scan per channel with its own B and C;
  * permuting groups together with their channel blocks permutes the outputs;
  * splitting 32 states into two halves of 16: the readouts add and the final states concatenate;
  * planted mistakes in the group indexing are rejected by the brute-force pin.
"""
import shutil

import numpy as np
import pytest
from scipy.special import expit

from oracle import oracle as O
from tests.test_oracle_pins import brute_force, rel_err


def grouped_case(seed, L, D, G, N, h0_scale=0.0):
    g = np.random.default_rng(seed)
    x, z, dt = (g.standard_normal((L, D)) for _ in range(3))
    B, C = g.standard_normal((L, G, N)), g.standard_normal((L, G, N))
    bias = np.log(np.expm1(g.uniform(1e-3, 1e-1, D)))
    A = -np.exp(g.uniform(0, np.log(16), (D, N)))
    Dv = g.uniform(0, 1, D)
    h0 = h0_scale * g.standard_normal((D, N)) if h0_scale else None
    return dict(x=x, dt=dt, z=z, B=B, C=C, A=A, Dv=Dv, bias=bias, h0=h0)


def run(c, lib=None, seq_start=None):
    h0 = None if c["h0"] is None else c["h0"][None]
    return O.scan_fwd_groups(c["x"], c["dt"], c["z"], c["B"], c["C"], c["A"], c["Dv"], c["bias"], h0=h0,
                             seq_start=seq_start, lib=lib)


def brute_grouped(c):
    L, D = c["x"].shape
    G = c["B"].shape[1]
    per = D // G
    y = np.zeros((L, D))
    hl = np.zeros_like(c["A"])
    for g in range(G):
        sl = slice(g * per, (g + 1) * per)
        h0 = None if c["h0"] is None else c["h0"][sl]
        y[:, sl], hl[sl] = brute_force(c["x"][:, sl], c["dt"][:, sl], c["z"][:, sl], c["B"][:, g], c["C"][:, g],
                                       c["A"][sl], c["Dv"][sl], c["bias"][sl], h0)
    return y, hl


@pytest.mark.parametrize("seed,L,D,G,N,h0s", [(1, 23, 6, 3, 16, 0.0), (2, 31, 8, 2, 32, 1.0), (3, 17, 4, 4, 64, 0.5),
                                              (4, 12, 4, 1, 128, 1.0), (5, 9, 6, 6, 16, 2.0)])
def test_grouped_brute_force(oracle_lib, seed, L, D, G, N, h0s):
    c = grouped_case(seed, L, D, G, N, h0s)
    y, hl = run(c, oracle_lib)
    yb, hb = brute_grouped(c)
    assert rel_err(y, yb) < 1e-11
    assert rel_err(hl, hb) < 1e-11


def test_one_group_is_the_ungrouped_prefill(oracle_lib):
    c = grouped_case(6, 40, 5, 1, 16, 1.0)
    y, hl = run(c, oracle_lib)
    y1, hl1 = O.scan_fwd(c["x"], c["dt"], c["z"], c["B"][:, 0], c["C"][:, 0], c["A"], c["Dv"], c["bias"],
                         h0=c["h0"][None], lib=oracle_lib)
    np.testing.assert_array_equal(y, y1)
    np.testing.assert_array_equal(hl, hl1)


def test_group_per_channel_is_separate_scans(oracle_lib):
    c = grouped_case(7, 25, 4, 4, 32, 1.0)
    y, hl = run(c, oracle_lib)
    for d in range(4):
        yd, hd = O.scan_fwd(c["x"][:, d:d + 1], c["dt"][:, d:d + 1], c["z"][:, d:d + 1], c["B"][:, d], c["C"][:, d],
                            c["A"][d:d + 1], c["Dv"][d:d + 1], c["bias"][d:d + 1], h0=c["h0"][None, d:d + 1],
                            lib=oracle_lib)
        np.testing.assert_array_equal(y[:, d:d + 1], yd)
        np.testing.assert_array_equal(hl[:, d:d + 1], hd)


def test_group_permutation(oracle_lib):
    G, per, N = 3, 2, 16
    c = grouped_case(8, 20, G * per, G, N, 1.0)
    perm = [2, 0, 1]
    chan = np.concatenate([np.arange(g * per, (g + 1) * per) for g in perm])
    cp = dict(c)
    for k in ("x", "dt", "z"):
        cp[k] = c[k][:, chan]
    for k in ("A", "h0"):
        cp[k] = c[k][chan]
    for k in ("Dv", "bias"):
        cp[k] = c[k][chan]
    cp["B"], cp["C"] = c["B"][:, perm], c["C"][:, perm]
    y, hl = run(c, oracle_lib)
    yp, hlp = run(cp, oracle_lib)
    np.testing.assert_array_equal(yp, y[:, chan])
    np.testing.assert_array_equal(hlp[0], hl[0][chan])


def test_state_halves_add(oracle_lib):
    c = grouped_case(9, 30, 4, 2, 32, 1.0)
    c["Dv"] = np.zeros(4)
    y, hl = run(c, oracle_lib)
    parts = []
    for half in (slice(0, 16), slice(16, 32)):
        ch = dict(c, B=c["B"][:, :, half], C=c["C"][:, :, half], A=c["A"][:, half], h0=c["h0"][:, half])
        parts.append(run(ch, oracle_lib))
    gate = c["z"] * expit(c["z"])
    np.testing.assert_allclose(y / gate, parts[0][0] / gate + parts[1][0] / gate, rtol=1e-10, atol=1e-10)
    np.testing.assert_array_equal(hl[0], np.concatenate([parts[0][1][0], parts[1][1][0]], axis=1))


def test_rejects_groups_not_dividing_dim(oracle_lib):
    c = grouped_case(10, 4, 5, 2, 16)
    with pytest.raises(Exception):
        run(c, oracle_lib)


GROUP_MUTANTS = {
    "interleaved_groups": ("const int64_t g = d / per_group;", "const int64_t g = d % ngroups;"),
    "first_group_only": ("B + (t * ngroups + g) * dstate, C + (t * ngroups + g) * dstate,",
                         "B + (t * ngroups + 0) * dstate, C + (t * ngroups + 0) * dstate,"),
    "token_stride_without_groups": ("B + (t * ngroups + g) * dstate, C + (t * ngroups + g) * dstate,",
                                    "B + (t + g) * dstate, C + (t + g) * dstate,"),
    "c_from_other_group": ("C + (t * ngroups + g) * dstate,", "C + (t * ngroups + (g + 1) % ngroups) * dstate,"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(GROUP_MUTANTS))
def test_group_mutant_is_caught(tmp_path, name):
    src = O.SRC.read_text()
    old, new = GROUP_MUTANTS[name]
    assert src.count(old) == 1, "mutation anchor missing or ambiguous in oracle.c: " + name
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / ("lib_%s.so" % name)
    O.build(force=True, src=path, out=so)
    lib = O.load(so)
    c = grouped_case(11, 14, 6, 3, 16, 1.0)
    y, hl = run(c, lib)
    yb, hb = brute_grouped(c)
    assert rel_err(y, yb) > 1e-6 or rel_err(hl, hb) > 1e-6, "brute force did not reject mutant " + name
