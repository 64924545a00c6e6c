"""Pins of the oracle's sliding-window attention (oracle_swa) against facts that do not come from it.

What it computes: page "SAMBA混合注意力状态空间模型", 数学框架 -> 滑动窗口注意力 (softmax of the scaled
scores plus the window mask, times V; the mask as printed is inverted, read as: visible when the key is at
most `window` tokens back), and the hackernoon page, §2.1.2 (window of 2048 tokens, RoPE relative positions
inside the window).  Pins:
  * a hand-worked example (head size 4, two rotation pairs at different angles) whose value is written out
    with math.cos / math.exp: it fixes the 1/sqrt(d_k) scale, the rotation's direction and its pairing
    (c, c + d_k/2);
  * window edges: with q = 0 every visible key weighs the same, so one-hot values expose exactly which keys a
    query sees (key i - window included, i - window - 1 not, nothing across a sequence start);
  * window 0 returns v itself; hard attention with scores in the thousands (needs the maximum subtracted)
    picks the one highest-scoring visible key and ignores a higher one just outside the window;
  * RoPE depends on relative positions only: shifting every position by the same amount leaves the output
    unchanged, and keys rotated at the query's position instead of their own (a plausible slip) do not;
  * packed sequences equal separate calls; heads are independent; a subset of query rows equals the same
    rows of the full call;
  * RoPE alone (oracle_rope, the rotation used inside oracle_swa) keeps each pair's norm, adds angles, is the
    identity at angle 0 and turns (1, 0) into (0, 1) at a quarter turn.
A mutation test plants mistakes in copies of the oracle and checks that the pins reject every one.
"""
import math
import shutil

import numpy as np
import pytest

from oracle import oracle as O


def rope_tables(npos, hd, base=10000.0, shift=0):
    ang = (np.arange(npos)[:, None] + shift) * base ** (-2.0 * np.arange(hd // 2)[None, :] / hd)
    return np.cos(ang), np.sin(ang)


def hand_example(lib):
    # T = 2, one head of size 4: rotation pairs (0, 2) and (1, 3).  Position 1 turns pair 0 by a = pi/3 and
    # pair 1 by b = pi/2; position 0 does not turn.
    a, b = math.pi / 3, math.pi / 2
    cos = np.array([[1.0, 1.0], [math.cos(a), math.cos(b)]])
    sin = np.array([[0.0, 0.0], [math.sin(a), math.sin(b)]])
    q = np.array([[[0.0, 0.0, 0.0, 0.0]], [[1.0, 2.0, 0.0, 0.0]]])
    k = np.array([[[1.0, 1.0, 0.0, 0.0]], [[0.0, 0.0, 1.0, 1.0]]])
    v = np.array([[[1.0, 0.0, 0.0, 0.0]], [[0.0, 1.0, 0.0, 0.0]]])
    o = O.swa(q, k, v, window=1, rope_cos=cos, rope_sin=sin, lib=lib)
    # rotated: q1 = (cos a, 2 cos b, sin a, 2 sin b); k0 = (1, 1, 0, 0); k1 = (-sin a, -sin b, cos a, cos b)
    s0 = (math.cos(a) + 2 * math.cos(b)) / 2.0
    s1 = (-math.cos(a) * math.sin(a) - 2 * math.cos(b) * math.sin(b) + math.sin(a) * math.cos(a)
          + 2 * math.sin(b) * math.cos(b)) / 2.0
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    want = np.array([[[1.0, 0.0, 0.0, 0.0]], [[w0, 1.0 - w0, 0.0, 0.0]]])
    return float(np.max(np.abs(o - want)))


def window_support(lib, lengths=(9, 1, 6), window=3, rope=True):
    T = sum(lengths)
    hd = 2 * T
    seq_start = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    g = np.random.default_rng(5)
    q = np.zeros((T, 1, hd))
    k = g.standard_normal((T, 1, hd))
    v = np.eye(T, hd)[:, None, :]
    cos, sin = rope_tables(max(lengths), hd) if rope else (None, None)
    o = O.swa(q, k, v, window, cos, sin, seq_start=seq_start, lib=lib)
    want = np.zeros((T, 1, hd))
    for s in range(len(lengths)):
        for i in range(seq_start[s], seq_start[s + 1]):
            lo = max(seq_start[s], i - window)
            want[i, 0, lo:i + 1] = 1.0 / (i + 1 - lo)
    return float(np.max(np.abs(o - want)))


def hard_attention(lib, window=4):
    T, hd = 12, 16
    g = np.random.default_rng(6)
    k = np.eye(T, hd)[:, None, :]
    v = g.standard_normal((T, 1, hd))
    q = np.zeros((T, 1, hd))
    want = np.empty((T, 1, hd))
    for i in range(T):
        lo = max(0, i - window)
        q[i, 0, lo] = 2.0e4                 # the oldest visible key wins
        if i - window - 1 >= 0:
            q[i, 0, i - window - 1] = 4.0e4  # higher, but one token outside the window
        want[i] = v[lo]
    o = O.swa(q, k, v, window, lib=lib)
    return float(np.max(np.abs(o - want))) if np.all(np.isfinite(o)) else math.inf


def relative_position_gap(lib, shift=37):
    g = np.random.default_rng(7)
    T, H, hd = 20, 2, 8
    q, k, v = (g.standard_normal((T, H, hd)) for _ in range(3))
    c0, s0 = rope_tables(T, hd)
    c1, s1 = rope_tables(T, hd, shift=shift)
    o0 = O.swa(q, k, v, 6, c0, s0, lib=lib)
    o1 = O.swa(q, k, v, 6, c1, s1, lib=lib)
    on = O.swa(q, k, v, 6, lib=lib)
    return float(np.max(np.abs(o0 - o1))), float(np.max(np.abs(o0 - on)))


def test_hand_worked_example(oracle_lib):
    assert hand_example(oracle_lib) < 1e-14


@pytest.mark.parametrize("rope", [False, True])
@pytest.mark.parametrize("window", [0, 1, 3, 8, 100])
def test_window_support_exact(oracle_lib, window, rope):
    assert window_support(oracle_lib, window=window, rope=rope) < 1e-14


def test_window_zero_returns_v(oracle_lib):
    g = np.random.default_rng(8)
    q, k, v = (g.standard_normal((10, 3, 8)) for _ in range(3))
    cos, sin = rope_tables(10, 8)
    np.testing.assert_array_equal(O.swa(q, k, v, 0, cos, sin, lib=oracle_lib), v)


@pytest.mark.parametrize("window", [1, 4, 11])
def test_hard_attention_picks_visible_key(oracle_lib, window):
    assert hard_attention(oracle_lib, window) < 1e-12


def test_rope_relative_positions_only(oracle_lib):
    gap_shift, gap_norope = relative_position_gap(oracle_lib)
    assert gap_shift < 1e-12
    assert gap_norope > 1e-2


def test_full_window_is_causal_softmax_attention(oracle_lib):
    # with the window covering the whole sequence and no rotation, the layer is plain causal attention;
    # compared with the matrix form (scores, upper triangle masked, row softmax, times V)
    g = np.random.default_rng(9)
    T, H, hd = 17, 2, 8
    q, k, v = (g.standard_normal((T, H, hd)) for _ in range(3))
    o = O.swa(q, k, v, T, lib=oracle_lib)
    for h in range(H):
        s = q[:, h] @ k[:, h].T / math.sqrt(hd)
        s[np.triu_indices(T, 1)] = -np.inf
        p = np.exp(s - s.max(axis=1, keepdims=True))
        np.testing.assert_allclose(o[:, h], (p / p.sum(axis=1, keepdims=True)) @ v[:, h], rtol=1e-12, atol=1e-12)


def test_packed_equals_separate_and_heads_independent(oracle_lib):
    g = np.random.default_rng(10)
    lengths, H, hd, w = (7, 0, 12, 3), 3, 8, 4
    T = sum(lengths)
    q, k, v = (g.standard_normal((T, H, hd)) for _ in range(3))
    cos, sin = rope_tables(max(lengths), hd)
    st = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    o = O.swa(q, k, v, w, cos, sin, seq_start=st, lib=oracle_lib)
    for s in range(len(lengths)):
        a, b = st[s], st[s + 1]
        if b > a:
            np.testing.assert_array_equal(o[a:b], O.swa(q[a:b], k[a:b], v[a:b], w, cos, sin, lib=oracle_lib))
    perm = [2, 0, 1]
    op = O.swa(q[:, perm], k[:, perm], v[:, perm], w, cos, sin, seq_start=st, lib=oracle_lib)
    np.testing.assert_array_equal(op, o[:, perm])


def test_rope_alone_is_a_rotation_by_position(oracle_lib):
    # rotation is orthogonal pairwise (norms of (x[c], x[c+hd/2]) kept), angle-additive (table rows a, b, a+b),
    # the identity at angle 0, and a quarter turn maps (1, 0) to (0, 1)
    g = np.random.default_rng(11)
    T, H, hd = 6, 2, 8
    x = g.standard_normal((T, H, hd))
    cos, sin = rope_tables(64, hd)
    pos = np.array([0, 1, 5, 9, 30, 63])
    r = O.rope(x, cos, sin, pos, lib=oracle_lib)
    half = hd // 2
    np.testing.assert_allclose(r[..., :half] ** 2 + r[..., half:] ** 2, x[..., :half] ** 2 + x[..., half:] ** 2,
                               rtol=1e-12)
    np.testing.assert_array_equal(r[0], x[0])
    a, b = 9, 30
    twice = O.rope(O.rope(x, cos, sin, np.full(T, a), lib=oracle_lib), cos, sin, np.full(T, b), lib=oracle_lib)
    c2, s2 = rope_tables(a + b + 1, hd)
    once = O.rope(x, c2, s2, np.full(T, a + b), lib=oracle_lib)
    np.testing.assert_allclose(twice, once, rtol=1e-12, atol=1e-12)
    quarter_c, quarter_s = np.zeros((1, 1)), np.ones((1, 1))
    e = np.array([[[1.0, 0.0]]])
    np.testing.assert_array_equal(O.rope(e, quarter_c, quarter_s, [0], lib=oracle_lib), [[[0.0, 1.0]]])


def test_rows_subset_matches_full(oracle_lib):
    g = np.random.default_rng(12)
    lengths, H, hd, w = (9, 14), 2, 8, 5
    T = sum(lengths)
    q, k, v = (g.standard_normal((T, H, hd)) for _ in range(3))
    cos, sin = rope_tables(max(lengths), hd)
    st = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    full = O.swa(q, k, v, w, cos, sin, seq_start=st, lib=oracle_lib)
    rows = [0, 8, 9, 15, 22]
    part = O.swa(q, k, v, w, cos, sin, seq_start=st, rows=rows, lib=oracle_lib)
    np.testing.assert_array_equal(part[rows], full[rows])
    assert np.isnan(np.delete(part, rows, axis=0)).all()


def test_rejects_bad_arguments(oracle_lib):
    q = np.zeros((4, 1, 3))
    with pytest.raises(RuntimeError):
        O.swa(q, q, q, 2, lib=oracle_lib)  # odd head size
    q = np.zeros((4, 1, 4))
    with pytest.raises(RuntimeError):
        O.swa(q, q, q, -1, lib=oracle_lib)


def pins_hold(lib) -> bool:
    if hand_example(lib) > 1e-12:
        return False
    for w in (0, 1, 3):
        for rope in (False, True):
            if window_support(lib, window=w, rope=rope) > 1e-12:
                return False
    if hard_attention(lib) > 1e-9:
        return False
    gap_shift, gap_norope = relative_position_gap(lib)
    return gap_shift < 1e-12 and gap_norope > 1e-2


SWA_MUTANTS = {
    "window_one_short": ("const int64_t jlo = (i - window > t0) ? i - window : t0;",
                         "const int64_t jlo = (i - window + 1 > t0) ? i - window + 1 : t0;"),
    "window_one_long": ("const int64_t jlo = (i - window > t0) ? i - window : t0;",
                        "const int64_t jlo = (i - window - 1 > t0) ? i - window - 1 : t0;"),
    "scale_dropped": ("sc[j - jlo] = dot / sqrt((double)hd);", "sc[j - jlo] = dot;"),
    "rotation_sign": ("out[c] = x[c] * cs[c] - x[c + half] * sn[c];", "out[c] = x[c] * cs[c] + x[c + half] * sn[c];"),
    "adjacent_pairs": ("out[c + half] = x[c + half] * cs[c] + x[c] * sn[c];",
                       "out[c + half] = x[c + half] * cs[c] + x[(c + 1) % half] * sn[c];"),
    "keys_at_query_position": ("rope_cos + (j - t0) * (hd / 2), rope_sin + (j - t0) * (hd / 2)",
                               "rope_cos + (i - t0) * (hd / 2), rope_sin + (i - t0) * (hd / 2)"),
    "no_max_subtracted": ("sc[j] = exp(sc[j] - mx);", "sc[j] = exp(sc[j]);"),
    "sequences_leak": ("  while (seq_start[s + 1] <= i) ++s;\n  return s;", "  while (seq_start[s + 1] <= i) ++s;\n  return 0;"),
    "unnormalised": ("const double w = sc[j - jlo] / den;", "const double w = sc[j - jlo];"),
    "value_of_query": ("const double* vj = v + (j * H + h) * hd;", "const double* vj = v + (i * H + h) * hd;"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(SWA_MUTANTS))
def test_swa_mutant_is_caught(tmp_path, name):
    src = O.SRC.read_text()
    old, new = SWA_MUTANTS[name]
    assert src.count(old) == 1, "mutation anchor missing or ambiguous in oracle.c: " + name
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / ("lib_%s.so" % name)
    O.build(force=True, src=path, out=so)
    lib = O.load(so)
    try:
        ok = pins_hold(lib)
    except Exception:
        ok = False
    assert not ok, "pins did not reject mutant " + name
