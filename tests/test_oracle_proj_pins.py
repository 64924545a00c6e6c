"""Pins of the oracle's selection projections (oracle_proj) against facts that do not come from it.

The projections are the linear maps of page "SAMBA混合注意力状态空间模型", 数学框架 -> Mamba层
(B_t = Linear_B(x_t), C_t = Linear_C(x_t), and Linear_Δ(x_t) inside τ_Δ), stored as the rows of one
matrix W [dim + 2*dstate][dim].  Pins: a hand-worked example, selection by unit rows (identity and
single-column picks), linearity in x and in W, agreement with numpy's matrix product, and planted
mistakes (transposed W, a dropped term, B and C swapped, a row offset) that the pins reject.
"""
import shutil

import numpy as np
import pytest

from oracle import oracle as O


def test_hand_worked_example(oracle_lib):
    # dim 2, dstate 1: W rows = [Linear_Δ row 0, Linear_Δ row 1, Linear_B, Linear_C]
    x = np.array([[1.0, 2.0], [3.0, -1.0]])
    W = np.array([[1.0, 0.0], [0.5, 0.5], [2.0, -1.0], [0.0, 3.0]])
    dt, B, C = O.proj(x, W, dstate=1, lib=oracle_lib)
    np.testing.assert_array_equal(dt, [[1.0, 1.5], [3.0, 1.0]])
    np.testing.assert_array_equal(B, [[0.0], [7.0]])
    np.testing.assert_array_equal(C, [[6.0], [-3.0]])


def test_unit_rows_select(oracle_lib):
    g = np.random.default_rng(1)
    dim, N, T = 24, 16, 7
    x = g.standard_normal((T, dim))
    W = np.zeros((dim + 2 * N, dim))
    W[:dim] = np.eye(dim)
    pickB, pickC = g.integers(0, dim, N), g.integers(0, dim, N)
    W[dim + np.arange(N), pickB] = 1.0
    W[dim + N + np.arange(N), pickC] = 1.0
    dt, B, C = O.proj(x, W, dstate=N, lib=oracle_lib)
    np.testing.assert_array_equal(dt, x)
    np.testing.assert_array_equal(B, x[:, pickB])
    np.testing.assert_array_equal(C, x[:, pickC])


def test_linear_in_x_and_w(oracle_lib):
    g = np.random.default_rng(2)
    dim, N, T = 32, 16, 9
    x1, x2 = g.standard_normal((T, dim)), g.standard_normal((T, dim))
    W1, W2 = g.standard_normal((dim + 2 * N, dim)), g.standard_normal((dim + 2 * N, dim))
    r = [np.concatenate(O.proj(a, w, N, lib=oracle_lib), axis=1) for a, w in
         ((x1, W1), (x2, W1), (2 * x1 - 3 * x2, W1), (x1, W2), (x1, W1 + W2))]
    np.testing.assert_allclose(r[2], 2 * r[0] - 3 * r[1], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r[4], r[0] + r[3], rtol=1e-12, atol=1e-12)


def test_matches_numpy_matrix_product(oracle_lib):
    g = np.random.default_rng(3)
    dim, N, T = 64, 16, 33
    x, W = g.standard_normal((T, dim)), g.standard_normal((dim + 2 * N, dim))
    dt, B, C = O.proj(x, W, N, lib=oracle_lib)
    ref = x @ W.T
    np.testing.assert_allclose(np.concatenate([dt, B, C], axis=1), ref, rtol=1e-12, atol=1e-12)


PROJ_MUTANTS = {
    "transposed_weight": ("acc += x[t * dim + k] * W[j * dim + k];", "acc += x[t * dim + k] * W[k * dim + (j % dim)];"),
    "dropped_last_term": ("for (int64_t k = 0; k < dim; ++k) acc += x[t * dim + k] * W[j * dim + k];",
                          "for (int64_t k = 0; k + 1 < dim; ++k) acc += x[t * dim + k] * W[j * dim + k];"),
    "b_c_swapped": ("else if (j < dim + dstate) B[t * dstate + (j - dim)] = acc;",
                    "else if (j < dim + dstate) C[t * dstate + (j - dim)] = acc;"),
    "row_offset": ("if (j < dim) dt[t * dim + j] = acc;", "if (j < dim) dt[t * dim + (j + 1) % dim] = acc;"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(PROJ_MUTANTS))
def test_proj_mutant_is_caught(tmp_path, name):
    src = O.SRC.read_text()
    old, new = PROJ_MUTANTS[name]
    assert src.count(old) == 1, "mutation anchor missing or ambiguous: " + name
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / ("lib_%s.so" % name)
    O.build(force=True, src=path, out=so)
    lib = O.load(so)
    g = np.random.default_rng(4)
    dim, N, T = 24, 16, 5
    x, W = g.standard_normal((T, dim)), g.standard_normal((dim + 2 * N, dim))
    try:
        got = np.concatenate(O.proj(x, W, N, lib=lib), axis=1)
    except Exception:
        return
    assert not np.allclose(got, x @ W.T, rtol=1e-9, atol=1e-9), "pins did not reject mutant " + name
