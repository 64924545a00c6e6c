"""The comparison helpers the GPU parity tests use (host logic only)."""
import numpy as np
import pytest

from tests.parity import CONTRACT, channel_err, check_bf16_y, check_fp32, norm_err


def test_norm_err_is_normalised_by_the_largest_magnitude():
    o = np.array([[1.0, -4.0], [2.0, 0.5]])
    g = o + np.array([[0.0, 0.0], [0.04, 0.0]])
    assert norm_err(g, o) == pytest.approx(0.01)


def test_channel_diagnostic_sees_an_error_in_a_small_channel():
    rng = np.random.default_rng(0)
    o = rng.standard_normal((200, 8))
    o[:, 3] *= 1e-2                      # a channel of small scale
    g = o.copy()
    g[17, 3] += 5e-4                      # 5 % of that channel, 1e-4 of the tensor's max
    assert norm_err(g, o) < CONTRACT       # hidden under the tensor's max
    assert channel_err(g, o) > CONTRACT    # but not per channel
    with pytest.raises(AssertionError, match="per-\\(sequence, channel\\)"):
        check_fp32(g, o, "small channel", trip=1.0)


def test_channel_diagnostic_is_per_sequence_and_skips_silent_channels():
    o = np.ones((10, 3))
    o[:, 2] = 0.0                         # an all-zero channel has no scale of its own
    g = o.copy()
    g[:, 2] = 1e-9
    assert channel_err(g, o) == 0.0
    o2 = np.vstack([o, 100.0 * o])         # a second sequence of larger scale does not mask the first
    g2 = o2.copy()
    g2[3, 0] += 0.01
    assert channel_err(g2, o2, np.array([0, 10, 20])) == pytest.approx(0.01)
    assert channel_err(g2, o2) == pytest.approx(0.01 / 100.0)


def test_bf16_bound_allows_one_rounding():
    o = np.linspace(-3, 3, 64).reshape(16, 4)
    g = o * (1 + 2.0 ** -9)
    assert check_bf16_y(g, o, "one rounding") <= 1.0
    with pytest.raises(AssertionError):
        check_bf16_y(o * (1 + 2.0 ** -6), o, "three roundings")
