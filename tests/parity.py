"""Comparison helpers for GPU-vs-oracle parity (imported by the GPU tests and the smoke check).

Tolerance (the stated contract is a maximum relative error of 2e-3 on y and
h_last with bf16 inputs and an fp32 state; read as):
  * fp32 outputs (h_last always; y when written as fp32): the error of each
    output tensor, per sequence, normalised by that tensor's largest oracle
    magnitude, max|g - o| / max|o| <= 2e-3;
  * bf16 y: one bf16 rounding of a value that meets the fp32 bar, i.e. per
    (sequence, channel) |g - o| <= 2^-8 |o| + 2e-3 * max|o|.
A relative elementwise reading is impossible: bf16 rounding alone is 3.9e-3
and y changes sign.  A tighter tripwire (TRIP) is also asserted on fp32
outputs; it follows from fp32 arithmetic (a few ulp per step, accumulated over
the state's memory) and exists to catch small bugs the contract would hide.
"""
from __future__ import annotations

import numpy as np

CONTRACT = 2e-3
TRIP = 1e-4
BF16_U = 2.0 ** -8


def norm_err(g, o) -> float:
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    if o.size == 0:
        return 0.0
    scale = float(np.max(np.abs(o)))
    diff = float(np.max(np.abs(g - o)))
    if scale == 0.0:
        return diff
    return diff / scale


# Per-(sequence, channel) diagnostic: the same error with each column normalised by its own largest oracle
# magnitude, so that a channel of small scale cannot hide under the largest channel of the sequence.
# Columns below this fraction of the sequence's largest magnitude are left out (their own scale is then
# rounding noise of the inputs, not a signal the contract speaks of).
CHANNEL_FLOOR = 1e-3
LAST_CHANNEL_ERR = {}


def channel_err(g, o, seq_bounds=None) -> float:
    """Worst per-(sequence, column) normalised error of 2-D [rows][columns] arrays (0 for other shapes)."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    if o.ndim != 2 or o.shape[1] < 2 or o.size == 0:
        return 0.0
    parts = [(0, len(o))] if seq_bounds is None else list(zip(seq_bounds[:-1], seq_bounds[1:]))
    worst = 0.0
    for a, b in parts:
        if b <= a:
            continue
        oo, gg = o[a:b], g[a:b]
        colmax = np.max(np.abs(oo), axis=0)
        keep = colmax > CHANNEL_FLOOR * max(float(np.max(colmax)), 1e-300)
        if not np.any(keep):
            continue
        e = np.max(np.abs(gg[:, keep] - oo[:, keep]), axis=0) / colmax[keep]
        worst = max(worst, float(np.max(e)))
    return worst


def check_fp32(g, o, what: str, seq_bounds=None, trip: float = TRIP) -> float:
    """fp32 output: per-sequence normalised error <= contract (and <= trip); for [rows][columns] outputs the
    per-(sequence, column) diagnostic must also meet the contract."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    assert np.all(np.isfinite(g)), what + ": non-finite GPU output"
    worst = 0.0
    parts = [(0, len(o))] if seq_bounds is None else list(zip(seq_bounds[:-1], seq_bounds[1:]))
    for a, b in parts:
        e = norm_err(g[a:b], o[a:b])
        worst = max(worst, e)
    assert worst <= CONTRACT, "%s: normalised error %.3e > contract %.1e" % (what, worst, CONTRACT)
    assert worst <= trip, "%s: normalised error %.3e > tripwire %.1e" % (what, worst, trip)
    ce = channel_err(g, o, seq_bounds)
    LAST_CHANNEL_ERR[what] = ce
    assert ce <= CONTRACT, "%s: per-(sequence, channel) error %.3e > contract %.1e" % (what, ce, CONTRACT)
    return worst


def check_bf16_y(g, o, what: str, seq_bounds=None) -> float:
    """bf16 y [tokens][dim]: |g - o| <= 2^-8 |o| + 2e-3 max|o| per (sequence, channel)."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    assert np.all(np.isfinite(g)), what + ": non-finite GPU output"
    parts = [(0, len(o))] if seq_bounds is None else list(zip(seq_bounds[:-1], seq_bounds[1:]))
    worst = 0.0
    for a, b in parts:
        if b <= a:
            continue
        oo, gg = o[a:b], g[a:b]
        colmax = np.max(np.abs(oo), axis=0, keepdims=True)
        bound = BF16_U * np.abs(oo) + CONTRACT * colmax
        ratio = np.abs(gg - oo) / np.maximum(bound, 1e-300)
        worst = max(worst, float(np.max(ratio)))
    assert worst <= 1.0, "%s: bf16 y exceeds one rounding + contract (worst ratio %.3f)" % (what, worst)
    return worst
