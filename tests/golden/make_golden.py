"""Writes oracle_small.json: a small seeded case and the oracle's fp64 outputs.

Calls only oracle/ (and the seeded input recipe); the stored values are a
regression fixture for the oracle itself, never an input to or output of the
GPU path.  Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import sys
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parents[2]
sys.path.insert(0, str(ROOT))
from oracle import oracle as O  # noqa: E402
from selective_state_space_05_amd import inputs as I  # noqa: E402


def main():
    lens = [5, 0, 9, 3]
    T, D, N = sum(lens), 4, 16
    inp = I.make_fwd_inputs_np(0, T, D, N, in_dtype="bf16")
    h0 = I.make_h0(0, len(lens), D, N, scale=0.5)
    ss = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    y, h = O.scan_fwd(inp["x_f32"], inp["dt_f32"], inp["z_f32"], inp["B_f32"], inp["C_f32"], inp["A"], inp["D"],
                      inp["dt_bias"], h0=h0, seq_start=ss)
    data = {
        "about": "seeded recipe (config 0 seeds, bf16-rounded inputs, packed lengths 5,0,9,3); outputs of oracle/oracle.c",
        "inputs": {"x": inp["x_f32"].tolist(), "dt": inp["dt_f32"].tolist(), "z": inp["z_f32"].tolist(),
                   "B": inp["B_f32"].tolist(), "C": inp["C_f32"].tolist(), "A": inp["A"].tolist(),
                   "D": inp["D"].tolist(), "dt_bias": inp["dt_bias"].tolist(), "h0": h0.tolist(),
                   "seq_start": ss.tolist()},
        "y": y.tolist(), "h_last": h.tolist(),
    }
    (Path(__file__).parent / "oracle_small.json").write_text(json.dumps(data, indent=None, separators=(",", ":")))


if __name__ == "__main__":
    main()
