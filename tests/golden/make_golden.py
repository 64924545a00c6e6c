"""Writes oracle_small.json (the selective scan) and oracle_variants_small.json (the SSD layer and gated
linear attention): small seeded cases and the oracle's fp64 outputs.

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


def variants():
    lens = [7, 0, 11]
    ss = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, H, G, N = sum(lens), 4, 2, 8
    si = I.make_ssd_inputs_np(9, T, H, G, N, head_dim=4)
    h0s = I.make_ssd_h0(9, len(lens), H, N, head_dim=4, scale=0.5)
    ys, hs = O.ssd(si["x_f32"], si["dt_f32"], si["B_f32"], si["C_f32"], si["A"], si["D"], si["dt_bias"],
                   z=si["z_f32"], h0=h0s, seq_start=ss)
    gi = I.make_gla_inputs_np(10, T, 2, 8, 4)
    h0g = (0.5 * np.random.default_rng(10).standard_normal((len(lens), 2, 4, 8))).astype(np.float32)
    og, hg = O.gla(gi["q_f32"], gi["k_f32"], gi["v_f32"], gi["gk_f32"], h0=h0g, seq_start=ss)
    data = {
        "about": "seeded recipes (SSD config 9, GLA config 10; bf16-rounded inputs; packed lengths 7,0,11); "
                 "outputs of oracle/oracle.c",
        "seq_start": ss.tolist(),
        "ssd": {"inputs": {k: si[k + "_f32"].tolist() for k in ("x", "dt", "z", "B", "C")} |
                          {k: si[k].tolist() for k in ("A", "D", "dt_bias")} | {"h0": h0s.tolist()},
                "y": ys.tolist(), "h_last": hs.tolist()},
        "gla": {"inputs": {k: gi[k + "_f32"].tolist() for k in ("q", "k", "v", "gk")} | {"h0": h0g.tolist()},
                "o": og.tolist(), "h_last": hg.tolist()},
    }
    (Path(__file__).parent / "oracle_variants_small.json").write_text(json.dumps(data, indent=None,
                                                                                 separators=(",", ":")))


if __name__ == "__main__":
    main()
    variants()
