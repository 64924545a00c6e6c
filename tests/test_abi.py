"""C ABI checks that need no GPU: symbols, struct layout, validation codes, launch plan.

Validation runs on the host before any HIP call, so every invalid-argument case
returns its documented status here without a device.  Pointers are fake,
never-dereferenced addresses.
"""
import ctypes
import os
import re
import subprocess
from pathlib import Path

import pytest

from selective_state_space_05_amd import scan as S
from selective_state_space_05_amd import gla as GL
from selective_state_space_05_amd import ssd as D
from selective_state_space_05_amd import swa as W

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "samba_scan.h"
PROBE_HEADER = ROOT / "include" / "samba_probe.h"
HEADERS = sorted(h for h in (ROOT / "include").glob("*.h") if h != PROBE_HEADER)


# tests/test_abi_sanitized.py runs this file against a host-sanitized build of the library
LIB_OVERRIDE = os.environ.get("SAMBA_ABI_TEST_LIBRARY")


@pytest.fixture(scope="module")
def lib():
    D.load_library(LIB_OVERRIDE)
    GL.load_library(LIB_OVERRIDE)
    return W.load_library(LIB_OVERRIDE)


def header_functions(headers=HEADERS):
    names = set()
    for h in headers:
        txt = re.sub(r"/\*.*?\*/", "", h.read_text(), flags=re.S)
        names |= set(re.findall(r"\b(samba_\w+)\s*\(", txt))
    return sorted(names)


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert set(names) == set(S.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_probe_library_exports_its_header():
    """libsamba_probe.so (the ALU issue-rate probes) exports every function samba_probe.h declares."""
    from selective_state_space_05_amd import probe as PR
    plib = PR.load_library()
    names = header_functions([PROBE_HEADER])
    assert names == ["samba_probe_alu", "samba_probe_instructions_per_round"]
    for n in names:
        assert hasattr(plib, n), n
    assert PR.instructions_per_round("fmac_vop2") == 16 and PR.instructions_per_round("fma_vop3") == 32
    assert PR.instructions_per_round("mix_4fmac_1exp") == 80
    assert plib.samba_probe_instructions_per_round(99) == 0
    # bad arguments are refused on the host, before any HIP call
    assert plib.samba_probe_alu(0, 0, 1, ctypes.c_void_p(64), None) == 1
    assert plib.samba_probe_alu(0, 1, 1, None, None) == 1
    assert plib.samba_probe_alu(99, 1, 1, ctypes.c_void_p(64), None) == 1


def test_abi_version_and_state_size(lib):
    assert lib.samba_scan_abi_version() == S.ABI_VERSION
    txt = HEADER.read_text()
    assert re.search(r"#define SAMBA_DSTATE 16\b", txt)
    assert re.search(r"#define SAMBA_SCAN_ABI_VERSION %d\b" % S.ABI_VERSION, txt)


def test_status_strings(lib):
    for code in range(10):
        assert lib.samba_status_string(code)
    assert lib.samba_status_string(12345) == b"unknown status"


STRUCTS = (("samba_scan_fwd_args", S.FwdArgs), ("samba_scan_step_args", S.StepArgs),
           ("samba_scan_bwd_args", S.BwdArgs), ("samba_proj_args", S.ProjArgs), ("samba_rope_args", W.RopeArgs),
           ("samba_swa_fwd_args", W.SwaFwdArgs), ("samba_swa_decode_args", W.SwaDecodeArgs),
           ("samba_scan_groups_args", S.GroupsArgs), ("samba_scan_step_groups_args", S.StepGroupsArgs),
           ("samba_ssd_args", D.SsdArgs), ("samba_gla_args", GL.GlaArgs))


def test_struct_layout_matches_header(tmp_path):
    """Compile a C probe against the header and compare sizeof/offsetof with the ctypes mirrors."""
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "samba_scan.h"', '#include "samba_swa.h"',
             '#include "samba_ssd.h"', '#include "samba_gla.h"', 'int main(void) {']
    for cname, py in STRUCTS:
        lines.append('printf("%s %%zu\\n", sizeof(%s));' % (cname, cname))
        for f, _ in py._fields_:
            lines.append('printf("%s.%s %%zu\\n", offsetof(%s, %s));' % (cname, f, cname, f))
    lines.append("return 0; }")
    src = tmp_path / "probe.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "probe"
    subprocess.check_call(["gcc", "-std=c99", "-I", str(ROOT / "include"), "-o", str(exe), str(src)])
    got = dict(l.split() for l in subprocess.check_output([str(exe)]).decode().splitlines())
    for cname, py in STRUCTS:
        assert int(got[cname]) == ctypes.sizeof(py)
        for f, _ in py._fields_:
            assert int(got["%s.%s" % (cname, f)]) == getattr(py, f).offset, (cname, f)


# --------------------------------------------------------------------------- #
# validation
# --------------------------------------------------------------------------- #
BASE = 0x7f0000000000


def fwd_ok(batch=2, seqlen=100, dim=64, in_dtype=S.SAMBA_BF16, y_dtype=S.SAMBA_BF16):
    a = S.FwdArgs()
    a.struct_size = ctypes.sizeof(S.FwdArgs)
    a.batch, a.seqlen, a.dim, a.dstate = batch, seqlen, dim, 16
    a.in_dtype, a.y_dtype = in_dtype, y_dtype
    gb = 1 << 30
    a.x, a.dt, a.z, a.B, a.C = BASE, BASE + gb, BASE + 2 * gb, BASE + 3 * gb, BASE + 4 * gb
    a.A, a.D, a.dt_bias = BASE + 5 * gb, BASE + 6 * gb, BASE + 7 * gb
    a.h0, a.h_last, a.y = BASE + 8 * gb, BASE + 9 * gb, BASE + 10 * gb
    return a


def step_ok(batch=4, dim=64):
    a = S.StepArgs()
    a.struct_size = ctypes.sizeof(S.StepArgs)
    a.batch, a.dim, a.dstate = batch, dim, 16
    a.in_dtype, a.y_dtype = S.SAMBA_BF16, S.SAMBA_BF16
    gb = 1 << 30
    a.state, a.x, a.dt, a.z, a.B, a.C = BASE, BASE + gb, BASE + 2 * gb, BASE + 3 * gb, BASE + 4 * gb, BASE + 5 * gb
    a.A, a.D, a.dt_bias, a.y = BASE + 6 * gb, BASE + 7 * gb, BASE + 8 * gb, BASE + 9 * gb
    return a


def plan(lib, a, with_lanes=False):
    w, g, t, q = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    st = lib.samba_scan_fwd_plan(ctypes.byref(a), ctypes.byref(w), ctypes.byref(g), ctypes.byref(t), ctypes.byref(q))
    return (st, w.value, g.value, t.value, q.value) if with_lanes else (st, w.value, g.value, t.value)


FWD_CASES = {
    "struct_size": (lambda a: setattr(a, "struct_size", 8), 7),
    "dstate": (lambda a: setattr(a, "dstate", 8), 6),
    "in_dtype": (lambda a: setattr(a, "in_dtype", 7), 3),
    "y_dtype": (lambda a: setattr(a, "y_dtype", -1), 3),
    "neg_batch": (lambda a: setattr(a, "batch", -1), 2),
    "neg_seqlen": (lambda a: setattr(a, "seqlen", -5), 2),
    "zero_dim": (lambda a: setattr(a, "dim", 0), 2),
    "dim_2_pow_24": (lambda a: setattr(a, "dim", 1 << 24), 2),   # slice byte offsets must stay in 32 bits
    "time_slices": (lambda a: setattr(a, "time_slices", 3), 6),
    "time_slices_32": (lambda a: setattr(a, "time_slices", 32), 6),
    "null_x": (lambda a: setattr(a, "x", None), 1),
    "null_A": (lambda a: setattr(a, "A", None), 1),
    "null_y": (lambda a: setattr(a, "y", None), 1),
    "null_B": (lambda a: setattr(a, "B", None), 1),
    "misaligned_B": (lambda a: setattr(a, "B", a.B + 8), 4),
    "misaligned_h0": (lambda a: setattr(a, "h0", a.h0 + 4), 4),
    "misaligned_x": (lambda a: setattr(a, "x", a.x + 1), 4),
    "misaligned_y_f32": (lambda a: (setattr(a, "y_dtype", S.SAMBA_F32), setattr(a, "y", a.y + 2)), 4),
    "y_overlaps_x": (lambda a: setattr(a, "y", a.x + 64), 5),
    "h_last_overlaps_h0": (lambda a: setattr(a, "h_last", a.h0 + 64), 5),
    "h_last_overlaps_A": (lambda a: setattr(a, "h_last", a.A), 5),
    "misaligned_h_ckpt": (lambda a: setattr(a, "h_ckpt", BASE + 12 * (1 << 30) + 8), 4),
    "h_ckpt_overlaps_x": (lambda a: setattr(a, "h_ckpt", a.x + 64), 5),
    "h_ckpt_overlaps_y": (lambda a: setattr(a, "h_ckpt", a.y), 5),
    "varlen_batch": (lambda a: (setattr(a, "cu_seqlens", BASE + 11 * (1 << 30)), setattr(a, "nseq", 3)), 2),
    "varlen_nseq0": (lambda a: (setattr(a, "batch", 1), setattr(a, "cu_seqlens", BASE + 11 * (1 << 30)),
                                setattr(a, "nseq", 0)), 2),
}


@pytest.mark.parametrize("name", sorted(FWD_CASES))
def test_fwd_rejects(lib, name):
    a = fwd_ok()
    mutate, code = FWD_CASES[name]
    mutate(a)
    assert lib.samba_scan_fwd(ctypes.byref(a), None) == code
    assert plan(lib, a)[0] == code


def test_fwd_null_args(lib):
    assert lib.samba_scan_fwd(None, None) == 1
    assert lib.samba_scan_step(None, None) == 1


def test_fwd_in_place_carry_allowed(lib):
    a = fwd_ok()
    a.h_last = a.h0
    assert plan(lib, a)[0] == 0


def test_fwd_largest_dim_accepted(lib):
    """dim = 2^24 - 1 is the largest the prefill takes (one token: every buffer fits its 1 GiB slot)."""
    assert plan(lib, fwd_ok(batch=1, seqlen=1, dim=(1 << 24) - 1))[0] == 0


def test_fwd_no_tokens_allows_null_token_pointers(lib):
    a = fwd_ok(seqlen=0)
    a.x = a.dt = a.z = a.B = a.C = a.y = None
    assert plan(lib, a)[0] == 0


STEP_CASES = {
    "struct_size": (lambda a: setattr(a, "struct_size", 4), 7),
    "dstate": (lambda a: setattr(a, "dstate", 32), 6),
    "dtype": (lambda a: setattr(a, "in_dtype", 5), 3),
    "neg_batch": (lambda a: setattr(a, "batch", -2), 2),
    "null_state": (lambda a: setattr(a, "state", None), 1),
    "null_C": (lambda a: setattr(a, "C", None), 1),
    "misaligned_state": (lambda a: setattr(a, "state", a.state + 4), 4),
    "misaligned_C": (lambda a: setattr(a, "C", a.C + 8), 4),
    "y_overlaps_state": (lambda a: setattr(a, "y", a.state + 16), 5),
    "state_overlaps_x": (lambda a: setattr(a, "state", a.x), 5),
}


@pytest.mark.parametrize("name", sorted(STEP_CASES))
def test_step_rejects(lib, name):
    a = step_ok()
    mutate, code = STEP_CASES[name]
    mutate(a)
    assert lib.samba_scan_step(ctypes.byref(a), None) == code


def test_step_empty_batch_is_noop(lib):
    a = step_ok(batch=0)
    assert lib.samba_scan_step(ctypes.byref(a), None) == 0


# --------------------------------------------------------------------------- #
# launch plan (host logic; falls back to 256 CUs when no device is visible)
# --------------------------------------------------------------------------- #
def test_plan_low_parallelism_splits_time(lib):
    """One long sequence of 4096 channels: one 16-wave workgroup per 16-channel tile (256 on 256 CUs)."""
    a = fwd_ok(batch=1, seqlen=16384, dim=4096)
    assert plan(lib, a, True) == (0, 16, 256, 1024, 4)
    a.lanes_per_channel = 8     # forced: 8-channel tiles, two 8-wave workgroups per CU
    assert plan(lib, a, True) == (0, 8, 512, 512, 8)


def test_plan_half_gpu_shape_uses_eight_lanes(lib):
    """B1 L4096 D2048: 128 sixteen-channel tiles would leave half of 256 CUs idle; 256 eight-channel tiles."""
    a = fwd_ok(batch=1, seqlen=4096, dim=2048)
    assert plan(lib, a, True) == (0, 16, 256, 1024, 8)


def test_plan_eight_lanes_rules(lib):
    a = fwd_ok(batch=1, seqlen=1000, dim=100)
    a.lanes_per_channel = 8
    for ts in (2, 4, 8, 16):
        a.time_slices = ts
        assert plan(lib, a, True) == (0, ts, 13, 64 * ts, 8)
    a.time_slices = 1                       # no sequential 8-lane kernel
    assert plan(lib, a)[0] == 6 and lib.samba_scan_fwd(ctypes.byref(a), None) == 6
    a.time_slices = 0
    a.h_ckpt = BASE + 12 * (1 << 30)        # checkpoints come from the 4-lane kernel only
    assert plan(lib, a)[0] == 6
    a.lanes_per_channel = 0                 # automatic: checkpoints keep 4 lanes
    assert plan(lib, a, True)[4] == 4
    a.h_ckpt = None
    for bad in (1, 2, 3, 16, -4):
        a.lanes_per_channel = bad
        assert plan(lib, a)[0] == 6 and lib.samba_scan_fwd(ctypes.byref(a), None) == 6


def test_plan_batched_runs_sequential(lib):
    a = fwd_ok(batch=64, seqlen=2048, dim=4096)
    st, w, g, t = plan(lib, a)
    assert st == 0 and w == 1 and t == 256 and g == 64 * 64


def test_plan_short_sequences_limit_slices(lib):
    """Time is split only into slices (8 tokens each) that the average sequence fills at least twice over."""
    for seqlen, want in ((12, 1), (20, 2), (40, 4)):
        a = fwd_ok(batch=1, seqlen=seqlen, dim=64)
        a.lanes_per_channel = 4
        st, w, g, t = plan(lib, a)
        assert st == 0 and w == want, (seqlen, w)
    # automatic lanes: 8 only where 16-token slices still split the sequence at least twice
    for seqlen, want in ((12, (1, 4)), (20, (2, 4)), (40, (2, 8)), (100, (2, 8)))[:3]:
        a = fwd_ok(batch=1, seqlen=seqlen, dim=64)
        st, w, g, t, q = plan(lib, a, True)
        assert st == 0 and (w, q) == want, (seqlen, w, q)


def test_plan_forced_slices(lib):
    for ts in (1, 2, 4, 8, 16):
        a = fwd_ok(batch=1, seqlen=1000, dim=100)
        a.time_slices = ts
        a.lanes_per_channel = 4
        st, w, g, t = plan(lib, a)
        assert st == 0 and w == ts
        assert g == (7 if ts > 1 else 2) and t == (64 * ts if ts > 1 else 256)


# --------------------------------------------------------------------------- #
# backward: workspace size and validation
# --------------------------------------------------------------------------- #
def bwd_ok(batch=2, seqlen=100, dim=64, in_dtype=S.SAMBA_BF16):
    a = S.BwdArgs()
    a.struct_size = ctypes.sizeof(S.BwdArgs)
    a.batch, a.seqlen, a.dim, a.dstate = batch, seqlen, dim, 16
    a.in_dtype = in_dtype
    gb = 1 << 30
    names = ("x", "dt", "z", "B", "C", "A", "D", "dt_bias", "h0", "dy", "dh_last", "dx", "ddt", "dz", "dB", "dC",
             "dA", "dD", "ddt_bias", "dh0", "workspace")
    for i, n in enumerate(names):
        setattr(a, n, BASE + i * gb)
    a.workspace_bytes = 1 << 29
    return a


def ws_bytes(lib, a):
    n = ctypes.c_size_t()
    st = lib.samba_scan_bwd_workspace_size(ctypes.byref(a), ctypes.byref(n))
    return st, n.value


def r256(v):
    return (v + 255) // 256 * 256


@pytest.mark.parametrize("batch,seqlen,dim", [(2, 100, 64), (4, 4096, 4096), (1, 0, 16), (3, 7, 40)])
def test_bwd_workspace_size(lib, batch, seqlen, dim):
    """checkpoints (state before every 8th token of each sequence) + per-tile dB/dC partial rows +
    per-sequence parameter partial rows, each rounded up to 256 bytes."""
    a = bwd_ok(batch, seqlen, dim)
    st, n = ws_bytes(lib, a)
    tokens, tiles = batch * seqlen, (dim + 15) // 16
    want = r256((tokens // 8 + batch + 1) * dim * 64) + r256(tiles * tokens * 128) + r256(batch * dim * 80)
    assert st == 0 and n == want


BWD_CASES = {
    "struct_size": (lambda a: setattr(a, "struct_size", 8), 7),
    "dstate": (lambda a: setattr(a, "dstate", 4), 6),
    "in_dtype": (lambda a: setattr(a, "in_dtype", 2), 3),
    "neg_seqlen": (lambda a: setattr(a, "seqlen", -1), 2),
    "dim_2_pow_24": (lambda a: setattr(a, "dim", 1 << 24), 2),
    "time_slices_16": (lambda a: setattr(a, "time_slices", 16), 6),
    "time_slices_3": (lambda a: setattr(a, "time_slices", 3), 6),
    "null_dy": (lambda a: setattr(a, "dy", None), 1),
    "null_dB": (lambda a: setattr(a, "dB", None), 1),
    "null_dA": (lambda a: setattr(a, "dA", None), 1),
    "null_workspace": (lambda a: setattr(a, "workspace", None), 9),
    "small_workspace": (lambda a: setattr(a, "workspace_bytes", 1024), 9),
    "misaligned_workspace": (lambda a: setattr(a, "workspace", a.workspace + 64), 9),
    "misaligned_dB": (lambda a: setattr(a, "dB", a.dB + 4), 4),
    "misaligned_dh_last": (lambda a: setattr(a, "dh_last", a.dh_last + 8), 4),
    "misaligned_dx": (lambda a: setattr(a, "dx", a.dx + 1), 4),
    "dx_overlaps_x": (lambda a: setattr(a, "dx", a.x + 2), 5),
    "dB_overlaps_dC": (lambda a: setattr(a, "dB", a.dC + 16), 5),
    "workspace_overlaps_dy": (lambda a: setattr(a, "workspace", a.dy), 5),
    "dh0_overlaps_h0": (lambda a: setattr(a, "dh0", a.h0), 5),
    "varlen_batch": (lambda a: (setattr(a, "cu_seqlens", BASE + 40 * (1 << 30)), setattr(a, "nseq", 3)), 2),
    "misaligned_h_ckpt": (lambda a: setattr(a, "h_ckpt", BASE + 41 * (1 << 30) + 4), 4),
    "h_ckpt_overlaps_dx": (lambda a: setattr(a, "h_ckpt", a.dx), 5),
}


@pytest.mark.parametrize("name", sorted(BWD_CASES))
def test_bwd_rejects(lib, name):
    a = bwd_ok()
    mutate, code = BWD_CASES[name]
    mutate(a)
    assert lib.samba_scan_bwd(ctypes.byref(a), None) == code


def test_ckpt_bytes(lib):
    """h_ckpt holds slots = tokens/8 + nseq + 1 rows of dim x 16 fp32 states."""
    n = ctypes.c_size_t()
    for batch, seqlen, nseq, dim in ((4, 4096, 4, 4096), (1, 100, 7, 40), (2, 0, 2, 16)):
        assert lib.samba_scan_ckpt_bytes(batch, seqlen, nseq, dim, ctypes.byref(n)) == 0
        assert n.value == (batch * seqlen // 8 + nseq + 1) * dim * 64
    assert lib.samba_scan_ckpt_bytes(1, 8, 1, 0, ctypes.byref(n)) == 2
    assert lib.samba_scan_ckpt_bytes(1, 8, 1, 1 << 24, ctypes.byref(n)) == 2
    assert lib.samba_scan_ckpt_bytes(1, 8, 1, 8, None) == 1


def test_bwd_workspace_without_checkpoint_section(lib):
    a = bwd_ok(4, 4096, 4096)
    st, full = ws_bytes(lib, a)
    a.h_ckpt = BASE + 42 * (1 << 30)
    st2, small = ws_bytes(lib, a)
    assert st == st2 == 0 and full - small == r256((4 * 4096 // 8 + 4 + 1) * 4096 * 64)


def test_bwd_null_args(lib):
    assert lib.samba_scan_bwd(None, None) == 1
    n = ctypes.c_size_t()
    assert lib.samba_scan_bwd_workspace_size(None, ctypes.byref(n)) == 1
    assert lib.samba_scan_bwd_workspace_size(ctypes.byref(bwd_ok()), None) == 1


# --------------------------------------------------------------------------- #
# selection projections: validation
# --------------------------------------------------------------------------- #
def proj_ok(tokens=100, dim=64, dstate=16):
    a = S.ProjArgs()
    a.struct_size = ctypes.sizeof(S.ProjArgs)
    a.tokens, a.dim, a.dstate = tokens, dim, dstate
    a.in_dtype, a.out_dtype = S.SAMBA_BF16, S.SAMBA_BF16
    gb = 1 << 30
    a.x, a.W, a.dt, a.B, a.C = BASE, BASE + gb, BASE + 2 * gb, BASE + 3 * gb, BASE + 4 * gb
    return a


PROJ_CASES = {
    "struct_size": (lambda a: setattr(a, "struct_size", 4), 7),
    "f32_inputs": (lambda a: setattr(a, "in_dtype", S.SAMBA_F32), 3),
    "out_dtype": (lambda a: setattr(a, "out_dtype", 9), 3),
    "dim_not_multiple_of_8": (lambda a: setattr(a, "dim", 60), 2),
    "dim_2_pow_22": (lambda a: setattr(a, "dim", 1 << 22), 2),   # 256-row tile byte offsets past 2^31
    "neg_tokens": (lambda a: setattr(a, "tokens", -1), 2),
    "zero_dstate": (lambda a: setattr(a, "dstate", 0), 2),
    "null_W": (lambda a: setattr(a, "W", None), 1),
    "null_dt": (lambda a: setattr(a, "dt", None), 1),
    "misaligned_x": (lambda a: setattr(a, "x", a.x + 8), 4),
    "misaligned_dt": (lambda a: setattr(a, "dt", a.dt + 1), 4),
    "dt_overlaps_x": (lambda a: setattr(a, "dt", a.x + 64), 5),
    "B_overlaps_C": (lambda a: setattr(a, "B", a.C + 2), 5),
}


@pytest.mark.parametrize("name", sorted(PROJ_CASES))
def test_proj_rejects(lib, name):
    a = proj_ok()
    mutate, code = PROJ_CASES[name]
    mutate(a)
    assert lib.samba_proj(ctypes.byref(a), None) == code


def test_proj_no_tokens_is_noop(lib):
    a = proj_ok(tokens=0)
    a.x = a.dt = a.B = a.C = None
    assert lib.samba_proj(ctypes.byref(a), None) == 0
    assert lib.samba_proj(None, None) == 1


# --------------------------------------------------------------------------- #
# sliding-window attention: validation
# --------------------------------------------------------------------------- #
GB = 1 << 30


def rope_ok(batch=2, seqlen=100, heads=4, hd=128):
    a = W.RopeArgs()
    a.struct_size = ctypes.sizeof(W.RopeArgs)
    a.batch, a.seqlen, a.heads, a.head_dim = batch, seqlen, heads, hd
    a.cos, a.sin, a.npos = BASE, BASE + GB, 4096
    a.q_in, a.k_in, a.q_out, a.k_out = BASE + 2 * GB, BASE + 3 * GB, BASE + 4 * GB, BASE + 5 * GB
    return a


ROPE_CASES = {
    "struct_size": (lambda a: setattr(a, "struct_size", 4), 7),
    "neg_batch": (lambda a: setattr(a, "batch", -1), 2),
    "zero_heads": (lambda a: setattr(a, "heads", 0), 2),
    "head_dim_not_16": (lambda a: setattr(a, "head_dim", 72), 2),
    "zero_npos": (lambda a: setattr(a, "npos", 0), 2),
    "head_dim_too_large": (lambda a: setattr(a, "head_dim", 4112), 2),
    "too_many_features": (lambda a: setattr(a, "heads", 8193), 2),
    "varlen_batch": (lambda a: (setattr(a, "cu_seqlens", BASE + 6 * GB), setattr(a, "nseq", 2)), 2),
    "varlen_nseq0": (lambda a: (setattr(a, "batch", 1), setattr(a, "cu_seqlens", BASE + 6 * GB)), 2),
    "null_cos": (lambda a: setattr(a, "cos", None), 1),
    "q_in_without_out": (lambda a: setattr(a, "q_out", None), 1),
    "k_out_without_in": (lambda a: setattr(a, "k_in", None), 1),
    "misaligned_q": (lambda a: setattr(a, "q_in", a.q_in + 2), 4),
    "misaligned_sin": (lambda a: setattr(a, "sin", a.sin + 4), 4),
    "q_out_overlaps_k_in": (lambda a: setattr(a, "q_out", a.k_in + 256), 5),
    "k_out_shifted_on_k_in": (lambda a: setattr(a, "k_out", a.k_in + 16), 5),
    "q_out_overlaps_k_out": (lambda a: setattr(a, "q_out", a.k_out), 5),
    "k_out_overlaps_cos": (lambda a: setattr(a, "k_out", a.cos), 5),
}


@pytest.mark.parametrize("name", sorted(ROPE_CASES))
def test_rope_rejects(lib, name):
    a = rope_ok()
    mutate, code = ROPE_CASES[name]
    mutate(a)
    assert lib.samba_rope(ctypes.byref(a), None) == code


def test_rope_noops(lib):
    a = rope_ok(seqlen=0)
    a.q_in = a.k_in = a.q_out = a.k_out = None
    assert lib.samba_rope(ctypes.byref(a), None) == 0
    a = rope_ok()
    a.q_in = a.k_in = a.q_out = a.k_out = None   # nothing to rotate
    assert lib.samba_rope(ctypes.byref(a), None) == 0
    assert lib.samba_rope(None, None) == 1


def swa_ok(batch=2, seqlen=300, heads=4, hd=128, out_dtype=S.SAMBA_BF16):
    a = W.SwaFwdArgs()
    a.struct_size = ctypes.sizeof(W.SwaFwdArgs)
    a.batch, a.seqlen, a.heads, a.head_dim = batch, seqlen, heads, hd
    a.window, a.out_dtype = 64, out_dtype
    a.q, a.k, a.v, a.o = BASE, BASE + GB, BASE + 2 * GB, BASE + 3 * GB
    return a


SWA_CASES = {
    "struct_size": (lambda a: setattr(a, "struct_size", 4), 7),
    "head_dim_64": (lambda a: setattr(a, "head_dim", 64), 6),
    "neg_window": (lambda a: setattr(a, "window", -1), 2),
    "zero_heads": (lambda a: setattr(a, "heads", 0), 2),
    "too_many_heads": (lambda a: setattr(a, "heads", 5000), 2),
    "neg_seqlen": (lambda a: setattr(a, "seqlen", -1), 2),
    "out_dtype": (lambda a: setattr(a, "out_dtype", 5), 3),
    "varlen_batch": (lambda a: (setattr(a, "cu_seqlens", BASE + 5 * GB), setattr(a, "nseq", 2)), 2),
    "null_v": (lambda a: setattr(a, "v", None), 1),
    "null_o": (lambda a: setattr(a, "o", None), 1),
    "misaligned_k": (lambda a: setattr(a, "k", a.k + 8), 4),
    "misaligned_o_f32": (lambda a: (setattr(a, "out_dtype", S.SAMBA_F32), setattr(a, "o", a.o + 2)), 4),
    "o_overlaps_q": (lambda a: setattr(a, "o", a.q + 128), 5),
    "o_overlaps_v": (lambda a: setattr(a, "o", a.v), 5),
    "o_overlaps_cu": (lambda a: (setattr(a, "batch", 1), setattr(a, "cu_seqlens", a.o + 64), setattr(a, "nseq", 2)), 5),
}


@pytest.mark.parametrize("name", sorted(SWA_CASES))
def test_swa_fwd_rejects(lib, name):
    a = swa_ok()
    mutate, code = SWA_CASES[name]
    mutate(a)
    assert lib.samba_swa_fwd(ctypes.byref(a), None) == code


def test_swa_fwd_no_tokens_is_noop(lib):
    a = swa_ok(seqlen=0)
    a.q = a.k = a.v = a.o = None
    assert lib.samba_swa_fwd(ctypes.byref(a), None) == 0
    assert lib.samba_swa_fwd(None, None) == 1


def dec_ok(batch=4, heads=4, hd=128, window=64, cache_len=65):
    a = W.SwaDecodeArgs()
    a.struct_size = ctypes.sizeof(W.SwaDecodeArgs)
    a.batch, a.heads, a.head_dim, a.window, a.cache_len = batch, heads, hd, window, cache_len
    a.out_dtype = S.SAMBA_BF16
    a.pos, a.q, a.k, a.v = BASE, BASE + GB, BASE + 2 * GB, BASE + 3 * GB
    a.k_cache, a.v_cache, a.o = BASE + 4 * GB, BASE + 5 * GB, BASE + 6 * GB
    return a


DEC_CASES = {
    "struct_size": (lambda a: setattr(a, "struct_size", 4), 7),
    "head_dim_64": (lambda a: setattr(a, "head_dim", 64), 6),
    "cache_shorter_than_window": (lambda a: setattr(a, "cache_len", 64), 2),
    "neg_window": (lambda a: setattr(a, "window", -1), 2),
    "zero_heads": (lambda a: setattr(a, "heads", 0), 2),
    "out_dtype": (lambda a: setattr(a, "out_dtype", 3), 3),
    "null_pos": (lambda a: setattr(a, "pos", None), 1),
    "null_k_cache": (lambda a: setattr(a, "k_cache", None), 1),
    "misaligned_v_cache": (lambda a: setattr(a, "v_cache", a.v_cache + 8), 4),
    "misaligned_pos": (lambda a: setattr(a, "pos", a.pos + 2), 4),
    "o_overlaps_q": (lambda a: setattr(a, "o", a.q), 5),
    "k_cache_overlaps_v_cache": (lambda a: setattr(a, "k_cache", a.v_cache + 256), 5),
    "v_cache_overlaps_v": (lambda a: setattr(a, "v_cache", a.v - 256), 5),
    "o_overlaps_pos": (lambda a: setattr(a, "o", a.pos), 5),
}


@pytest.mark.parametrize("name", sorted(DEC_CASES))
def test_swa_decode_rejects(lib, name):
    a = dec_ok()
    mutate, code = DEC_CASES[name]
    mutate(a)
    assert lib.samba_swa_decode(ctypes.byref(a), None) == code


def test_swa_decode_empty_batch_is_noop(lib):
    a = dec_ok(batch=0)
    a.pos = a.q = a.k = a.v = a.k_cache = a.v_cache = a.o = None
    assert lib.samba_swa_decode(ctypes.byref(a), None) == 0


# --------------------------------------------------------------------------- #
# grouped prefill: validation
# --------------------------------------------------------------------------- #
def groups_ok(batch=2, seqlen=100, dim=64, dstate=32, ngroups=2):
    a = S.GroupsArgs()
    a.struct_size = ctypes.sizeof(S.GroupsArgs)
    a.batch, a.seqlen, a.dim, a.dstate, a.ngroups = batch, seqlen, dim, dstate, ngroups
    a.in_dtype, a.y_dtype = S.SAMBA_BF16, S.SAMBA_BF16
    a.x, a.dt, a.z, a.B, a.C = BASE, BASE + GB, BASE + 2 * GB, BASE + 3 * GB, BASE + 4 * GB
    a.A, a.D, a.dt_bias = BASE + 5 * GB, BASE + 6 * GB, BASE + 7 * GB
    a.h0, a.h_last, a.y = BASE + 8 * GB, BASE + 9 * GB, BASE + 10 * GB
    return a


GROUPS_CASES = {
    "struct_size": (lambda a: setattr(a, "struct_size", 4), 7),
    "dstate_24": (lambda a: setattr(a, "dstate", 24), 6),
    "dstate_8": (lambda a: setattr(a, "dstate", 8), 6),
    "groups_not_dividing": (lambda a: setattr(a, "ngroups", 3), 2),
    "group_not_whole_waves": (lambda a: (setattr(a, "dstate", 16), setattr(a, "ngroups", 8)), 2),
    "zero_groups": (lambda a: setattr(a, "ngroups", 0), 2),
    "neg_seqlen": (lambda a: setattr(a, "seqlen", -1), 2),
    "in_dtype": (lambda a: setattr(a, "in_dtype", 4), 3),
    "null_B": (lambda a: setattr(a, "B", None), 1),
    "null_A": (lambda a: setattr(a, "A", None), 1),
    "misaligned_C": (lambda a: setattr(a, "C", a.C + 8), 4),
    "misaligned_h_last": (lambda a: setattr(a, "h_last", a.h_last + 4), 4),
    "y_overlaps_B": (lambda a: setattr(a, "y", a.B + 64), 5),
    "h_last_overlaps_h0_shifted": (lambda a: setattr(a, "h_last", a.h0 + 16), 5),
    "varlen_batch": (lambda a: (setattr(a, "cu_seqlens", BASE + 11 * GB), setattr(a, "nseq", 3)), 2),
}


@pytest.mark.parametrize("name", sorted(GROUPS_CASES))
def test_groups_rejects(lib, name):
    a = groups_ok()
    mutate, code = GROUPS_CASES[name]
    mutate(a)
    assert lib.samba_scan_fwd_groups(ctypes.byref(a), None) == code


def test_groups_no_sequences_is_noop(lib):
    a = groups_ok(batch=0)
    assert lib.samba_scan_fwd_groups(ctypes.byref(a), None) == 0
    assert lib.samba_scan_fwd_groups(None, None) == 1


def step_groups_ok(batch=4, dim=64, dstate=64, ngroups=4):
    a = S.StepGroupsArgs()
    a.struct_size = ctypes.sizeof(S.StepGroupsArgs)
    a.batch, a.dim, a.dstate, a.ngroups = batch, dim, dstate, ngroups
    a.in_dtype, a.y_dtype = S.SAMBA_BF16, S.SAMBA_F32
    a.state, a.x, a.dt, a.z, a.B, a.C = BASE, BASE + GB, BASE + 2 * GB, BASE + 3 * GB, BASE + 4 * GB, BASE + 5 * GB
    a.A, a.D, a.dt_bias, a.y = BASE + 6 * GB, BASE + 7 * GB, BASE + 8 * GB, BASE + 9 * GB
    return a


STEP_GROUPS_CASES = {
    "struct_size": (lambda a: setattr(a, "struct_size", 4), 7),
    "dstate_48": (lambda a: setattr(a, "dstate", 48), 6),
    "groups_not_dividing": (lambda a: setattr(a, "ngroups", 3), 2),
    "neg_batch": (lambda a: setattr(a, "batch", -2), 2),
    "y_dtype": (lambda a: setattr(a, "y_dtype", 9), 3),
    "null_state": (lambda a: setattr(a, "state", None), 1),
    "misaligned_state": (lambda a: setattr(a, "state", a.state + 8), 4),
    "y_overlaps_state": (lambda a: setattr(a, "y", a.state + 64), 5),
    "state_overlaps_B": (lambda a: setattr(a, "state", a.B), 5),
}


@pytest.mark.parametrize("name", sorted(STEP_GROUPS_CASES))
def test_step_groups_rejects(lib, name):
    a = step_groups_ok()
    mutate, code = STEP_GROUPS_CASES[name]
    mutate(a)
    assert lib.samba_scan_step_groups(ctypes.byref(a), None) == code


def test_step_groups_empty_batch_is_noop(lib):
    a = step_groups_ok(batch=0)
    assert lib.samba_scan_step_groups(ctypes.byref(a), None) == 0


# --------------------------------------------------------------------------- #
# state-space duality prefill: validation
# --------------------------------------------------------------------------- #
def ssd_ok(batch=2, seqlen=100, heads=8, dstate=128, ngroups=2):
    a = D.SsdArgs()
    a.struct_size = ctypes.sizeof(D.SsdArgs)
    a.batch, a.seqlen, a.heads, a.head_dim, a.dstate, a.ngroups = batch, seqlen, heads, 64, dstate, ngroups
    a.y_dtype = S.SAMBA_BF16
    a.x, a.dt, a.z, a.B, a.C = BASE, BASE + GB, BASE + 2 * GB, BASE + 3 * GB, BASE + 4 * GB
    a.A, a.D, a.dt_bias = BASE + 5 * GB, BASE + 6 * GB, BASE + 7 * GB
    a.h0, a.h_last, a.y = BASE + 8 * GB, BASE + 9 * GB, BASE + 10 * GB
    a.workspace, a.workspace_bytes = BASE + 12 * GB, GB
    return a


def ssd_ws(lib, a):
    n = ctypes.c_size_t(0)
    assert lib.samba_ssd_workspace_size(ctypes.byref(a), ctypes.byref(n)) == 0
    return n.value


@pytest.mark.parametrize("batch,seqlen,G,varlen", [(2, 100, 2, False), (4, 4096, 1, False), (1, 1000, 4, True),
                                                   (3, 0, 1, False)])
def test_ssd_workspace_size(lib, batch, seqlen, G, varlen):
    """With the C Bᵀ pre-pass, 12 KiB per (chunk slot, group): batched sequences own ceil(L / 64) slots
    each, packed streams tokens / 64 + nseq slots; no tokens, no workspace.  Formed inside the prefill
    kernel (and by default), none."""
    a = ssd_ok(batch=batch, seqlen=seqlen, heads=4 * G, ngroups=G)
    if varlen:
        a.cu_seqlens, a.nseq = BASE + 11 * GB, 5
    slots = (batch * seqlen) // 64 + 5 if varlen else batch * -(-seqlen // 64)
    a.cb_mode = D.CB_PREPASS
    assert ssd_ws(lib, a) == (slots * G * 12288 if batch * seqlen else 0)
    for mode in (D.CB_IN_KERNEL, D.CB_AUTO):
        a.cb_mode = mode
        assert ssd_ws(lib, a) == 0


SSD_CASES = {
    "struct_size": (lambda a: setattr(a, "struct_size", 4), 7),
    "cb_mode": (lambda a: setattr(a, "cb_mode", 3), 6),
    "cb_mode_negative": (lambda a: setattr(a, "cb_mode", -1), 6),
    "head_dim_128": (lambda a: setattr(a, "head_dim", 128), 6),
    "dstate_16": (lambda a: setattr(a, "dstate", 16), 6),
    "dstate_256": (lambda a: setattr(a, "dstate", 256), 6),
    "groups_not_dividing": (lambda a: setattr(a, "ngroups", 3), 2),
    "zero_heads": (lambda a: setattr(a, "heads", 0), 2),
    "neg_seqlen": (lambda a: setattr(a, "seqlen", -1), 2),
    "y_dtype": (lambda a: setattr(a, "y_dtype", 7), 3),
    "null_x": (lambda a: setattr(a, "x", None), 1),
    "null_A": (lambda a: setattr(a, "A", None), 1),
    "misaligned_x": (lambda a: setattr(a, "x", a.x + 8), 4),
    "misaligned_z": (lambda a: setattr(a, "z", a.z + 4), 4),
    "misaligned_h0": (lambda a: setattr(a, "h0", a.h0 + 8), 4),
    "misaligned_y_f32": (lambda a: (setattr(a, "y_dtype", S.SAMBA_F32), setattr(a, "y", a.y + 8)), 4),
    "y_overlaps_x": (lambda a: setattr(a, "y", a.x + 128), 5),
    "y_overlaps_z": (lambda a: setattr(a, "y", a.z), 5),
    "h_last_overlaps_B": (lambda a: setattr(a, "h_last", a.B + 256), 5),
    "h_last_overlaps_h0_shifted": (lambda a: setattr(a, "h_last", a.h0 + 16), 5),
    "varlen_batch": (lambda a: (setattr(a, "cu_seqlens", BASE + 11 * GB), setattr(a, "nseq", 3)), 2),
    "offsets_past_31_bits": (lambda a: (setattr(a, "seqlen", 1 << 19), setattr(a, "heads", 64),
                                        setattr(a, "ngroups", 1)), 2),
    "too_many_heads": (lambda a: (setattr(a, "seqlen", 1), setattr(a, "batch", 1), setattr(a, "heads", 1 << 17),
                                  setattr(a, "ngroups", 1)), 2),
    "null_workspace": (lambda a: setattr(a, "workspace", None), 9),
    "small_workspace": (lambda a: setattr(a, "workspace_bytes", 4096), 9),
    "misaligned_workspace": (lambda a: setattr(a, "workspace", a.workspace + 128), 9),
    "workspace_overlaps_y": (lambda a: setattr(a, "workspace", a.y), 5),
    "workspace_overlaps_C": (lambda a: setattr(a, "workspace", a.C + 256), 5),
}


@pytest.mark.parametrize("name", sorted(SSD_CASES))
def test_ssd_rejects(lib, name):
    a = ssd_ok()
    if "workspace" in name:
        a.cb_mode = D.CB_PREPASS   # (the only form that takes a workspace)
    mutate, code = SSD_CASES[name]
    mutate(a)
    assert lib.samba_ssd_fwd(ctypes.byref(a), None) == code


def test_ssd_noops(lib):
    a = ssd_ok(batch=0)
    assert lib.samba_ssd_fwd(ctypes.byref(a), None) == 0
    assert lib.samba_ssd_fwd(None, None) == 1
    n = ctypes.c_size_t(7)
    assert lib.samba_ssd_workspace_size(None, ctypes.byref(n)) == 1
    assert lib.samba_ssd_workspace_size(ctypes.byref(a), None) == 1
    assert lib.samba_ssd_workspace_size(ctypes.byref(a), ctypes.byref(n)) == 0 and n.value == 0


# --------------------------------------------------------------------------- #
# gated linear attention: validation
# --------------------------------------------------------------------------- #
def gla_ok(batch=2, seqlen=100, heads=4, head_dim=64, dstate=128):
    a = GL.GlaArgs()
    a.struct_size = ctypes.sizeof(GL.GlaArgs)
    a.batch, a.seqlen, a.heads, a.head_dim, a.dstate = batch, seqlen, heads, head_dim, dstate
    a.in_dtype, a.y_dtype = S.SAMBA_BF16, S.SAMBA_F32
    a.q, a.k, a.gk, a.v = BASE, BASE + GB, BASE + 2 * GB, BASE + 3 * GB
    a.h0, a.h_last, a.o = BASE + 4 * GB, BASE + 5 * GB, BASE + 6 * GB
    a.workspace, a.workspace_bytes = BASE + 7 * GB, GB
    return a


def gla_ws_bytes(nslots, heads, dstate):
    # per (chunk slot, head): scaled q and k as bf16 hi + lo planes, A hi + lo, e^{b_64}
    return nslots * heads * (4 * 64 * dstate * 2 + 2 * 64 * 64 * 2 + 4 * dstate)


GLA_CASES = {
    "workspace_null": (lambda a: setattr(a, "workspace", None), 9),
    "workspace_small": (lambda a: setattr(a, "workspace_bytes", gla_ws_bytes(4, 4, 128) - 1), 9),
    "workspace_misaligned": (lambda a: setattr(a, "workspace", a.workspace + 128), 4),
    "workspace_overlaps_o": (lambda a: setattr(a, "workspace", a.o), 5),
    "struct_size": (lambda a: setattr(a, "struct_size", 4), 7),
    "dstate_48": (lambda a: setattr(a, "dstate", 48), 6),
    "dstate_512": (lambda a: setattr(a, "dstate", 512), 6),
    "head_dim_not_whole_waves": (lambda a: setattr(a, "head_dim", 3), 2),
    "zero_heads": (lambda a: setattr(a, "heads", 0), 2),
    "neg_seqlen": (lambda a: setattr(a, "seqlen", -1), 2),
    "in_dtype": (lambda a: setattr(a, "in_dtype", 5), 3),
    "null_gk": (lambda a: setattr(a, "gk", None), 1),
    "misaligned_q": (lambda a: setattr(a, "q", a.q + 8), 4),
    "misaligned_h0": (lambda a: setattr(a, "h0", a.h0 + 4), 4),
    "o_overlaps_v": (lambda a: setattr(a, "o", a.v + 64), 5),
    "h_last_overlaps_k": (lambda a: setattr(a, "h_last", a.k), 5),
    "h_last_overlaps_h0_shifted": (lambda a: setattr(a, "h_last", a.h0 + 16), 5),
    "varlen_batch": (lambda a: (setattr(a, "cu_seqlens", BASE + 11 * GB), setattr(a, "nseq", 3)), 2),
    "offsets_past_32_bits": (lambda a: (setattr(a, "seqlen", 1 << 22), setattr(a, "heads", 16)), 2),
}


@pytest.mark.parametrize("name", sorted(GLA_CASES))
def test_gla_rejects(lib, name):
    a = gla_ok()
    mutate, code = GLA_CASES[name]
    mutate(a)
    assert lib.samba_gla_fwd(ctypes.byref(a), None) == code


def test_gla_workspace_size(lib):
    n = ctypes.c_size_t(0)
    a = gla_ok()                       # bf16, 128 keys, 64 values: the chunked form, 2 x 2 chunks
    assert lib.samba_gla_workspace_size(ctypes.byref(a), ctypes.byref(n)) == 0 and n.value == gla_ws_bytes(4, 4, 128)
    a = gla_ok(dstate=256, seqlen=64)
    assert lib.samba_gla_workspace_size(ctypes.byref(a), ctypes.byref(n)) == 0 and n.value == gla_ws_bytes(2, 4, 256)
    a.cu_seqlens, a.nseq, a.batch, a.seqlen = BASE + 11 * GB, 3, 1, 1000   # packed: tokens / 64 + nseq slots
    assert lib.samba_gla_workspace_size(ctypes.byref(a), ctypes.byref(n)) == 0 and n.value == gla_ws_bytes(15 + 3, 4, 256)
    for mutate in (lambda a: setattr(a, "in_dtype", S.SAMBA_F32), lambda a: setattr(a, "dstate", 64),
                   lambda a: setattr(a, "head_dim", 48), lambda a: setattr(a, "batch", 0)):
        a = gla_ok()
        mutate(a)                      # the recurrent form (or no tokens): no workspace
        assert lib.samba_gla_workspace_size(ctypes.byref(a), ctypes.byref(n)) == 0 and n.value == 0
    a = gla_ok(dstate=48)
    assert lib.samba_gla_workspace_size(ctypes.byref(a), ctypes.byref(n)) == 6
    assert lib.samba_gla_workspace_size(ctypes.byref(gla_ok()), None) == 1


def test_gla_noops(lib):
    a = gla_ok(batch=0)
    assert lib.samba_gla_fwd(ctypes.byref(a), None) == 0
    assert lib.samba_gla_fwd(None, None) == 1
    a = gla_ok()
    a.h_last = a.h0                     # in place is allowed
    a.batch = 0
    assert lib.samba_gla_fwd(ctypes.byref(a), None) == 0
