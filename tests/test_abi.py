"""C ABI of libssd.so on the host: exports and argument checks (no GPU needed).

Every check in the library runs before any HIP call, so each error path is
exercised here with fake (never dereferenced) device addresses.
"""
import ctypes
import os
import re

import pytest

from state_space_sequence_ssd_amd import ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000  # 16- and 256-byte aligned fake device address, never dereferenced


def header_functions():
    src = open(os.path.join(ROOT, "include", "ssd.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w[\w\s\*]*?\b(ssd_\w+)\s*\(", src, re.M)))


def test_exports_every_declared_symbol():
    lib = ssd.load_library()
    declared = header_functions()
    assert set(declared) == set(ssd.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.ssd_version() == 1


def test_struct_layouts_match_header(tmp_path):
    """Every ctypes mirror field sits at the offset the C compiler gives it."""
    import subprocess
    structs = {"ssd_conv_args": ssd.SsdConvArgs, "ssd_scan_args": ssd.SsdScanArgs,
               "ssd_decode_args": ssd.SsdDecodeArgs}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "ssd.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'printf("{cname} sizeof %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = {}
    for line in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines():
        c, f, v = line.split()
        got[(c, f)] = int(v)
    for cname, py in structs.items():
        assert got[(cname, "sizeof")] == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)


def scan_args(**kw):
    a = ssd.SsdScanArgs()
    a.struct_size = ctypes.sizeof(ssd.SsdScanArgs)
    a.dtype = ssd.SSD_DTYPE_BF16
    a.batch, a.seqlen, a.nheads, a.headdim, a.dstate, a.ngroups, a.chunk_size = 4, 4096, 128, 64, 128, 8, 128
    cd = 128 * 64 + 2 * 8 * 128
    for t in ("x", "B", "C", "y"):
        setattr(a, t, FAKE)
        setattr(a, t + "_stride_batch", 4096 * cd)
        setattr(a, t + "_stride_token", cd)
    a.dt, a.dt_stride_batch, a.dt_stride_token = FAKE, 4096 * 128, 128
    a.A = FAKE
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def scan_rc(a, ws=None, ws_bytes=1 << 40):
    lib = ssd.load_library()
    return lib.ssd_chunk_scan_fwd(ctypes.byref(a), ws, ws_bytes, None)


@pytest.mark.parametrize("field,value,code", [
    ("struct_size", 8, 1), ("dtype", 7, 2), ("batch", 0, 1), ("nheads", 0, 1), ("ngroups", 3, 1),
    ("headdim", 32, 2), ("dstate", 64, 2), ("chunk_size", 32, 2), ("chunk_size", 100, 2), ("seg_chunks", -1, 1),
    ("A", None, 1), ("x", None, 1), ("y", None, 1), ("dt", None, 1),
    ("x", FAKE + 2, 4), ("B_stride_token", 2048 + 2, 4), ("x_stride_token", 1024, 1),
    ("C_stride_token", 1 << 22, 1), ("dt_stride_token", 1 << 22, 1),
])
def test_scan_argument_errors(field, value, code):
    a = scan_args(**{field: value})
    assert scan_rc(a) == code
    assert ssd.load_library().ssd_last_error().decode()


@pytest.mark.parametrize("q", [64, 128, 256])
def test_scan_accepts_model_chunk_sizes(q):
    """The model's chunk length is 64, 128 or 256; the result does not depend on it."""
    lib = ssd.load_library()
    assert lib.ssd_chunk_scan_workspace_size(ctypes.byref(scan_args(chunk_size=q))) == 0


def test_scan_seq_idx_rules():
    assert scan_rc(scan_args(seq_idx=FAKE, num_seqs=3)) == 1          # batch != 1
    assert scan_rc(scan_args(batch=1, seq_idx=FAKE, num_seqs=0)) == 1  # num_seqs < 1


def test_scan_state_alignment():
    assert scan_rc(scan_args(initial_state=FAKE + 4)) == 4
    assert scan_rc(scan_args(final_state=FAKE + 8)) == 4


def test_workspace_sizes_and_too_small():
    lib = ssd.load_library()
    # Nemotron-H 8B shape: 4 x 128 (row, head) pairs fill the chip -> no segments, no workspace
    assert lib.ssd_chunk_scan_workspace_size(ctypes.byref(scan_args())) == 0
    # one long row with 64 heads -> segmented: per-segment states need workspace
    a = scan_args(batch=1, seqlen=16384, nheads=64)
    need = lib.ssd_chunk_scan_workspace_size(ctypes.byref(a))
    assert need > 0 and need % 256 == 0
    assert scan_rc(a, ws=FAKE, ws_bytes=need - 1) == 3
    assert scan_rc(a, ws=None, ws_bytes=need) == 3
    assert scan_rc(a, ws=FAKE + 16, ws_bytes=need) == 4
    # packed sequences always need the work-list table
    p = scan_args(batch=1, seqlen=1000, nheads=40, seq_idx=FAKE, num_seqs=32)
    assert lib.ssd_chunk_scan_workspace_size(ctypes.byref(p)) > 0
    bad = scan_args(headdim=16)
    assert lib.ssd_chunk_scan_workspace_size(ctypes.byref(bad)) == ctypes.c_size_t(-1).value


def conv_args(**kw):
    a = ssd.SsdConvArgs()
    a.struct_size = ctypes.sizeof(ssd.SsdConvArgs)
    a.dtype = ssd.SSD_DTYPE_BF16
    a.batch, a.seqlen, a.channels, a.width = 2, 100, 64, 4
    a.x, a.x_stride_batch, a.x_stride_token = FAKE, 6400, 64
    a.out, a.out_stride_batch, a.out_stride_token = FAKE, 6400, 64
    a.weight = FAKE
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,code", [
    ("struct_size", 4, 1), ("dtype", 3, 2), ("width", 3, 2), ("channels", 12, 2), ("weight", None, 1),
    ("x", None, 1), ("out", FAKE + 4, 4), ("x_stride_token", 60, 4), ("seq_idx", FAKE, 1),
    ("conv_state_in", FAKE + 2, 4),
])
def test_conv_argument_errors(field, value, code):
    lib = ssd.load_library()
    assert lib.ssd_conv1d_silu(ctypes.byref(conv_args(**{field: value})), None) == code


def decode_args(**kw):
    a = ssd.SsdDecodeArgs()
    a.struct_size = ctypes.sizeof(ssd.SsdDecodeArgs)
    a.dtype = ssd.SSD_DTYPE_BF16
    a.batch, a.nheads, a.headdim, a.dstate, a.ngroups, a.conv_width = 4, 16, 64, 128, 4, 4
    a.xBC, a.xBC_stride_batch = FAKE, 16 * 64 + 2 * 4 * 128
    a.dt, a.dt_stride_batch = FAKE, 16
    a.A, a.ssm_state, a.y, a.y_stride_batch = FAKE, FAKE, FAKE, 16 * 64
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,code", [
    ("struct_size", 0, 1), ("dtype", 9, 2), ("ngroups", 3, 1), ("headdim", 128, 2),
    ("ssm_state", None, 1), ("ssm_state", FAKE + 4, 4), ("conv_state", FAKE, 1),
    ("xBC_stride_batch", 10, 1), ("y", None, 1),
])
def test_decode_argument_errors(field, value, code):
    lib = ssd.load_library()
    assert lib.ssd_decode_step(ctypes.byref(decode_args(**{field: value})), None) == code


def test_library_has_no_cpu_fallback_symbols():
    """The product library exports only the ABI (no oracle or host compute entry)."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", ssd.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert {e for e in exported if e.startswith("ssd_")} == set(ssd.EXPORTS)
    assert not any("oracle" in e for e in exported)


def test_automatic_segments_follow_the_kernel_tile():
    """Automatic segmentation cuts fp32 inputs at the fp32 kernel's 64-token
    sub-chunks and bf16 inputs at 128-token tiles; an explicit seg_chunks
    counts 128-token tiles for both.  The workspace holds a local and an
    entry state (64 x 128 fp32) per (segment, head) plus the decays, each
    block 256-byte aligned."""
    lib = ssd.load_library()
    state = 64 * 128 * 4

    def need(**kw):
        return lib.ssd_chunk_scan_workspace_size(
            ctypes.byref(scan_args(batch=1, seqlen=512, nheads=8, ngroups=1, **kw)))

    def expected(nseg):
        return 2 * nseg * 8 * state + (-(-nseg * 8 * 4 // 256)) * 256
    assert need(dtype=ssd.SSD_DTYPE_F32) == expected(8)   # 64-token segments
    assert need() == expected(4)                          # bf16: 128-token segments
    assert need(dtype=ssd.SSD_DTYPE_F32, seg_chunks=2) == expected(2)
