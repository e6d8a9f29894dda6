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
               "ssd_decode_args": ssd.SsdDecodeArgs, "ssd_norm_args": ssd.SsdNormArgs,
               "ssd_mimo_decode_args": ssd.SsdMimoDecodeArgs, "ssd_scan_bwd_args": ssd.SsdScanBwdArgs,
               "ssd_conv_scan_args": ssd.SsdConvScanArgs, "ssd_linear_args": ssd.SsdLinearArgs}
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


def conv_scan_args(**kw):
    a = ssd.SsdConvScanArgs()
    a.struct_size = ctypes.sizeof(ssd.SsdConvScanArgs)
    a.dtype = ssd.SSD_DTYPE_BF16
    a.batch, a.seqlen, a.nheads, a.headdim, a.dstate, a.ngroups, a.chunk_size = 4, 4096, 128, 64, 128, 8, 128
    a.conv_width = 4
    cd = 128 * 64 + 2 * 8 * 128
    a.xBC, a.xBC_stride_batch, a.xBC_stride_token = FAKE, 4096 * cd, cd
    a.y, a.y_stride_batch, a.y_stride_token = FAKE, 4096 * 8192, 8192
    a.conv_weight = FAKE
    a.dt, a.dt_stride_batch, a.dt_stride_token = FAKE, 4096 * 128, 128
    a.A = FAKE
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def conv_scan_rc(a, ws=None, ws_bytes=1 << 40):
    return ssd.load_library().ssd_conv_scan_fwd(ctypes.byref(a), ws, ws_bytes, None)


@pytest.mark.parametrize("field,value,code", [
    ("struct_size", 8, 1), ("dtype", 7, 2), ("conv_width", 3, 2), ("conv_weight", None, 1), ("xBC", None, 1),
    ("xBC", FAKE + 2, 4), ("xBC_stride_token", 8192, 1), ("xBC_stride_token", 10240 + 2, 4),
    ("conv_weight", FAKE + 4, 4), ("conv_state_in", FAKE + 8, 4), ("conv_state_out", FAKE + 8, 4),
    ("batch", 0, 1), ("ngroups", 3, 1), ("headdim", 32, 2), ("A", None, 1), ("y", None, 1), ("dt", None, 1),
    ("y_stride_token", 1024, 1), ("final_state", FAKE + 8, 4),
])
def test_conv_scan_argument_errors(field, value, code):
    a = conv_scan_args(**{field: value})
    assert conv_scan_rc(a) == code
    assert ssd.load_library().ssd_last_error().decode()


def test_conv_scan_workspace():
    """The workspace holds the B|C conv output (bf16; every channel for fp32) and the scan's own."""
    lib = ssd.load_library()
    need = lib.ssd_conv_scan_workspace_size(ctypes.byref(conv_scan_args()))
    assert need == 4 * 4096 * 2 * 8 * 128 * 2  # no scan workspace at this shape
    need32 = lib.ssd_conv_scan_workspace_size(ctypes.byref(conv_scan_args(dtype=ssd.SSD_DTYPE_F32,
                                                                             xBC_stride_batch=4096 * 10240)))
    assert need32 == 4 * 4096 * 10240 * 4
    a = conv_scan_args()
    assert conv_scan_rc(a, ws=FAKE, ws_bytes=need - 1) == 3
    assert conv_scan_rc(a, ws=None, ws_bytes=need) == 3
    assert conv_scan_rc(a, ws=FAKE + 16, ws_bytes=need) == 4
    # segmented: the scan's per-segment states come after the conv output
    seg = conv_scan_args(batch=1, seqlen=16384, nheads=64, xBC_stride_batch=16384 * (64 * 64 + 2048),
                         xBC_stride_token=64 * 64 + 2048, y_stride_token=64 * 64,
                         dt_stride_batch=16384 * 64, dt_stride_token=64)
    conv_part = 16384 * 2048 * 2
    assert lib.ssd_conv_scan_workspace_size(ctypes.byref(seg)) > conv_part
    assert lib.ssd_conv_scan_workspace_size(ctypes.byref(conv_scan_args(headdim=16))) == ctypes.c_size_t(-1).value


def linear_args(**kw):
    a = ssd.SsdLinearArgs()
    a.struct_size = ctypes.sizeof(ssd.SsdLinearArgs)
    a.dtype = ssd.SSD_DTYPE_BF16
    a.M, a.N, a.K = 16384, 18560, 4096
    a.x, a.x_stride = FAKE, 4096
    a.w, a.w_stride = FAKE, 4096
    a.y, a.y_stride = FAKE, 18560
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,code", [
    ("struct_size", 4, 1), ("dtype", ssd.SSD_DTYPE_F32, 2), ("M", -1, 1), ("K", 100, 2), ("K", 0, 2),
    ("N", 12, 2), ("x", None, 1), ("w", None, 1), ("y", None, 1), ("x_stride", 4000, 1),
    ("y_stride", 1 << 22, 1), ("x", FAKE + 8, 4), ("w_stride", 4096 + 4, 4),
])
def test_linear_argument_errors(field, value, code):
    assert ssd.load_library().ssd_linear(ctypes.byref(linear_args(**{field: value})), None) == code
    assert ssd.load_library().ssd_last_error().decode()


def test_linear_empty_is_a_no_op():
    """M = 0 or N = 0: nothing to compute, success before any HIP call."""
    lib = ssd.load_library()
    assert lib.ssd_linear(ctypes.byref(linear_args(M=0, x=None, y=None)), None) == 0
    assert lib.ssd_linear(ctypes.byref(linear_args(N=0, w=None, y=None)), None) == 0


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
    block 256-byte aligned.  fp32 batch rows of at most 1024 tokens run as
    one quadratic form and need no workspace at all."""
    lib = ssd.load_library()
    state = 64 * 128 * 4

    def need(seqlen, **kw):
        return lib.ssd_chunk_scan_workspace_size(
            ctypes.byref(scan_args(batch=1, seqlen=seqlen, nheads=8, ngroups=1, **kw)))

    def expected(nseg):
        return 2 * nseg * 8 * state + (-(-nseg * 8 * 4 // 256)) * 256
    assert need(2048, dtype=ssd.SSD_DTYPE_F32) == expected(32)   # 64-token segments
    assert need(512) == expected(4)                              # bf16: 128-token segments
    assert need(2048, dtype=ssd.SSD_DTYPE_F32, seg_chunks=2) == expected(8)
    for L in (1, 512, 1024):
        assert need(L, dtype=ssd.SSD_DTYPE_F32) == 0 and need(L, dtype=ssd.SSD_DTYPE_F32, seg_chunks=1) == 0
    assert need(1025, dtype=ssd.SSD_DTYPE_F32) > 0


def test_decode_heads_per_group_limit():
    """One decode workgroup holds a group's conv outputs and y in LDS: up to
    250 heads per group are accepted, 251 are UNSUPPORTED.  The accepted case
    is stopped by a later check (a batch stride below the row width), so no
    kernel is launched."""
    lib = ssd.load_library()
    for hpg, code in ((250, 1), (251, 2), (16, 1)):
        a = decode_args(nheads=hpg, ngroups=1, xBC_stride_batch=8)
        assert lib.ssd_decode_step(ctypes.byref(a), None) == code, hpg


def test_noalloc_scratch_size_constant_matches_header():
    src = open(os.path.join(ROOT, "include", "ssd.h")).read()
    m = re.search(r"#define SSD_NOALLOC_SCRATCH_BYTES \((\d+)u \* 1024u \* 1024u\)", src)
    assert m and int(m.group(1)) * 1024 * 1024 == ssd.NOALLOC_SCRATCH_BYTES


def test_noalloc_fits_every_automatic_segmentation():
    """With seg_chunks = 0 the workspace of any shape fits the no-allocation
    entry point's array: batch rows and packed streams (one to four
    sequences, where segmentation is deepest), both dtypes, 1 to 600 heads."""
    lib = ssd.load_library()
    worst = 0
    for dtype in (ssd.SSD_DTYPE_BF16, ssd.SSD_DTYPE_F32):
        for H in list(range(1, 64)) + list(range(64, 601, 7)) + [255, 256, 257, 500, 510, 511, 512, 513]:
            for rows in (1, 2, 3, 4):
                for L in (100_000, 1 << 20):
                    for packed in (False, True):
                        a = scan_args(dtype=dtype, nheads=H, ngroups=1, seqlen=L,
                                      batch=1 if packed else rows)
                        for t in ("x", "y"):
                            setattr(a, t + "_stride_token", ((H * 64 + 7) // 8) * 8)
                        a.dt_stride_token = H
                        if packed:
                            a.seq_idx, a.num_seqs = FAKE, rows
                        n = lib.ssd_chunk_scan_workspace_size(ctypes.byref(a))
                        assert n != ctypes.c_size_t(-1).value, lib.ssd_last_error()
                        worst = max(worst, n)
    assert worst <= ssd.NOALLOC_SCRATCH_BYTES, worst
    assert worst > 0.9 * ssd.NOALLOC_SCRATCH_BYTES   # the bound is tight, not padded


def test_noalloc_rejects_a_workspace_beyond_its_array():
    """An explicit one-tile segmentation of the Nemotron-H 8B shape needs
    1 GiB of segment states: refused before any HIP call."""
    lib = ssd.load_library()
    a = scan_args(seg_chunks=1)
    need = lib.ssd_chunk_scan_workspace_size(ctypes.byref(a))
    assert need > ssd.NOALLOC_SCRATCH_BYTES
    assert lib.ssd_chunk_scan_fwd_noalloc(ctypes.byref(a), None) == 3
    msg = lib.ssd_last_error().decode()
    assert "noalloc" in msg and str(need) in msg
    # argument errors come first, as in ssd_chunk_scan_fwd
    assert lib.ssd_chunk_scan_fwd_noalloc(ctypes.byref(scan_args(ngroups=3)), None) == 1


def norm_args(**kw):
    a = ssd.SsdNormArgs()
    a.struct_size = ctypes.sizeof(ssd.SsdNormArgs)
    a.dtype = ssd.SSD_DTYPE_BF16
    a.batch, a.seqlen, a.channels, a.group_size, a.eps = 4, 4096, 8192, 1024, 1e-5
    a.y, a.y_stride_batch, a.y_stride_token = FAKE, 4096 * 8192, 8192
    a.z, a.z_stride_batch, a.z_stride_token = FAKE, 4096 * 18560, 18560
    a.weight = FAKE
    a.out, a.out_stride_batch, a.out_stride_token = FAKE, 4096 * 8192, 8192
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,code", [
    ("struct_size", 4, 1), ("dtype", 5, 2), ("channels", 1000, 1), ("group_size", 1020, 2),
    ("group_size", 8200 * 2, 2), ("eps", -1.0, 1), ("eps", float("inf"), 1), ("eps", float("nan"), 1),
    ("weight", None, 1), ("y", None, 1), ("out", FAKE + 8, 4), ("z_stride_token", 18561, 4),
    ("y_stride_token", 4096, 1), ("batch", 0, 1),
])
def test_norm_argument_errors(field, value, code):
    lib = ssd.load_library()
    kw = {field: value}
    if field == "group_size":
        kw["channels"] = value * 8
    assert lib.ssd_gated_rmsnorm(ctypes.byref(norm_args(**kw)), None) == code
    assert lib.ssd_last_error().decode()


def test_norm_fp32_group_limit():
    lib = ssd.load_library()
    a = norm_args(dtype=ssd.SSD_DTYPE_F32, group_size=8192, channels=8192)
    assert lib.ssd_gated_rmsnorm(ctypes.byref(a), None) == 2


def mimo_args(**kw):
    a = ssd.SsdMimoDecodeArgs()
    a.struct_size = ctypes.sizeof(ssd.SsdMimoDecodeArgs)
    a.dtype = ssd.SSD_DTYPE_BF16
    a.batch, a.nheads, a.headdim, a.dstate, a.ngroups, a.rank = 4, 16, 64, 128, 4, 4
    a.x, a.x_stride_batch = FAKE, 16 * 64 * 4
    a.B, a.B_stride_batch, a.C, a.C_stride_batch = FAKE, 4 * 128 * 4, FAKE, 4 * 128 * 4
    a.dt, a.dt_stride_batch = FAKE, 16
    a.A, a.ssm_state, a.y, a.y_stride_batch = FAKE, FAKE, FAKE, 16 * 64 * 4
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,code", [
    ("struct_size", 0, 1), ("dtype", 9, 2), ("ngroups", 3, 1), ("headdim", 32, 2), ("rank", 3, 2),
    ("rank", 16, 2), ("x", None, 1), ("ssm_state", FAKE + 4, 4), ("trapezoid", 1, 1),
    ("x_stride_batch", 100, 1), ("B_stride_batch", 500, 1),
])
def test_mimo_argument_errors(field, value, code):
    lib = ssd.load_library()
    assert lib.ssd_decode_step_mimo(ctypes.byref(mimo_args(**{field: value})), None) == code
    assert lib.ssd_last_error().decode()


def test_mimo_lds_limit():
    """A group's X, previous X and Y must fit one workgroup's LDS: 16 heads per
    group at rank 8 with the trapezoidal term fit, 64 do not.  The accepted
    case is stopped by a later check, so no kernel is launched."""
    lib = ssd.load_library()
    ok = mimo_args(rank=8, trapezoid=1, prev_x=FAKE, prev_B=FAKE, x_stride_batch=8)
    assert lib.ssd_decode_step_mimo(ctypes.byref(ok), None) == 1
    big = mimo_args(nheads=64, ngroups=1, rank=8, trapezoid=1, prev_x=FAKE, prev_B=FAKE)
    assert lib.ssd_decode_step_mimo(ctypes.byref(big), None) == 2


def bwd_args(**kw):
    a = ssd.SsdScanBwdArgs()
    a.struct_size = ctypes.sizeof(ssd.SsdScanBwdArgs)
    a.dtype = ssd.SSD_DTYPE_BF16
    a.batch, a.seqlen, a.nheads, a.headdim, a.dstate, a.ngroups = 4, 4096, 128, 64, 128, 8
    for f in ("x", "dt", "B", "C", "dy", "dx", "ddt", "dB", "dC", "A", "dA"):
        setattr(a, f, FAKE)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,code", [
    ("struct_size", 4, 1), ("dtype", 4, 2), ("ngroups", 3, 1), ("dstate", 64, 2), ("dA", None, 1),
    ("dy", None, 1), ("dB", FAKE + 8, 4), ("initial_state", FAKE + 4, 4),
])
def test_bwd_argument_errors(field, value, code):
    lib = ssd.load_library()
    assert lib.ssd_chunk_scan_bwd(ctypes.byref(bwd_args(**{field: value})), FAKE, 1 << 40, None) == code


def test_bwd_workspace_layout():
    """The backward workspace: the state entering every 32-token chunk of every
    (row, head), per-head dB and dC partials, per-(row, head) scalars, each
    block 256-byte aligned; a smaller workspace is refused."""
    lib = ssd.load_library()
    a = bwd_args(batch=2, seqlen=100, nheads=8, ngroups=2)
    n = lib.ssd_chunk_scan_bwd_workspace_size(ctypes.byref(a))
    up = lambda v: -(-v // 256) * 256
    expect = up(2 * 8 * 4 * 64 * 128 * 4) + 2 * up(2 * 100 * 8 * 128 * 4) + up(2 * 8 * 3 * 4)
    assert n == expect
    assert lib.ssd_chunk_scan_bwd(ctypes.byref(a), FAKE, n - 1, None) == 3
    assert lib.ssd_chunk_scan_bwd(ctypes.byref(a), FAKE + 16, n, None) == 4
