"""ssd_chunk_scan_fwd_noalloc (library-owned workspace) against
ssd_chunk_scan_fwd (caller workspace), through the C ABI.

Both run the same plan and kernels, so the outputs must agree bit for bit;
they are also held to the oracle's bar.  Two calls in a row on the shared
array, the second smaller than the first, then the first again: what the
array keeps from one call never leaks into the next.
"""
import numpy as np
import pytest
import torch

from state_space_sequence_ssd_amd import inputs, ssd
from tests.gpu_helpers import BF, DEV, oracle_layer, rel, split_xbc, to_dev, to_np

pytestmark = pytest.mark.gpu


def _tensors(d, w):
    H, G = w.nheads, w.ngroups
    dtp = BF if w.bf16 else torch.float32
    seq = to_dev(d["seq_idx"]) if "seq_idx" in d else None
    nseq = w.num_seqs if seq is not None else None
    if w.conv:
        v = ssd.ssd_conv1d_silu(to_dev(d["xBC"], dtp), to_dev(d["conv_w"]), seq_idx=seq, num_seqs=nseq)
        x, B, C = split_xbc(v, H, G)
    else:
        x, B, C = to_dev(d["x"], dtp), to_dev(d["B"], dtp), to_dev(d["C"], dtp)
    kw = dict(dt_bias=to_dev(d["dt_bias"]), D=to_dev(d["D"]), seq_idx=seq, num_seqs=nseq,
              initial_state=to_dev(d["initial_state"]) if "initial_state" in d else None)
    return x, to_dev(d["dt"], dtp), to_dev(d["A"]), B, C, kw


def _both(w, seed):
    print(f"case {w.name} seed={seed}", flush=True)
    d = inputs.make_scan_inputs(w, seed=seed)
    x, dt, A, B, C, kw = _tensors(d, w)
    rows = w.num_seqs
    need = ssd.ssd_chunk_scan_workspace_size(x, dt, A, B, C, seq_idx=kw["seq_idx"], num_seqs=kw["num_seqs"])
    assert 0 < need <= ssd.NOALLOC_SCRATCH_BYTES, need
    fs_ref = torch.full((rows, w.nheads, 64, 128), float("nan"), device=DEV)
    y_ref = ssd.ssd_chunk_scan_fwd(x, dt, A, B, C, final_state=fs_ref, **kw)
    y = torch.full_like(y_ref, float("nan"))
    fs = torch.full_like(fs_ref, float("nan"))
    ssd.ssd_chunk_scan_fwd_noalloc(x, dt, A, B, C, y, final_state=fs, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref) and torch.equal(fs, fs_ref), "no-alloc result differs from the workspace call"
    return d, y, fs, need


def _check_oracle(d, w, y, fs):
    ry, rf = oracle_layer(d, w)
    ey, ef = rel(to_np(y), ry), rel(to_np(fs), rf)
    print(f"  y rel err {ey:.3e}  final-state rel err {ef:.3e}", flush=True)
    bar = 2e-2 if w.bf16 else 1e-4
    assert ey <= bar and ef <= bar


def test_noalloc_two_calls_in_a_row():
    big = inputs.nemotron3_nano()                      # 8 segments x 64 heads: 32 MiB of states
    small = inputs.ScanWorkload("packed_seg_h8_g2_init", 1, 0, 8, 2, bf16=True, conv=False,
                                final_state=True, packed_lengths=np.array([300, 5, 0, 700, 1]),
                                init_std=0.3)
    small.seqlen = int(small.packed_lengths.sum())
    d1, y1, f1, n1 = _both(big, seed=2)
    _check_oracle(d1, big, y1, f1)
    d2, y2, f2, n2 = _both(small, seed=7)
    assert n2 < n1
    _check_oracle(d2, small, y2, f2)
    _, y3, f3, _ = _both(big, seed=2)
    assert torch.equal(y3, y1) and torch.equal(f3, f1)


def test_noalloc_fp32_and_no_workspace_needed():
    """The fp32 kernel's segmented path, and a call that needs no workspace
    (enough (row, head) pairs): the library array is not even looked up."""
    w = inputs.ScanWorkload("fp32_seg_b1_l1500_h4_g1_init", 1, 1500, 4, 1, bf16=False, conv=False,
                            final_state=True, init_std=0.3)
    d, y, fs, _ = _both(w, seed=5)
    _check_oracle(d, w, y, fs)
    w2 = inputs.ScanWorkload("bf16_b4_l256_h128_g8", 4, 256, 128, 8, bf16=True, conv=False, final_state=True)
    d2 = inputs.make_scan_inputs(w2, seed=6)
    x, dt, A, B, C, kw = _tensors(d2, w2)
    assert ssd.ssd_chunk_scan_workspace_size(x, dt, A, B, C) == 0
    y_ref = ssd.ssd_chunk_scan_fwd(x, dt, A, B, C, **kw)
    y = torch.empty_like(y_ref)
    ssd.ssd_chunk_scan_fwd_noalloc(x, dt, A, B, C, y, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
