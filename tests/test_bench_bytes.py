"""The roofline denominators of bench.py, pinned by hand-derived sizes.

Each expected value is written out from the workload's shapes (each input
and output tensor moved once, in its I/O dtype), term by term, so a wrong
term in bench.py's formulas shows up here.  The per-token figures match the
measurement table of the hot-path scope (37,120 B/token for the Nemotron-H
8B scan, 20,608 B/token for Nemotron 3 Nano).
"""
import numpy as np

import bench
from state_space_sequence_ssd_amd import inputs

KIB = 1024


def test_scan_bytes_nemotron_h_8b():
    w = inputs.nemotron_h_8b()
    assert (w.batch, w.seqlen, w.nheads, w.ngroups) == (4, 4096, 128, 8)
    per_token = (128 * 64 * 2      # x, bf16: 16 KiB
                 + 128 * 64 * 2    # y, bf16: 16 KiB
                 + 2 * 8 * 128 * 2  # B and C, bf16: 4 KiB
                 + 128 * 2)        # dt, bf16
    assert per_token == 37_120 == 36 * KIB + 256
    final_states = 4 * 128 * 64 * 128 * 4   # fp32, one per batch row and head
    params = 3 * 128 * 4                     # A, D, dt_bias (fp32 per head)
    expected = 4 * 4096 * per_token + final_states + params
    assert expected == 624_952_832
    assert bench.scan_algorithmic_bytes(w) == expected


def test_scan_bytes_nemotron3_nano():
    w = inputs.nemotron3_nano()
    assert (w.batch, w.seqlen, w.nheads, w.ngroups) == (1, 16384, 64, 8)
    per_token = 64 * 64 * 2 * 2 + 2 * 8 * 128 * 2 + 64 * 2
    assert per_token == 20_608
    expected = 16384 * per_token + 64 * 64 * 128 * 4 + 3 * 64 * 4
    assert bench.scan_algorithmic_bytes(w) == expected == 339_739_392


def test_scan_bytes_packed_counts_seq_idx_and_both_states():
    w = inputs.packed_3b()
    T = int(w.packed_lengths.sum())
    assert w.batch == 1 and w.seqlen == T and w.num_seqs == 32 and w.init_std > 0
    per_token = 40 * 64 * 2 * 2 + 2 * 8 * 128 * 2 + 40 * 2 + 4   # + seq_idx (int32)
    states = 2 * 32 * 40 * 64 * 128 * 4                            # initial and final
    assert bench.scan_algorithmic_bytes(w) == T * per_token + states + 3 * 40 * 4


def test_conv_bytes_nemotron_h_8b():
    w = inputs.nemotron_h_8b()
    conv_dim = 128 * 64 + 2 * 8 * 128
    assert w.conv_dim == conv_dim == 10240
    expected = 2 * 4 * 4096 * conv_dim * 2 + conv_dim * 4 * 4   # in + out (bf16), fp32 taps
    assert bench.conv_algorithmic_bytes(w) == expected == 671_252_480


def test_decode_bytes_per_layer():
    dw = inputs.decode_29_layers()
    b, H, P, N, CD = 256, 128, 64, 128, 10240
    assert (dw.batch, dw.nheads, dw.headdim, dw.dstate, dw.conv_dim) == (b, H, P, N, CD)
    expected = (2 * b * H * P * N * 4     # fp32 state, read and written once: 2 GiB
                + b * CD * 2              # the raw x|B|C token
                + 2 * b * 3 * CD * 2      # conv state, read and written
                + b * H * P * 2           # y
                + b * H * 2               # dt
                + CD * 4 * 4              # conv taps
                + 3 * H * 4)              # A, D, dt_bias
    assert bench.decode_algorithmic_bytes(dw) == expected == 2_188_609_024


def test_scan_flops_nemotron_h_8b():
    # causal pairs Q(Q+1)/2 per chunk for C B^T (once per group) and for M x
    # (per head), both as multiply-adds, plus the state update and the
    # state->output product (2 H P N each per token)
    w = inputs.nemotron_h_8b()
    T, Q, G, H, P, N = 16384, 128, 8, 128, 64, 128
    per_chunk = 2 * (Q * (Q + 1) // 2) * (G * N + H * P) + Q * 2 * (2 * H * P * N)
    assert bench.scan_flops(w) == T // Q * per_chunk
    assert abs(bench.scan_flops(w) / 1e9 - 88.2) < 0.05


def test_bench_refuses_more_than_one_gpu():
    """Everything here runs on one GPU: --gpus N > 1 stops before touching a device."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr + r.stdout


def test_oracle_beside_restores_threads_and_reports_parity():
    """The oracle is timed on all OpenMP threads and on one (cores = 1), the
    thread count is left as it was found, and the parity error is taken
    against the all-thread outputs of the sample (here an all-zero stand-in
    for the GPU outputs, so the error is exactly 1)."""
    import ctypes
    from types import SimpleNamespace
    import torch
    for w, a, o in [
        (inputs.ScanWorkload("tiny_conv", 2, 256, 8, 2, bf16=True, conv=True, final_state=True),
         {}, {"rows": 1}),
        (inputs.ScanWorkload("tiny_packed", 1, 300, 4, 2, bf16=False, conv=False, final_state=True,
                             packed_lengths=np.array([100, 0, 150, 50]), init_std=0.3),
         {}, {"seqs": 2}),
    ]:
        d = inputs.make_scan_inputs(w, seed=3)
        run = SimpleNamespace(w=w, d=d, y=torch.zeros(w.batch, w.seqlen, w.nheads, 64),
                              fs=torch.zeros(w.num_seqs, w.nheads, 64, 128))
        gomp = ctypes.CDLL("libgomp.so.1")
        before = gomp.omp_get_max_threads()
        allc, one = bench.oracle_beside(run, a, o)
        assert gomp.omp_get_max_threads() == before
        assert allc["cores"] == before and one["cores"] == 1
        assert allc["kind"] == one["kind"] == "oracle" and allc["value"] > 0 and one["value"] > 0
        assert allc["parity"]["y_rel_err"] == 1.0 and allc["parity"]["final_state_rel_err"] == 1.0
        assert allc["parity"]["bar"] == (2e-2 if w.bf16 else 1e-4)
