"""CPU self-checks of the GPU tests' oracle helper (restricting heads/rows is exact)."""
import numpy as np

from state_space_sequence_ssd_amd import inputs
from tests.gpu_helpers import oracle_layer


def test_restricted_oracle_matches_full():
    for w in (inputs.ScanWorkload("t", 2, 70, 8, 4, bf16=True, conv=True, final_state=True, init_std=0.3),
              inputs.ScanWorkload("p", 1, 0, 6, 3, bf16=True, conv=True, final_state=True,
                                  packed_lengths=np.array([5, 30, 9]), init_std=0.3),
              inputs.ScanWorkload("n", 2, 40, 6, 2, bf16=False, conv=False, final_state=True)):
        w.seqlen = w.seqlen if w.packed_lengths is None else int(w.packed_lengths.sum())
        d = inputs.make_scan_inputs(w, seed=2)
        ry, rf = oracle_layer(d, w)
        heads = [1, w.nheads - 1]
        rows = None if w.packed_lengths is not None else [1]
        sy, sf = oracle_layer(d, w, heads=heads, rows=rows)
        rsel = slice(None) if rows is None else rows
        assert np.array_equal(sy, ry[rsel][:, :, heads])
        assert np.array_equal(sf, rf[rsel][:, heads])
