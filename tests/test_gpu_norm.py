"""Gated RMSNorm on the GPU vs the fp64 oracle, through the C ABI.

Bars: max|gpu - oracle| / max|oracle| <= 2e-2 for bf16 (the output is
rounded to bf16: about 2^-9 of each element), <= 1e-4 for fp32.
"""
import numpy as np
import pytest
import torch

import oracle
from state_space_sequence_ssd_amd import inputs, ssd
from tests.gpu_helpers import BF, DEV, rel, to_dev, to_np

pytestmark = pytest.mark.gpu

TOL = {True: 2e-2, False: 1e-4}

CASES = [
    # (batch, L, channels, group_size, bf16, gate, before)
    (2, 37, 8192, 1024, True, True, False),     # Nemotron-H 8B width, 8 groups
    (2, 37, 8192, 1024, True, True, True),
    (1, 20, 8192, 8192, True, True, False),     # one group over the whole width
    (3, 5, 4096, 64, True, False, False),       # head-sized groups, no gate
    (1, 9, 120, 40, True, True, False),         # groups not a multiple of one wave pass
    (2, 11, 8192, 1024, False, True, False),
    (2, 11, 4096, 4096, False, True, True),
    (1, 7, 96, 12, False, False, False),
]


@pytest.mark.parametrize("batch,L,CH,gs,bf16,gate,before", CASES)
def test_norm_small(batch, L, CH, gs, bf16, gate, before):
    print(f"case batch={batch} L={L} CH={CH} gs={gs} bf16={bf16} gate={gate} before={before}", flush=True)
    d = inputs.norm_inputs(batch, L, CH, seed=CH + gs, bf16=bf16)
    dt = BF if bf16 else torch.float32
    # z as a view into a wider in-projection row, y with padded batch rows
    zbuf = torch.zeros((batch, L, CH + 72), dtype=dt, device=DEV)
    zbuf[..., 40:40 + CH] = to_dev(d["z"], dt)
    z = zbuf[..., 40:40 + CH] if gate else None
    ybuf = torch.zeros((batch, L + 2, CH), dtype=dt, device=DEV)
    ybuf[:, :L] = to_dev(d["y"], dt)
    y = ybuf[:, :L]
    out = ssd.ssd_gated_rmsnorm(y, to_dev(d["w"]), gs, z=z, norm_before_gate=before, eps=1e-5)
    torch.cuda.synchronize()
    ref = oracle.gated_rmsnorm(d["y"], d["z"] if gate else None, d["w"], gs, norm_before_gate=before,
                               eps=1e-5)
    e = rel(to_np(out), ref)
    print(f"  rel err {e:.3e}", flush=True)
    assert e <= TOL[bf16]


def test_norm_head_layout_and_out_view():
    """y straight from the scan's (batch, L, H, P) layout, out into a view of a
    wider buffer whose other bytes stay untouched."""
    d = inputs.norm_inputs(2, 33, 16 * 64, seed=5)
    y = to_dev(d["y"], BF).view(2, 33, 16, 64)
    obuf = torch.full((2, 33, 16 * 64 + 16), 9.0, dtype=BF, device=DEV)
    out = obuf[..., 8:8 + 16 * 64].unflatten(2, (16, 64))
    z = to_dev(d["z"], BF).view(2, 33, 16, 64)
    ssd.ssd_gated_rmsnorm(y, to_dev(d["w"]), 256, z=z, out=out)
    torch.cuda.synchronize()
    ref = oracle.gated_rmsnorm(d["y"], d["z"], d["w"], 256)
    assert rel(to_np(out).reshape(2, 33, -1), ref) <= TOL[True]
    assert torch.all(obuf[..., :8] == 9.0) and torch.all(obuf[..., 8 + 16 * 64:] == 9.0)


def test_norm_zero_rows_and_empty():
    """A zero row gives zeros (eps > 0), and an empty sequence launches nothing."""
    y = torch.zeros((1, 3, 1024), dtype=BF, device=DEV)
    out = ssd.ssd_gated_rmsnorm(y, torch.ones(1024, device=DEV), 512, z=torch.ones_like(y))
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    e = ssd.ssd_gated_rmsnorm(torch.zeros((2, 0, 64), dtype=BF, device=DEV), torch.ones(64, device=DEV), 64)
    assert e.numel() == 0


def test_norm_full_nemotron_h_8b():
    """The mixer output of the Nemotron-H 8B workload (4 x 4096 tokens, 8192
    channels, 8 groups of 1024) with its gate: every element."""
    print("case nemotron_h_8b gated norm (every element)", flush=True)
    d = inputs.norm_inputs(4, 4096, 8192, seed=1)
    y, z = to_dev(d["y"], BF), to_dev(d["z"], BF)
    out = ssd.ssd_gated_rmsnorm(y, to_dev(d["w"]), 1024, z=z)
    torch.cuda.synchronize()
    og = to_np(out)
    del out, y, z
    ref = oracle.gated_rmsnorm(d["y"], d["z"], d["w"], 1024)
    e = rel(og, ref)
    print(f"  rel err {e:.3e}", flush=True)
    assert e <= TOL[True]
