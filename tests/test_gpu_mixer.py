"""The whole Mamba-2 mixer (in_proj -> conv + scan -> gated RMSNorm -> out_proj)
as a sequence of libssd calls, on the GPU.

* Small shapes against the oracle's chain of the same steps (linear, conv,
  scan, gated norm, linear in fp64): max|gpu - oracle| / max|oracle| <= 3e-2.
  The GPU rounds to bf16 after each of five steps (the in_proj output, the
  conv output, y, the normalised y and the result), each about 2^-9
  relative, so the bar is looser than a single step's 2e-2.
* The full Nemotron-H 8B layer shape: every step on the exact strided views
  the composition uses (x|B|C, dt and z are column slices of the in_proj
  output), each against the same call on contiguous copies, bit for bit;
  then the composition against those calls made one by one.
"""
import numpy as np
import pytest
import torch

import oracle
from state_space_sequence_ssd_amd import inputs, ssd
from tests.gpu_helpers import BF, DEV, rel, to_dev, to_np

pytestmark = pytest.mark.gpu


def dev_mixer(d):
    t = {k: to_dev(v, BF if k in ("hidden", "in_proj_w", "out_proj_w") else None) for k, v in d.items()}
    return t


def oracle_mixer(d, H, G, P=64, N=128, eps=1e-5):
    batch, L, _ = d["hidden"].shape
    d_inner, conv_dim = H * P, H * P + 2 * G * N
    zxbcdt = oracle.linear(d["hidden"].reshape(batch * L, -1), d["in_proj_w"]).reshape(batch, L, -1)
    z = zxbcdt[..., :d_inner]
    xbc = zxbcdt[..., d_inner:d_inner + conv_dim]
    dt = zxbcdt[..., d_inner + conv_dim:]
    v = oracle.conv1d_silu(xbc, d["conv_w"])
    x = v[..., :d_inner].reshape(batch, L, H, P)
    B = v[..., d_inner:d_inner + G * N].reshape(batch, L, G, N)
    C = v[..., d_inner + G * N:].reshape(batch, L, G, N)
    y = oracle.ssd_scan(x, dt, d["dt_bias"], d["A"], B, C, d["D"])
    yn = oracle.gated_rmsnorm(y.reshape(batch, L, d_inner), z, d["norm_w"], d_inner // G, eps=eps)
    return oracle.linear(yn.reshape(batch * L, d_inner), d["out_proj_w"]).reshape(batch, L, -1)


@pytest.mark.parametrize("batch,L,d_model,H,G", [(2, 300, 256, 8, 2), (1, 513, 512, 16, 4)])
def test_mixer_small(batch, L, d_model, H, G):
    print(f"case mixer batch={batch} L={L} d_model={d_model} H={H} G={G}", flush=True)
    d = inputs.mixer_inputs(batch, L, d_model, H, G, seed=9)
    t = dev_mixer(d)
    out = ssd.mamba2_mixer_fwd(t["hidden"], t["in_proj_w"], t["conv_w"], t["dt_bias"], t["A"], t["D"],
                               t["norm_w"], t["out_proj_w"], H, G)
    torch.cuda.synchronize()
    ref = oracle_mixer(d, H, G)
    e = rel(to_np(out), ref)
    print(f"  mixer rel err {e:.3e}", flush=True)
    assert e <= 3e-2


def _zxbcdt(L, H, G, seed, batch=1, P=64, N=128):
    width = 2 * H * P + 2 * G * N + H
    return to_dev(inputs.normal((batch, L, width), 1.0, seed, 40, True), BF)


def test_mixer_views_full_size():
    """Nemotron-H 8B shape (4 x 4096 tokens, 128 heads, 8 groups): the fused conv +
    scan on the x|B|C and dt column views of an in_proj output, and the gated norm
    on the z view, equal the same calls on contiguous copies bit for bit."""
    H, G, P, N, batch, L = 128, 8, 64, 128, 4, 4096
    d_inner, conv_dim = H * P, H * P + 2 * G * N
    print(f"case mixer views batch={batch} L={L} H={H} G={G}", flush=True)
    zx = _zxbcdt(L, H, G, seed=10, batch=batch)
    z, xbc, dt = zx[..., :d_inner], zx[..., d_inner:d_inner + conv_dim], zx[..., d_inner + conv_dim:]
    d = inputs.mixer_inputs(1, 1, 64, H, G, seed=9)   # per-channel and per-head parameters only
    cw, dtb, A, D, nw = (to_dev(d[k]) for k in ("conv_w", "dt_bias", "A", "D", "norm_w"))
    fs_v = torch.empty((batch, H, P, N), device=DEV)
    fs_c = torch.empty_like(fs_v)
    y_v = ssd.ssd_conv_scan_fwd(xbc, cw, dt, A, H, G, dt_bias=dtb, D=D, final_state=fs_v)
    y_c = ssd.ssd_conv_scan_fwd(xbc.contiguous(), cw, dt.contiguous(), A, H, G, dt_bias=dtb, D=D, final_state=fs_c)
    torch.cuda.synchronize()
    assert torch.equal(y_v, y_c) and torch.equal(fs_v, fs_c)
    n_v = ssd.ssd_gated_rmsnorm(y_v.flatten(2), nw, d_inner // G, z=z)
    n_c = ssd.ssd_gated_rmsnorm(y_v.flatten(2), nw, d_inner // G, z=z.contiguous())
    torch.cuda.synchronize()
    assert torch.equal(n_v, n_c)
    assert bool(torch.isfinite(n_v.float()).all())


def test_mixer_full_size():
    """The composition at the Nemotron-H 8B layer shape (d_model 4096) equals its
    steps called one by one."""
    H, G, batch, L, d_model = 128, 8, 4, 4096, 4096
    d_inner = H * 64
    print(f"case mixer full size batch={batch} L={L} d_model={d_model}", flush=True)
    d = inputs.mixer_inputs(batch, L, d_model, H, G, seed=9)
    t = dev_mixer(d)
    out = ssd.mamba2_mixer_fwd(t["hidden"], t["in_proj_w"], t["conv_w"], t["dt_bias"], t["A"], t["D"],
                               t["norm_w"], t["out_proj_w"], H, G)
    zx = ssd.ssd_linear(t["hidden"], t["in_proj_w"])
    conv_dim = d_inner + 2 * G * 128
    y = ssd.ssd_conv_scan_fwd(zx[..., d_inner:d_inner + conv_dim].contiguous(), t["conv_w"],
                              zx[..., d_inner + conv_dim:].contiguous(), t["A"], H, G, dt_bias=t["dt_bias"],
                              D=t["D"])
    yn = ssd.ssd_gated_rmsnorm(y.flatten(2), t["norm_w"], d_inner // G, z=zx[..., :d_inner].contiguous())
    ref = ssd.ssd_linear(yn, t["out_proj_w"])
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert bool(torch.isfinite(out.float()).all())
