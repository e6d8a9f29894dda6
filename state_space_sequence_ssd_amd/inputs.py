"""Seeded synthetic inputs for the SSD layer.

This module only draws numbers; it holds none of the layer's arithmetic, so
both the GPU path's tests and the fp64 oracle consume exactly the same
values.  Draws use numpy's PCG64 seeded per (workload, field); bf16 fields
are drawn in fp32 and rounded to the nearest bf16 (ties to even), so the
float32 arrays returned here hold exactly the values the GPU receives.

Distributions (variance notation N(mean, var)):
    x, dt_raw, D ~ N(0, 1)          B, C ~ N(0, 1/128)
    softplus(dt_bias) log-uniform in [1e-3, 1e-1]
    A = -exp(U(log 1, log 16))      conv weight ~ N(0, 1/4)
    packed initial_state ~ N(0, 0.1)   decode ssm_state ~ N(0, 1)
Shapes follow the Mamba-2 configurations of the pages: head_dim 64,
d_state 128, n_groups 8, chunk 128, conv width 4 ("Nemotron-H style Hybrid
Mamba-Transformer 3B feasibility study", sec. 1.4, 1.5, 2.2), and the 29
Mamba-2 layers of "Bamba-9B" (model architecture section).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

HEADDIM = 64
DSTATE = 128
CHUNK = 128
CONV_WIDTH = 4


def bf16_round(a) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    out = rounded.astype(np.uint32).view(np.float32).reshape(a.shape)
    # NaN/inf pass through untouched (never produced by these generators)
    bad = ~np.isfinite(a)
    if bad.any():
        out = np.where(bad, a, out)
    return out


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(seed), int(stream)]))


def normal(shape, std: float, seed: int, stream: int, bf16: bool) -> np.ndarray:
    a = _rng(seed, stream).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return bf16_round(a) if bf16 else a


def head_params(H: int, seed: int):
    """dt_bias, A, D per head (fp32)."""
    r = _rng(seed, 101)
    d = np.exp(r.uniform(np.log(1e-3), np.log(1e-1), size=H))
    dt_bias = np.log(np.expm1(d)).astype(np.float32)      # softplus(dt_bias) = d
    A = (-np.exp(r.uniform(0.0, np.log(16.0), size=H))).astype(np.float32)
    D = r.standard_normal(size=H).astype(np.float32)
    return dt_bias, A, D


def conv_weight(channels: int, seed: int, width: int = CONV_WIDTH) -> np.ndarray:
    return _rng(seed, 102).standard_normal(size=(channels, width)).astype(np.float32) * np.float32(0.5)


def packed_lengths(n: int, lo: int, hi: int, seed: int) -> np.ndarray:
    return _rng(seed, 103).integers(lo, hi + 1, size=n).astype(np.int64)


@dataclass
class ScanWorkload:
    """One prefill workload: shapes, dtype and which optional parts it uses."""
    name: str
    batch: int
    seqlen: int
    nheads: int
    ngroups: int
    bf16: bool
    conv: bool
    final_state: bool
    packed_lengths: Optional[np.ndarray] = None    # packed mode when given
    init_std: float = 0.0                          # initial_state ~ N(0, init_std^2) if > 0
    headdim: int = HEADDIM
    dstate: int = DSTATE
    chunk: int = CHUNK

    @property
    def conv_dim(self) -> int:
        return self.nheads * self.headdim + 2 * self.ngroups * self.dstate

    @property
    def num_seqs(self) -> int:
        return len(self.packed_lengths) if self.packed_lengths is not None else self.batch

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen


def make_scan_inputs(w: ScanWorkload, seed: int) -> dict:
    """All inputs of one prefill workload as float32/int32 numpy arrays.

    With w.conv the x|B|C tensor is the raw conv input `xBC` (batch, L, conv_dim)
    drawn from the x / B / C distributions per channel block; otherwise x, B, C
    are drawn directly in their (batch, L, H, P) / (batch, L, G, N) shapes.
    """
    H, G, P, N = w.nheads, w.ngroups, w.headdim, w.dstate
    L, Bt = w.seqlen, w.batch
    out = {}
    if w.conv:
        x = normal((Bt, L, H * P), 1.0, seed, 1, w.bf16)
        b = normal((Bt, L, G * N), 2.0 ** -3.5, seed, 2, w.bf16)
        c = normal((Bt, L, G * N), 2.0 ** -3.5, seed, 3, w.bf16)
        out["xBC"] = np.concatenate([x, b, c], axis=2)
        out["conv_w"] = conv_weight(w.conv_dim, seed)
    else:
        out["x"] = normal((Bt, L, H, P), 1.0, seed, 1, w.bf16)
        out["B"] = normal((Bt, L, G, N), 2.0 ** -3.5, seed, 2, w.bf16)
        out["C"] = normal((Bt, L, G, N), 2.0 ** -3.5, seed, 3, w.bf16)
    out["dt"] = normal((Bt, L, H), 1.0, seed, 4, w.bf16)
    out["dt_bias"], out["A"], out["D"] = head_params(H, seed)
    if w.packed_lengths is not None:
        lens = np.asarray(w.packed_lengths, dtype=np.int64)
        out["seq_idx"] = np.repeat(np.arange(len(lens), dtype=np.int32), lens)
    if w.init_std > 0:
        out["initial_state"] = normal((w.num_seqs, H, P, N), w.init_std, seed, 5, False)
    return out


@dataclass
class DecodeWorkload:
    name: str
    batch: int
    nheads: int
    ngroups: int
    layers: int
    bf16: bool = True
    headdim: int = HEADDIM
    dstate: int = DSTATE
    conv_width: int = CONV_WIDTH

    @property
    def conv_dim(self) -> int:
        return self.nheads * self.headdim + 2 * self.ngroups * self.dstate

    def state_bytes(self) -> int:
        return self.batch * self.nheads * self.headdim * self.dstate * 4


def make_decode_small_inputs(w: DecodeWorkload, seed: int, layer: int) -> dict:
    """Token, dt, conv state and per-head params of one decode layer (host, float32).

    The 1 GiB fp32 ssm_state is drawn separately (see decode_state_host /
    decode_state_device) so full-size runs need not materialise it on the host.
    """
    H, G, P, N = w.nheads, w.ngroups, w.headdim, w.dstate
    s = seed * 1000 + layer
    xb = [normal((w.batch, H * P), 1.0, s, 11, w.bf16),
          normal((w.batch, G * N), 2.0 ** -3.5, s, 12, w.bf16),
          normal((w.batch, G * N), 2.0 ** -3.5, s, 13, w.bf16)]
    cs = [normal((w.batch, w.conv_width - 1, H * P), 1.0, s, 14, w.bf16),
          normal((w.batch, w.conv_width - 1, G * N), 2.0 ** -3.5, s, 15, w.bf16),
          normal((w.batch, w.conv_width - 1, G * N), 2.0 ** -3.5, s, 16, w.bf16)]
    out = {
        "xBC": np.concatenate(xb, axis=1),
        "conv_state": np.concatenate(cs, axis=2),
        "dt": normal((w.batch, H), 1.0, s, 17, w.bf16),
        "conv_w": conv_weight(w.conv_dim, s),
    }
    out["dt_bias"], out["A"], out["D"] = head_params(H, s)
    return out


def decode_state_host(w: DecodeWorkload, seed: int, layer: int, batch_rows=None) -> np.ndarray:
    """ssm_state ~ N(0,1) fp32 on the host (small workloads)."""
    shape = (w.batch, w.nheads, w.headdim, w.dstate)
    return normal(shape, 1.0, seed * 1000 + layer, 18, False)


def decode_state_device(w: DecodeWorkload, seed: int, layer: int, device):
    """ssm_state ~ N(0,1) fp32 drawn on the device with torch's seeded Philox
    generator (the full-size 29 x 1 GiB states are drawn where they live)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + layer)
    return torch.randn((w.batch, w.nheads, w.headdim, w.dstate), generator=g,
                       device=device, dtype=torch.float32)


# ---------------------------------------------------------------------------
# The five synthetic workloads.
# ---------------------------------------------------------------------------

def tiny_fp32() -> ScanWorkload:
    """Tiny fp32 forward: 1 x 512 tokens, 8 heads, 1 group, no conv."""
    return ScanWorkload("tiny_fp32_h8_l512", 1, 512, 8, 1, bf16=False, conv=False,
                        final_state=True)


def nemotron_h_8b() -> ScanWorkload:
    """Nemotron-H 8B layer shape: d_model 4096 x expand 2 -> 128 heads, 8 groups,
    batch 4 x 4096 tokens, conv + SiLU before the scan."""
    return ScanWorkload("nemotron_h_8b_b4_l4096", 4, 4096, 128, 8, bf16=True, conv=True,
                        final_state=True)


def nemotron3_nano() -> ScanWorkload:
    """Nemotron 3 Nano layer shape: 64 heads, 8 groups, 1 x 16384 tokens, conv,
    final state returned."""
    return ScanWorkload("nemotron3_nano_b1_l16384", 1, 16384, 64, 8, bf16=True, conv=True,
                        final_state=True)


def packed_3b(seed: int = 3) -> ScanWorkload:
    """FRANKENSTALLM-H 3B draft shape: 40 heads, 8 groups; 32 sequences of
    U[64, 4096] tokens packed into one stream, initial states ~ N(0, 0.1)."""
    lens = packed_lengths(32, 64, 4096, seed)
    return ScanWorkload("packed_3b_h40_32seqs", 1, int(lens.sum()), 40, 8, bf16=True,
                        conv=False, final_state=True, packed_lengths=lens,
                        init_std=float(np.sqrt(0.1)))


def decode_29_layers() -> DecodeWorkload:
    """Batch-256 decode at the Nemotron-H 8B shape through 29 Mamba-2 layers."""
    return DecodeWorkload("decode_b256_h128_29layers", 256, 128, 8, 29)


def norm_inputs(batch: int, seqlen: int, channels: int, seed: int, bf16: bool = True) -> dict:
    """Inputs of the gated RMSNorm: y and z ~ N(0, 1) (the scan output and the
    gate half of the in-projection), weight ~ 1 + N(0, 0.01)."""
    return {"y": normal((batch, seqlen, channels), 1.0, seed, 21, bf16),
            "z": normal((batch, seqlen, channels), 1.0, seed, 22, bf16),
            "w": (1.0 + normal((channels,), 0.1, seed, 23, False)).astype(np.float32)}


def mixer_inputs(batch: int, seqlen: int, d_model: int, nheads: int, ngroups: int, seed: int,
                 headdim: int = HEADDIM, dstate: int = DSTATE) -> dict:
    """Hidden states and random-init weights of one Mamba-2 mixer (bf16-exact
    values): hidden ~ N(0, 1); in_proj and out_proj ~ N(0, 1/fan_in); conv
    taps ~ N(0, 1/4); norm weight ~ 1 + N(0, 0.01); per-head dt_bias, A, D as
    for the scan workloads."""
    d_inner = nheads * headdim
    conv_dim = d_inner + 2 * ngroups * dstate
    d_in_proj = 2 * d_inner + 2 * ngroups * dstate + nheads
    out = {
        "hidden": normal((batch, seqlen, d_model), 1.0, seed, 31, True),
        "in_proj_w": normal((d_in_proj, d_model), d_model ** -0.5, seed, 32, True),
        "out_proj_w": normal((d_model, d_inner), d_inner ** -0.5, seed, 33, True),
        "conv_w": conv_weight(conv_dim, seed),
        "norm_w": (1.0 + normal((d_inner,), 0.1, seed, 34, False)).astype(np.float32),
    }
    out["dt_bias"], out["A"], out["D"] = head_params(nheads, seed)
    return out


def mimo_decode_inputs(batch: int, nheads: int, ngroups: int, rank: int, seed: int, bf16: bool = True) -> dict:
    """One MIMO decode token: x, previous x ~ N(0, 1) (batch, H, P, R); B, C,
    previous B ~ N(0, 1/128) (batch, G, N, R); dt_raw ~ N(0, 1); lam ~ U(0, 1);
    per-head params as for the scan workloads.  The fp32 state is drawn
    separately (decode_state_host / decode_state_device)."""
    H, G, P, N, R = nheads, ngroups, HEADDIM, DSTATE, rank
    out = {"x": normal((batch, H, P, R), 1.0, seed, 51, bf16),
           "B": normal((batch, G, N, R), 2.0 ** -3.5, seed, 52, bf16),
           "C": normal((batch, G, N, R), 2.0 ** -3.5, seed, 53, bf16),
           "dt": normal((batch, H), 1.0, seed, 54, bf16),
           "prev_x": normal((batch, H, P, R), 1.0, seed, 55, bf16),
           "prev_B": normal((batch, G, N, R), 2.0 ** -3.5, seed, 56, bf16)}
    lam = _rng(seed, 57).uniform(0.0, 1.0, size=(batch, H)).astype(np.float32)
    out["lam"] = bf16_round(lam) if bf16 else lam
    out["dt_bias"], out["A"], out["D"] = head_params(H, seed)
    return out
