"""Helpers shared by the GPU parity tests: run the HIP path from numpy inputs.

Inputs come from state_space_sequence_ssd_amd.inputs (exactly representable
in the GPU dtype); expected values come from oracle/ only.
"""
import numpy as np
import torch

import oracle
from state_space_sequence_ssd_amd import ssd

DEV = torch.device("cuda:0")
BF = torch.bfloat16


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return t.to(dtype) if dtype is not None else t


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel(a, ref):
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    err = np.max(np.abs(a - ref)) if ref.size else 0.0
    return float(err / den) if den > 0 else float(err)


def split_xbc(v, H, G, P=64, N=128):
    """Views of x, B, C inside a (batch, L, conv_dim) tensor or array."""
    b, L = v.shape[0], v.shape[1]
    if isinstance(v, torch.Tensor):
        return (v[..., :H * P].view(b, L, H, P), v[..., H * P:H * P + G * N].view(b, L, G, N),
                v[..., H * P + G * N:].view(b, L, G, N))
    return (v[..., :H * P].reshape(b, L, H, P), v[..., H * P:H * P + G * N].reshape(b, L, G, N),
            v[..., H * P + G * N:].reshape(b, L, G, N))


def gpu_layer(d, w, seg_chunks=0, final=True, chunk_size=128):
    """conv (if the workload has it) + chunk scan on the GPU.  Returns (y, final_state)."""
    H, G = w.nheads, w.ngroups
    dt_t = BF if w.bf16 else torch.float32
    seq_idx = to_dev(d["seq_idx"]) if "seq_idx" in d else None
    rows = w.num_seqs
    if w.conv:
        xbc = to_dev(d["xBC"], dt_t)
        v = ssd.ssd_conv1d_silu(xbc, to_dev(d["conv_w"]), seq_idx=seq_idx,
                                num_seqs=rows if seq_idx is not None else None)
        x, B, C = split_xbc(v, H, G)
    else:
        x, B, C = to_dev(d["x"], dt_t), to_dev(d["B"], dt_t), to_dev(d["C"], dt_t)
    fs = torch.full((rows, H, 64, 128), float("nan"), device=DEV) if final else None
    init = to_dev(d["initial_state"]) if "initial_state" in d else None
    y = ssd.ssd_chunk_scan_fwd(x, to_dev(d["dt"], dt_t), to_dev(d["A"]), B, C,
                               dt_bias=to_dev(d["dt_bias"]), D=to_dev(d["D"]), seq_idx=seq_idx,
                               num_seqs=rows if seq_idx is not None else None,
                               initial_state=init, final_state=fs, seg_chunks=seg_chunks,
                               chunk_size=chunk_size)
    torch.cuda.synchronize()
    return y, fs


def oracle_layer(d, w, heads=None, rows=None):
    """Oracle of the whole layer, optionally restricted to some heads / batch rows.

    Without a restriction the oracle runs once over whole tensors (its OpenMP
    loop spreads the (row, head) recurrences over the host cores).
    Restricting is exact: the conv is per channel, and each head only reads
    its own x channels, dt column and its group's B/C channels.
    Returns y (batch', L, H', P) and final_state (rows', H', P, N).
    """
    H, G, P, N = w.nheads, w.ngroups, w.headdim, w.dstate
    if heads is None and rows is None:
        seq_idx = d.get("seq_idx")
        nseq = w.num_seqs if seq_idx is not None else None
        if w.conv:
            v = oracle.conv1d_silu(d["xBC"], d["conv_w"], seq_idx=seq_idx, num_seqs=nseq)
            x, B, C = split_xbc(v, H, G, P, N)
            del v
        else:
            x, B, C = d["x"], d["B"], d["C"]
        return oracle.ssd_scan(x, d["dt"], d["dt_bias"], d["A"], B, C, d["D"], seq_idx=seq_idx,
                               num_seqs=nseq, initial_state=d.get("initial_state"),
                               want_final_state=True)
    heads = list(range(H)) if heads is None else list(heads)
    hpg = H // G
    groups = sorted({h // hpg for h in heads})
    bsel = slice(None) if rows is None else list(rows)
    if w.conv:
        xbc = d["xBC"][bsel]
        xch = np.concatenate([np.arange(h * P, (h + 1) * P) for h in heads])
        bch = np.concatenate([H * P + np.arange(g * N, (g + 1) * N) for g in groups])
        cch = np.concatenate([H * P + G * N + np.arange(g * N, (g + 1) * N) for g in groups])
        ch = np.concatenate([xch, bch, cch])
        v = oracle.conv1d_silu(xbc[..., ch], d["conv_w"][ch], seq_idx=d.get("seq_idx"),
                               num_seqs=w.num_seqs if "seq_idx" in d else None)
        b_, L = v.shape[0], v.shape[1]
        x = v[..., :len(xch)].reshape(b_, L, len(heads), P)
        B = v[..., len(xch):len(xch) + len(bch)].reshape(b_, L, len(groups), N)
        C = v[..., len(xch) + len(bch):].reshape(b_, L, len(groups), N)
    else:
        x = d["x"][bsel][:, :, heads]
        B = d["B"][bsel][:, :, groups]
        C = d["C"][bsel][:, :, groups]
    # re-map heads onto the selected groups: run one head at a time
    ys, fss = [], []
    seq_idx = d.get("seq_idx")
    init = d.get("initial_state")
    for k, h in enumerate(heads):
        gi = groups.index(h // hpg)
        sl = slice(k, k + 1)
        if init is None:
            h0 = None
        elif seq_idx is None:
            h0 = init[bsel][:, [h]]
        else:
            h0 = init[:, [h]]
        y, fs = oracle.ssd_scan(x[:, :, sl], d["dt"][bsel][:, :, [h]], d["dt_bias"][[h]], d["A"][[h]],
                                B[:, :, gi:gi + 1], C[:, :, gi:gi + 1], d["D"][[h]],
                                seq_idx=seq_idx, num_seqs=w.num_seqs if seq_idx is not None else None,
                                initial_state=h0, want_final_state=True)
        ys.append(y)
        fss.append(fs)
    return np.concatenate(ys, axis=2), np.concatenate(fss, axis=1)
