"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Bars: max|gpu - oracle| / max|oracle| <= 2e-2 for bf16 inputs (fp32 state and
accumulation), <= 1e-4 for fp32 inputs; the same bound separately for final
states.  Integer-like outputs (the conv-state shift) are compared bit-exactly.
"""
import numpy as np
import pytest
import torch

import oracle
from state_space_sequence_ssd_amd import inputs, ssd
from tests.gpu_helpers import BF, DEV, gpu_layer, oracle_layer, rel, split_xbc, to_dev, to_np

pytestmark = pytest.mark.gpu

TOL = {True: 2e-2, False: 1e-4}


def W(name, batch, L, H, G, bf16=True, conv=False, init=0.0, lens=None):
    if lens is not None:
        L = int(np.sum(lens))
    return inputs.ScanWorkload(name, batch, L, H, G, bf16=bf16, conv=conv, final_state=True,
                               packed_lengths=None if lens is None else np.asarray(lens),
                               init_std=init)


SMALL = [
    # (workload, seg_chunks)
    (W("bf16_conv_b2_l300_h16_g4_init", 2, 300, 16, 4, conv=True, init=0.3), 0),
    (W("bf16_b1_l129_h8_g2", 1, 129, 8, 2), 0),
    (W("bf16_b3_l128_h4_g4", 3, 128, 4, 4), 0),
    (W("bf16_b1_l1_h8_g1_init", 1, 1, 8, 1, init=0.3), 0),
    (W("bf16_seg1_b1_l700_h8_g2_init", 1, 700, 8, 2, init=0.3), 1),
    (W("bf16_seg2_conv_b2_l1000_h8_g8", 2, 1000, 8, 8, conv=True), 2),
    (W("bf16_packed_h8_g2_init", 1, 0, 8, 2, init=0.3, lens=[1, 3, 200, 129, 128, 64, 300, 2]), 0),
    (W("bf16_packed_seg1_h8_g2_init", 1, 0, 8, 2, init=0.3, lens=[1, 3, 200, 129, 128, 64, 300, 2]), 1),
    (W("bf16_packed_conv_h16_g8", 1, 0, 16, 8, conv=True, lens=[77, 5, 260]), 0),
    # sequences with no token (first, middle, last): their final state is their initial one
    (W("bf16_packed_empty_h8_g2_init", 1, 0, 8, 2, init=0.3, lens=[0, 5, 0, 130, 1, 0]), 0),
    (W("bf16_packed_empty_conv_seg1_h8_g2", 1, 0, 8, 2, conv=True, lens=[0, 200, 0, 3]), 1),
    # fp32 batch rows up to 1024 tokens: the one-launch quadratic form
    (inputs.tiny_fp32(), 0),
    (W("fp32_conv_b2_l200_h8_g2_init", 2, 200, 8, 2, bf16=False, conv=True, init=0.3), 0),
    (W("fp32_seg1_b1_l300_h4_g1_init", 1, 300, 4, 1, bf16=False, init=0.3), 1),
    (W("fp32_b1_l1_h4_g1_init", 1, 1, 4, 1, bf16=False, init=0.3), 0),
    (W("fp32_b3_l1000_h4_g2_init", 3, 1000, 4, 2, bf16=False, init=0.3), 0),
    (W("fp32_b1_l1024_h8_g1", 1, 1024, 8, 1, bf16=False), 0),
    # longer fp32 rows and packed streams: the chunked fp32 kernel
    (W("fp32_b1_l1100_h4_g1_init", 1, 1100, 4, 1, bf16=False, init=0.3), 0),
    (W("fp32_seg2_b2_l1500_h4_g2", 2, 1500, 4, 2, bf16=False), 2),
    (W("fp32_packed_h4_g2_init", 1, 0, 4, 2, bf16=False, init=0.3, lens=[130, 1, 7, 128]), 0),
]


@pytest.mark.parametrize("w,seg", SMALL, ids=[f"{w.name}" for w, _ in SMALL])
def test_layer_small(w, seg):
    print(f"case {w.name} seg_chunks={seg}", flush=True)
    d = inputs.make_scan_inputs(w, seed=11)
    y, fs = gpu_layer(d, w, seg_chunks=seg)
    ry, rf = oracle_layer(d, w)
    ey, ef = rel(to_np(y), ry), rel(to_np(fs), rf)
    print(f"  y rel err {ey:.3e}  final-state rel err {ef:.3e}")
    assert ey <= TOL[w.bf16] and ef <= TOL[w.bf16]


@pytest.mark.parametrize("q", [64, 256])
def test_model_chunk_sizes(q):
    """chunk_size 64 or 256 (the model's chunk length) gives the oracle's
    result: the chunked form is exact for any block length, and the kernels
    always tile by 128, so the output equals the chunk-128 run bit for bit."""
    w = W("bf16_conv_b2_l300_h16_g4_init", 2, 300, 16, 4, conv=True, init=0.3)
    print(f"case {w.name} chunk_size={q}", flush=True)
    d = inputs.make_scan_inputs(w, seed=11)
    y, fs = gpu_layer(d, w, chunk_size=q)
    y128, fs128 = gpu_layer(d, w)
    ry, rf = oracle_layer(d, w)
    ey, ef = rel(to_np(y), ry), rel(to_np(fs), rf)
    print(f"  y rel err {ey:.3e}  final-state rel err {ef:.3e}")
    assert ey <= TOL[True] and ef <= TOL[True]
    assert torch.equal(y, y128) and torch.equal(fs, fs128)


def test_fp32_block_length_invariance():
    """One fp32 sequence of 1,000 tokens through kernels that cut it into
    different blocks: the masked quadratic form over the whole row (one block
    of 1,000), the chunked fp32 kernel as a one-sequence packed stream (64-token
    sub-chunks), and the same with 128-token segments joined by the combine.
    The chunked form is exact for any block length, so the three agree to
    fp32 rounding and each matches the oracle.  Bound 2e-5 of the largest
    value: the chunked kernel hands the state from chunk to chunk 16 times
    (an fp32 decay product and sum each, ~2^-24 relative per operation) on
    top of fp32 cumulative log-decays within a chunk; measured 7.6e-6 for
    the final state, 2e-7 for y."""
    w = W("f32_b1_l1000_h8_g2_init", 1, 1000, 8, 2, bf16=False, init=0.3)
    d = inputs.make_scan_inputs(w, seed=23)
    ry, rf = oracle_layer(d, w)
    y_quad, f_quad = gpu_layer(d, w)
    dp = dict(d, seq_idx=np.zeros(w.seqlen, np.int32))
    y_chunk, f_chunk = gpu_layer(dp, w)
    y_seg, f_seg = gpu_layer(dp, w, seg_chunks=1)
    for name, (y, f) in {"quad": (y_quad, f_quad), "chunk": (y_chunk, f_chunk), "seg": (y_seg, f_seg)}.items():
        ey, ef = rel(to_np(y), ry), rel(to_np(f), rf)
        print(f"  {name}: y rel err {ey:.3e}  final-state rel err {ef:.3e}", flush=True)
        assert ey <= 1e-4 and ef <= 1e-4, name
    for a_, b_ in ((y_quad, y_chunk), (y_chunk, y_seg), (f_quad, f_chunk), (f_chunk, f_seg)):
        assert rel(to_np(a_), to_np(b_)) <= 2e-5


def test_fp32_long_row():
    """fp32 inputs over 16,384 tokens (256 chunk hand-offs of the fp32 state,
    automatic segments): y and the final state within the fp32 bar."""
    w = W("f32_b1_l16384_h8_g2_init", 1, 16384, 8, 2, bf16=False, init=0.3)
    print(f"case {w.name}", flush=True)
    d = inputs.make_scan_inputs(w, seed=29)
    y, fs = gpu_layer(d, w)
    ry, rf = oracle_layer(d, w)
    ey, ef = rel(to_np(y), ry), rel(to_np(fs), rf)
    print(f"  y rel err {ey:.3e}  final-state rel err {ef:.3e}", flush=True)
    assert ey <= 1e-4 and ef <= 1e-4


def test_packed_many_short_sequences():
    """5,000 sequences of 0-3 tokens: more work items than the plan ranks by
    length (they keep list order), empty sequences among them, and chunks
    holding several sequences."""
    rng = np.random.default_rng(17)
    lens = rng.integers(0, 4, 5000)
    w = W("bf16_packed_5000seqs_h2_g1_init", 1, 0, 2, 1, init=0.3, lens=lens)
    print(f"case {w.name} tokens={int(lens.sum())}", flush=True)
    d = inputs.make_scan_inputs(w, seed=19)
    y, fs = gpu_layer(d, w)
    ry, rf = oracle_layer(d, w)
    ey, ef = rel(to_np(y), ry), rel(to_np(fs), rf)
    print(f"  y rel err {ey:.3e}  final-state rel err {ef:.3e}")
    assert ey <= TOL[True] and ef <= TOL[True]


@pytest.mark.parametrize("nseq", [100, 200, 300])
def test_packed_sequence_counts(nseq):
    """Packed streams whose sequence count sets how many lanes share each
    sequence-bound search in the planner (8, 4 and 2 lanes at 100, 200 and
    300 sequences), with empty sequences among them."""
    rng = np.random.default_rng(nseq)
    lens = rng.integers(0, 40, nseq) * (rng.random(nseq) < 0.85)
    w = W(f"bf16_packed_{nseq}seqs_h2_g1_init", 1, 0, 2, 1, init=0.3, lens=lens)
    print(f"case {w.name} tokens={int(lens.sum())}", flush=True)
    d = inputs.make_scan_inputs(w, seed=nseq + 1)
    y, fs = gpu_layer(d, w)
    ry, rf = oracle_layer(d, w)
    ey, ef = rel(to_np(y), ry), rel(to_np(fs), rf)
    print(f"  y rel err {ey:.3e}  final-state rel err {ef:.3e}")
    assert ey <= TOL[True] and ef <= TOL[True]


def test_strong_decay():
    """Heads whose 32-token blocks decay by more than e^64 next to heads with
    mild decay, and a head with A = -1e4 that drives every off-diagonal term
    to zero: the mask tiles' exponents span the whole fp32 range."""
    w = W("bf16_strong_decay_b2_l300_h8_g2_init", 2, 300, 8, 2, init=0.3)
    d = inputs.make_scan_inputs(w, seed=21)
    d["A"] = (d["A"] * np.array([1, 40, 1, 80, 5, 200, 1, 1], np.float32)).astype(np.float32)
    d["A"][6] = np.float32(-1e4)
    dt = np.logaddexp(0.0, d["dt"].astype(np.float64) + d["dt_bias"][None, None, :])
    blocks = np.add.reduceat(-(dt[:, :288] * d["A"]), np.arange(0, 288, 32), axis=1)
    print(f"max 32-block log-decay per head: {blocks.max(axis=(0, 1)).round(1)}", flush=True)
    assert (blocks.max(axis=(0, 1)) > 64).sum() >= 3 and (blocks.max(axis=(0, 1)) < 64).sum() >= 3
    y, fs = gpu_layer(d, w)
    ry, rf = oracle_layer(d, w)
    ey, ef = rel(to_np(y), ry), rel(to_np(fs), rf)
    print(f"  y rel err {ey:.3e}  final-state rel err {ef:.3e}")
    assert ey <= TOL[True] and ef <= TOL[True]


def test_in_proj_layout_strided_views():
    """x, B, C and dt as views into one in-projection output per token
    (z | x | B | C | dt | pad), batch rows padded by 3 tokens, and y written
    into a view of a wider buffer: every token and batch stride differs from
    its row width.  Bytes outside y's view stay untouched."""
    w = W("bf16_inproj_views_b2_l300_h8_g2_init", 2, 300, 8, 2, init=0.3)
    d = inputs.make_scan_inputs(w, seed=17)
    H, G, P, N, Bt, L = w.nheads, w.ngroups, 64, 128, w.batch, w.seqlen
    HP, GN = H * P, G * N
    width = 2 * HP + 2 * GN + H + 8
    buf = torch.zeros((Bt, L + 3, width), dtype=BF, device=DEV)
    buf[:, :L, HP:2 * HP] = to_dev(d["x"], BF).reshape(Bt, L, HP)
    buf[:, :L, 2 * HP:2 * HP + GN] = to_dev(d["B"], BF).reshape(Bt, L, GN)
    buf[:, :L, 2 * HP + GN:2 * HP + 2 * GN] = to_dev(d["C"], BF).reshape(Bt, L, GN)
    buf[:, :L, 2 * HP + 2 * GN:2 * HP + 2 * GN + H] = to_dev(d["dt"], BF)
    x = buf[:, :L, HP:2 * HP].unflatten(2, (H, P))
    Bv = buf[:, :L, 2 * HP:2 * HP + GN].unflatten(2, (G, N))
    Cv = buf[:, :L, 2 * HP + GN:2 * HP + 2 * GN].unflatten(2, (G, N))
    dtv = buf[:, :L, 2 * HP + 2 * GN:2 * HP + 2 * GN + H]
    ybuf = torch.full((Bt, L, HP + 64), 7.0, dtype=BF, device=DEV)
    y = ybuf[..., 32:32 + HP].unflatten(2, (H, P))
    fs = torch.empty((Bt, H, P, N), device=DEV)
    ssd.ssd_chunk_scan_fwd(x, dtv, to_dev(d["A"]), Bv, Cv, dt_bias=to_dev(d["dt_bias"]), D=to_dev(d["D"]),
                           initial_state=to_dev(d["initial_state"]), final_state=fs, y=y)
    torch.cuda.synchronize()
    ry, rf = oracle_layer(d, w)
    ey, ef = rel(to_np(y), ry), rel(to_np(fs), rf)
    print(f"  y rel err {ey:.3e}  final-state rel err {ef:.3e}")
    assert ey <= TOL[True] and ef <= TOL[True]
    assert torch.all(ybuf[..., :32] == 7.0) and torch.all(ybuf[..., 32 + HP:] == 7.0)


def test_empty_sequence_keeps_initial_state():
    w = W("bf16_l0", 2, 0, 8, 2, init=0.3)
    d = inputs.make_scan_inputs(w, seed=3)
    y, fs = gpu_layer(d, w)
    assert y.numel() == 0
    assert torch.equal(fs.cpu(), torch.from_numpy(d["initial_state"]))


def test_repeat_runs_bitwise_identical():
    w = W("bf16_conv_b2_l600_h16_g4", 2, 600, 16, 4, conv=True, init=0.3)
    d = inputs.make_scan_inputs(w, seed=13)
    y1, f1 = gpu_layer(d, w, seg_chunks=2)
    y2, f2 = gpu_layer(d, w, seg_chunks=2)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


def test_segmentation_invariance():
    """Different segment splits of one sequence agree with each other and the oracle."""
    w = W("bf16_b1_l1500_h8_g2_init", 1, 1500, 8, 2, init=0.3)
    d = inputs.make_scan_inputs(w, seed=17)
    ry, rf = oracle_layer(d, w)
    for seg in (0, 1, 3, 12):
        y, fs = gpu_layer(d, w, seg_chunks=seg)
        assert rel(to_np(y), ry) <= 2e-2 and rel(to_np(fs), rf) <= 2e-2, seg


# ---------------------------------------------------------------------------
# conv alone (bf16 + fp32, packed, conv state in/out)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("bf16", [True, False])
def test_conv_states_and_packing(bf16):
    r = np.random.default_rng(5)
    CH, lens = 48, [2, 40, 1, 70]
    L = sum(lens)
    x = inputs.normal((1, L, CH), 1.0, 7, 1, bf16)
    w = (r.standard_normal((CH, 4)) * 0.5).astype(np.float32)
    b = (r.standard_normal(CH) * 0.1).astype(np.float32)
    st_in = inputs.normal((len(lens), 3, CH), 1.0, 7, 2, bf16)
    seq = np.repeat(np.arange(len(lens), dtype=np.int32), lens)
    dt = BF if bf16 else torch.float32
    so = torch.zeros((len(lens), 3, CH), dtype=dt, device=DEV)
    out = ssd.ssd_conv1d_silu(to_dev(x, dt), to_dev(w), bias=to_dev(b), seq_idx=to_dev(seq),
                              num_seqs=len(lens), conv_state_in=to_dev(st_in, dt), conv_state_out=so)
    torch.cuda.synchronize()
    ref, rso = oracle.conv1d_silu(x, w, bias=b, seq_idx=seq, num_seqs=len(lens), conv_state_in=st_in,
                                  want_state_out=True)
    assert rel(to_np(out), ref) <= TOL[bf16]
    assert np.array_equal(to_np(so), rso), "conv state export must be exact"


def test_conv_batch_mode_strided_input():
    """conv on a strided view (token stride > channels), batch rows, no state."""
    H, G = 8, 2
    w_ = W("c", 3, 333, H, G, conv=True)
    d = inputs.make_scan_inputs(w_, seed=9)
    CD = w_.conv_dim
    big = torch.zeros((3, 333, CD + 64), dtype=BF, device=DEV)
    big[..., 16:16 + CD] = to_dev(d["xBC"], BF)
    xv = big[..., 16:16 + CD]
    out = ssd.ssd_conv1d_silu(xv, to_dev(d["conv_w"]))
    torch.cuda.synchronize()
    ref = oracle.conv1d_silu(d["xBC"], d["conv_w"])
    assert rel(to_np(out), ref) <= 2e-2


# ---------------------------------------------------------------------------
# decode step
# ---------------------------------------------------------------------------
def test_debug_seq_idx_checks(monkeypatch):
    """SSD_DEBUG=1: a valid seq_idx runs unchanged; a decreasing or out-of-range
    one is refused (INVALID_ARG naming the first bad token) before any kernel
    reads by it."""
    w = W("bf16_packed_conv_h8_g2", 1, 0, 8, 2, conv=True, lens=[5, 130, 1, 64])
    d = inputs.make_scan_inputs(w, seed=4)
    y0, f0 = gpu_layer(d, w)
    monkeypatch.setenv("SSD_DEBUG", "1")
    y1, f1 = gpu_layer(d, w)
    assert torch.equal(y0, y1) and torch.equal(f0, f1)
    H, G, L = w.nheads, w.ngroups, w.seqlen
    xbc = to_dev(d["xBC"], BF)
    x, B, C = split_xbc(xbc, H, G)
    good = d["seq_idx"]
    for name, seq, first in [("decreasing", np.where(np.arange(L) == 100, 0, good), 100),
                             ("too large", np.where(np.arange(L) >= 150, 4, good), 150),
                             ("negative", np.where(np.arange(L) == 0, -1, good), 0)]:
        print(f"case {name}: first bad token {first}", flush=True)
        sq = to_dev(seq.astype(np.int32))
        with pytest.raises(ssd.SsdError) as ei:
            ssd.ssd_conv1d_silu(xbc, to_dev(d["conv_w"]), seq_idx=sq, num_seqs=4)
        assert ei.value.code == 1 and f"seq_idx[{first}]" in str(ei.value)
        with pytest.raises(ssd.SsdError) as ei:
            ssd.ssd_chunk_scan_fwd(x, to_dev(d["dt"], BF), to_dev(d["A"]), B, C, seq_idx=sq, num_seqs=4,
                                   final_state=torch.empty((4, H, 64, 128), device=DEV))
        assert ei.value.code == 1 and f"seq_idx[{first}]" in str(ei.value)
    torch.cuda.synchronize()


@pytest.mark.parametrize("bf16,conv", [(True, True), (True, False), (False, True), (False, False)])
def test_decode_small(bf16, conv):
    w = inputs.DecodeWorkload("dec", 3, 16, 4, 1, bf16=bf16)
    d = inputs.make_decode_small_inputs(w, seed=21, layer=0)
    st = inputs.decode_state_host(w, 21, 0)
    dt = BF if bf16 else torch.float32
    state = to_dev(st)
    cs = to_dev(d["conv_state"], dt) if conv else None
    y = ssd.ssd_decode_step(to_dev(d["xBC"], dt), to_dev(d["dt"], dt), to_dev(d["A"]), state,
                            w.nheads, w.ngroups, dt_bias=to_dev(d["dt_bias"]), D=to_dev(d["D"]),
                            conv_state=cs, conv_weight=to_dev(d["conv_w"]) if conv else None)
    torch.cuda.synchronize()
    ry, rs, rc = oracle.decode_step(d["xBC"], d["dt"], d["dt_bias"], d["A"], d["D"], st, w.nheads,
                                    64, 128, w.ngroups, conv_w=d["conv_w"] if conv else None,
                                    conv_state=d["conv_state"] if conv else None)
    assert rel(to_np(y), ry) <= TOL[bf16]
    assert rel(to_np(state), rs) <= TOL[bf16]
    if conv:
        assert np.array_equal(to_np(cs), rc)


def test_decode_strided_rows():
    """Decode with the token (x|B|C) and dt as views into one wider row per
    batch entry, and y written into a wider buffer (batch strides > widths)."""
    w = inputs.DecodeWorkload("dec_views", 5, 16, 4, 1)
    d = inputs.make_decode_small_inputs(w, seed=23, layer=0)
    st = inputs.decode_state_host(w, 23, 0)
    CD, H = w.conv_dim, w.nheads
    row = torch.zeros((w.batch, 40 + CD + H + 24), dtype=BF, device=DEV)
    row[:, 40:40 + CD] = to_dev(d["xBC"], BF)
    row[:, 40 + CD:40 + CD + H] = to_dev(d["dt"], BF)
    state, cs = to_dev(st), to_dev(d["conv_state"], BF)
    ybuf = torch.full((w.batch, H * 64 + 32), 3.0, dtype=BF, device=DEV)
    y = ybuf[:, 16:16 + H * 64].unflatten(1, (H, 64))
    ssd.ssd_decode_step(row[:, 40:40 + CD], row[:, 40 + CD:40 + CD + H], to_dev(d["A"]), state, H, w.ngroups,
                        dt_bias=to_dev(d["dt_bias"]), D=to_dev(d["D"]), conv_state=cs,
                        conv_weight=to_dev(d["conv_w"]), y=y)
    torch.cuda.synchronize()
    ry, rs, rc = oracle.decode_step(d["xBC"], d["dt"], d["dt_bias"], d["A"], d["D"], st, H, 64, 128,
                                    w.ngroups, conv_w=d["conv_w"], conv_state=d["conv_state"])
    assert rel(to_np(y), ry) <= TOL[True] and rel(to_np(state), rs) <= TOL[True]
    assert np.array_equal(to_np(cs), rc)
    assert torch.all(ybuf[:, :16] == 3.0) and torch.all(ybuf[:, 16 + H * 64:] == 3.0)


def test_prefill_then_decode_chain():
    """GPU prefill of L tokens (conv state + final state out) then GPU decode of
    token L == oracle prefill of L+1 tokens."""
    H, G, L = 8, 2, 257
    w = W("chain", 1, L + 1, H, G, conv=True, init=0.3)
    d = inputs.make_scan_inputs(w, seed=23)
    xbc = to_dev(d["xBC"], BF)
    cso = torch.zeros((1, 3, w.conv_dim), dtype=BF, device=DEV)
    v = ssd.ssd_conv1d_silu(xbc[:, :L], to_dev(d["conv_w"]), conv_state_out=cso)
    x, B, C = split_xbc(v, H, G)
    fs = torch.zeros((1, H, 64, 128), device=DEV)
    ssd.ssd_chunk_scan_fwd(x, to_dev(d["dt"], BF)[:, :L], to_dev(d["A"]), B, C,
                           dt_bias=to_dev(d["dt_bias"]), D=to_dev(d["D"]),
                           initial_state=to_dev(d["initial_state"]), final_state=fs)
    yd = ssd.ssd_decode_step(xbc[:, L].contiguous(), to_dev(d["dt"], BF)[:, L].contiguous(), to_dev(d["A"]),
                             fs, H, G, dt_bias=to_dev(d["dt_bias"]), D=to_dev(d["D"]), conv_state=cso,
                             conv_weight=to_dev(d["conv_w"]))
    torch.cuda.synchronize()
    ry, rf = oracle_layer(d, w)
    assert rel(to_np(yd), ry[:, L]) <= 2e-2
    assert rel(to_np(fs), rf) <= 2e-2


# ---------------------------------------------------------------------------
# full-size workloads, in the launch configuration the benchmark times,
# every element compared with the oracle
# ---------------------------------------------------------------------------
def _full(w, seed):
    print(f"case {w.name} seed={seed} (every head and row)", flush=True)
    d = inputs.make_scan_inputs(w, seed=seed)
    y, fs = gpu_layer(d, w)
    yg, fg = to_np(y), to_np(fs)
    del y, fs
    torch.cuda.empty_cache()
    ry, rf = oracle_layer(d, w)
    ey, ef = rel(yg, ry), rel(fg, rf)
    print(f"  y rel err {ey:.3e}  final-state rel err {ef:.3e}", flush=True)
    assert ey <= TOL[w.bf16] and ef <= TOL[w.bf16]


def test_full_tiny_fp32():
    _full(inputs.tiny_fp32(), seed=0)


def test_full_nemotron_h_8b():
    _full(inputs.nemotron_h_8b(), seed=1)


def test_full_nemotron3_nano():
    _full(inputs.nemotron3_nano(), seed=2)


def test_full_packed_3b():
    _full(inputs.packed_3b(), seed=3)


@pytest.mark.parametrize("layer", [0, 28])
def test_full_decode_layer(layer):
    """Every batch row of one decode layer (first application on fresh states)."""
    w = inputs.decode_29_layers()
    print(f"case {w.name} layer={layer} (all {w.batch} rows)", flush=True)
    d = inputs.make_decode_small_inputs(w, seed=4, layer=layer)
    state = inputs.decode_state_device(w, 4, layer, DEV)
    st0 = state.cpu().numpy()
    cs = to_dev(d["conv_state"], BF)
    y = ssd.ssd_decode_step(to_dev(d["xBC"], BF), to_dev(d["dt"], BF), to_dev(d["A"]), state,
                            w.nheads, w.ngroups, dt_bias=to_dev(d["dt_bias"]), D=to_dev(d["D"]),
                            conv_state=cs, conv_weight=to_dev(d["conv_w"]))
    torch.cuda.synchronize()
    yg, sg = to_np(y), state.cpu().numpy()
    del state
    torch.cuda.empty_cache()
    ry, rs, rc = oracle.decode_step(d["xBC"], d["dt"], d["dt_bias"], d["A"], d["D"], st0,
                                    w.nheads, 64, 128, w.ngroups, conv_w=d["conv_w"],
                                    conv_state=d["conv_state"])
    del st0
    ey, es = rel(yg, ry), rel(sg, rs)
    print(f"  y rel err {ey:.3e}  state rel err {es:.3e}", flush=True)
    assert ey <= 2e-2 and es <= 2e-2
    assert np.array_equal(to_np(cs), rc), "the conv-state shift is exact"


# ---------------------------------------------------------------------------
# dt = 0 exactly (dt_raw = -inf): y = D x + C h0 and the state stays frozen
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("bf16,seg,packed", [(True, 0, False), (True, 1, False), (True, 0, True),
                                             (False, 0, False), (False, 1, True)])
def test_dt_zero(bf16, seg, packed):
    """Heads 1 and 4 get dt_raw = -inf on every token (dt = 0: nothing enters
    the state and nothing decays, so y = D x + C h0 and the final state is the
    initial one, bit for bit); head 6 only on tokens 50..169, the others
    never.  Batch rows, segmented and packed launches, both dtypes."""
    H, G = 8, 2
    if packed:
        w = W(f"dt0_packed_bf16{int(bf16)}", 1, 0, H, G, bf16=bf16, init=0.3, lens=[90, 1, 200, 37])
    else:
        w = W(f"dt0_bf16{int(bf16)}", 2, 300, H, G, bf16=bf16, init=0.3)
    print(f"case {w.name} seg_chunks={seg}", flush=True)
    d = inputs.make_scan_inputs(w, seed=29)
    d["dt"][:, :, [1, 4]] = -np.inf
    d["dt"][:, 50:170, 6] = -np.inf
    y, fs = gpu_layer(d, w, seg_chunks=seg)
    ry, rf = oracle_layer(d, w)
    ey, ef = rel(to_np(y), ry), rel(to_np(fs), rf)
    print(f"  y rel err {ey:.3e}  final-state rel err {ef:.3e}", flush=True)
    assert np.all(np.isfinite(to_np(y)))
    assert ey <= TOL[bf16] and ef <= TOL[bf16]
    fz = fs[:, [1, 4]].cpu().numpy()
    assert np.array_equal(fz, d["initial_state"][:, [1, 4]]), "dt = 0 must freeze the state exactly"
    # the frozen heads' output is the closed form D x + C h0 (within the bar)
    xs = d["x"].astype(np.float64)
    g_of = np.arange(H) // (H // G)
    for h in (1, 4):
        if packed:
            seq = d["seq_idx"]
            cform = np.einsum("tn,tpn->tp", d["C"][0, :, g_of[h]].astype(np.float64),
                              d["initial_state"][seq, h].astype(np.float64))[None]
        else:
            cform = np.einsum("btn,bpn->btp", d["C"][:, :, g_of[h]].astype(np.float64),
                              d["initial_state"][:, h].astype(np.float64))
        ref_h = d["D"][h] * xs[:, :, h] + cform
        assert rel(to_np(y[:, :, h]), ref_h) <= TOL[bf16]
