"""The Python binding refuses bad tensors before any library call (CPU only).

The C ABI sees plain pointers and one dtype code per call, so it cannot
notice a tensor of another dtype, a wrong shape or a host pointer.  The
binding checks dtype, shape and contiguity first and the device last, so
each bad tensor below raises on CPU tensors, and a call whose tensors are all
well-formed raises only for not being on a GPU.
"""
import pytest
import torch

from state_space_sequence_ssd_amd import ssd

BF = torch.bfloat16
F32 = torch.float32


def scan_inputs(batch=2, L=10, H=4, G=2, dtype=BF, packed=False):
    P, N = 64, 128
    rows = 3 if packed else batch
    t = {
        "x": torch.zeros(batch, L, H, P, dtype=dtype), "dt": torch.zeros(batch, L, H, dtype=dtype),
        "A": torch.zeros(H), "B": torch.zeros(batch, L, G, N, dtype=dtype),
        "C": torch.zeros(batch, L, G, N, dtype=dtype), "dt_bias": torch.zeros(H), "D": torch.zeros(H),
        "initial_state": torch.zeros(rows, H, P, N), "final_state": torch.zeros(rows, H, P, N),
        "y": torch.zeros(batch, L, H, P, dtype=dtype),
    }
    if packed:
        t["seq_idx"] = torch.zeros(L, dtype=torch.int32)
        t["num_seqs"] = 3
    return t


def call_scan(t):
    t = dict(t)
    return ssd.ssd_chunk_scan_fwd(t.pop("x"), t.pop("dt"), t.pop("A"), t.pop("B"), t.pop("C"), **t)


def test_scan_good_cpu_tensors_refused_as_host_memory():
    for packed in (False, True):
        with pytest.raises(ValueError, match="GPU"):
            call_scan(scan_inputs(batch=1 if packed else 2, packed=packed))


@pytest.mark.parametrize("key,bad,exc", [
    ("dt", torch.zeros(2, 10, 4, dtype=F32), TypeError),            # fp32 dt with bf16 x
    ("B", torch.zeros(2, 10, 2, 128, dtype=F32), TypeError),
    ("C", torch.zeros(2, 10, 2, 128, dtype=torch.float16), TypeError),
    ("y", torch.zeros(2, 10, 4, 64, dtype=F32), TypeError),
    ("C", torch.zeros(2, 10, 1, 128, dtype=BF), ValueError),       # C groups differ from B
    ("dt", torch.zeros(2, 9, 4, dtype=BF), ValueError),
    ("y", torch.zeros(2, 10, 4, 32, dtype=BF), ValueError),
    ("A", torch.zeros(3), ValueError),
    ("A", torch.zeros(4, dtype=BF), TypeError),
    ("dt_bias", torch.zeros(5), ValueError),
    ("D", torch.zeros(8)[::2], TypeError),                          # not contiguous
    ("final_state", torch.zeros(1, 4, 64, 128), ValueError),        # fewer rows than the batch
    ("initial_state", torch.zeros(2, 4, 64, 64), ValueError),
    ("final_state", torch.zeros(2, 4, 64, 128, dtype=BF), TypeError),
])
def test_scan_bad_tensor_raises(key, bad, exc):
    t = scan_inputs()
    t[key] = bad
    with pytest.raises(exc):
        call_scan(t)


@pytest.mark.parametrize("seq,num,exc", [
    (torch.zeros(10, dtype=torch.int64), 3, TypeError),        # int64 (arange's default)
    (torch.zeros(9, dtype=torch.int32), 3, TypeError),         # not one entry per token
    (torch.zeros(20, dtype=torch.int32)[::2], 3, TypeError),   # strided
    (torch.zeros(10, dtype=torch.int32), None, ValueError),    # num_seqs missing
])
def test_scan_bad_seq_idx_raises(seq, num, exc):
    t = scan_inputs(batch=1, packed=True)
    t["seq_idx"], t["num_seqs"] = seq, num
    with pytest.raises(exc):
        call_scan(t)


def test_scan_packed_state_rows_follow_num_seqs():
    t = scan_inputs(batch=1, packed=True)
    t["final_state"] = torch.zeros(1, 4, 64, 128)      # batch rows, but there are 3 sequences
    with pytest.raises(ValueError, match="final_state"):
        call_scan(t)


def test_scan_workspace_size_checks_too():
    t = scan_inputs()
    with pytest.raises(TypeError):
        ssd.ssd_chunk_scan_workspace_size(t["x"], t["dt"].float(), t["A"], t["B"], t["C"])


def conv_inputs(dtype=BF):
    return {"x": torch.zeros(2, 10, 48, dtype=dtype), "weight": torch.zeros(48, 4)}


@pytest.mark.parametrize("kw,exc", [
    ({"weight": torch.zeros(40, 4)}, ValueError),
    ({"weight": torch.zeros(48, 4, dtype=BF)}, TypeError),
    ({"bias": torch.zeros(47)}, ValueError),
    ({"out": torch.zeros(2, 10, 48, dtype=F32)}, TypeError),
    ({"out": torch.zeros(2, 11, 48, dtype=BF)}, ValueError),
    ({"conv_state_in": torch.zeros(2, 3, 48, dtype=F32)}, TypeError),
    ({"conv_state_out": torch.zeros(1, 3, 48, dtype=BF)}, ValueError),
    ({"conv_state_in": torch.zeros(2, 4, 48, dtype=BF)}, ValueError),
])
def test_conv_bad_tensor_raises(kw, exc):
    t = conv_inputs()
    t.update(kw)
    with pytest.raises(exc):
        ssd.ssd_conv1d_silu(t.pop("x"), t.pop("weight"), **t)


def test_conv_good_cpu_tensors_refused_as_host_memory():
    with pytest.raises(ValueError, match="GPU"):
        ssd.ssd_conv1d_silu(**conv_inputs(),
                            conv_state_out=torch.zeros(2, 3, 48, dtype=BF))


def decode_inputs(batch=3, H=4, G=2, dtype=BF, conv=True):
    CD = H * 64 + 2 * G * 128
    t = {"xBC": torch.zeros(batch, CD, dtype=dtype), "dt": torch.zeros(batch, H, dtype=dtype),
         "A": torch.zeros(H), "ssm_state": torch.zeros(batch, H, 64, 128), "nheads": H, "ngroups": G,
         "dt_bias": torch.zeros(H), "D": torch.zeros(H)}
    if conv:
        t["conv_state"] = torch.zeros(batch, 3, CD, dtype=dtype)
        t["conv_weight"] = torch.zeros(CD, 4)
    return t


def call_decode(t):
    t = dict(t)
    return ssd.ssd_decode_step(t.pop("xBC"), t.pop("dt"), t.pop("A"), t.pop("ssm_state"), **t)


@pytest.mark.parametrize("key,bad,exc", [
    ("dt", torch.zeros(3, 4, dtype=F32), TypeError),
    ("xBC", torch.zeros(3, 100, dtype=BF), ValueError),
    ("ssm_state", torch.zeros(3, 4, 64, 128, dtype=BF), TypeError),
    ("ssm_state", torch.zeros(2, 4, 64, 128), ValueError),
    ("conv_state", torch.zeros(3, 3, 768, dtype=F32), TypeError),
    ("conv_state", torch.zeros(2, 3, 768, dtype=BF), ValueError),
    ("conv_weight", torch.zeros(700, 4), ValueError),
    ("conv_weight", None, ValueError),
    ("A", torch.zeros(2), ValueError),
    ("y", torch.zeros(3, 4, 64, dtype=F32), TypeError),
    ("y", torch.zeros(3, 2, 64, dtype=BF), ValueError),
])
def test_decode_bad_tensor_raises(key, bad, exc):
    t = decode_inputs()
    t[key] = bad
    with pytest.raises(exc):
        call_decode(t)


def test_decode_good_cpu_tensors_refused_as_host_memory():
    for conv in (True, False):
        with pytest.raises(ValueError, match="GPU"):
            call_decode(decode_inputs(conv=conv))


def test_linear_single_row_strided_view_raises():
    """A one-row x whose last dim is not unit-stride is refused (the kernel
    reads K contiguous elements per row)."""
    x = torch.zeros(1, 2 * 64, dtype=BF)[:, ::2]
    w = torch.zeros(32, 64, dtype=BF)
    with pytest.raises(ValueError, match="unit-stride"):
        ssd.ssd_linear(x, w)


def test_mimo_empty_batch_raises_cleanly():
    """batch 0 reaches the ordinary checks (here: host tensors) instead of
    indexing a missing row."""
    H, G, P, N, R = 4, 2, 64, 128, 2
    with pytest.raises(ValueError):
        ssd.ssd_decode_step_mimo(torch.zeros(0, H, P, R, dtype=BF), torch.zeros(0, G, N, R, dtype=BF),
                                 torch.zeros(0, G, N, R, dtype=BF), torch.zeros(0, H, dtype=BF), torch.zeros(H),
                                 torch.zeros(0, H, P, N))
