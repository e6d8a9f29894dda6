"""Thin ctypes binding of libssd.so (include/ssd.h), same entry-point names.

Argument marshalling only: every step of the layer runs in the HIP kernels
of libssd.so.  Tensors are torch CUDA (HIP) tensors; PyTorch supplies device
memory and the current stream, nothing else.  There is no CPU fallback: if
the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libssd.so")

SSD_DTYPE_F32 = 0
SSD_DTYPE_BF16 = 1
STATUS = {0: "SSD_OK", 1: "SSD_ERR_INVALID_ARG", 2: "SSD_ERR_UNSUPPORTED",
          3: "SSD_ERR_WORKSPACE_TOO_SMALL", 4: "SSD_ERR_MISALIGNED", 5: "SSD_ERR_HIP"}

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class SsdConvArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("dtype", _i32),
                ("batch", _i32), ("seqlen", _i32), ("channels", _i32), ("width", _i32),
                ("x", _vp), ("x_stride_batch", _i64), ("x_stride_token", _i64),
                ("out", _vp), ("out_stride_batch", _i64), ("out_stride_token", _i64),
                ("weight", _vp), ("bias", _vp), ("seq_idx", _vp), ("num_seqs", _i32),
                ("conv_state_in", _vp), ("conv_state_out", _vp)]


class SsdScanArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("dtype", _i32),
                ("batch", _i32), ("seqlen", _i32), ("nheads", _i32), ("headdim", _i32),
                ("dstate", _i32), ("ngroups", _i32), ("chunk_size", _i32), ("seg_chunks", _i32),
                ("x", _vp), ("x_stride_batch", _i64), ("x_stride_token", _i64),
                ("B", _vp), ("B_stride_batch", _i64), ("B_stride_token", _i64),
                ("C", _vp), ("C_stride_batch", _i64), ("C_stride_token", _i64),
                ("dt", _vp), ("dt_stride_batch", _i64), ("dt_stride_token", _i64),
                ("dt_bias", _vp), ("A", _vp), ("D", _vp), ("seq_idx", _vp), ("num_seqs", _i32),
                ("initial_state", _vp), ("final_state", _vp),
                ("y", _vp), ("y_stride_batch", _i64), ("y_stride_token", _i64)]


class SsdDecodeArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("dtype", _i32),
                ("batch", _i32), ("nheads", _i32), ("headdim", _i32), ("dstate", _i32),
                ("ngroups", _i32), ("conv_width", _i32),
                ("xBC", _vp), ("xBC_stride_batch", _i64), ("dt", _vp), ("dt_stride_batch", _i64),
                ("dt_bias", _vp), ("A", _vp), ("D", _vp), ("conv_weight", _vp), ("conv_bias", _vp),
                ("conv_state", _vp), ("ssm_state", _vp), ("y", _vp), ("y_stride_batch", _i64)]


EXPORTS = ["ssd_conv1d_silu", "ssd_chunk_scan_workspace_size", "ssd_chunk_scan_fwd",
           "ssd_decode_step", "ssd_last_error", "ssd_version"]

_lib = None


def load_library(path: str = LIB_PATH):
    """Load libssd.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; "
                           "g.build()'` (the HIP path has no fallback)")
    lib = ctypes.CDLL(path)
    lib.ssd_conv1d_silu.argtypes = [ctypes.POINTER(SsdConvArgs), _vp]
    lib.ssd_conv1d_silu.restype = ctypes.c_int
    lib.ssd_chunk_scan_workspace_size.argtypes = [ctypes.POINTER(SsdScanArgs)]
    lib.ssd_chunk_scan_workspace_size.restype = ctypes.c_size_t
    lib.ssd_chunk_scan_fwd.argtypes = [ctypes.POINTER(SsdScanArgs), _vp, ctypes.c_size_t, _vp]
    lib.ssd_chunk_scan_fwd.restype = ctypes.c_int
    lib.ssd_decode_step.argtypes = [ctypes.POINTER(SsdDecodeArgs), _vp]
    lib.ssd_decode_step.restype = ctypes.c_int
    lib.ssd_last_error.argtypes = []
    lib.ssd_last_error.restype = ctypes.c_char_p
    lib.ssd_version.argtypes = []
    lib.ssd_version.restype = ctypes.c_int
    _lib = lib
    return lib


class SsdError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


def _check(rc: int):
    if rc != 0:
        raise SsdError(rc, load_library().ssd_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SSD_DTYPE_BF16
    if t.dtype == torch.float32:
        return SSD_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _f32(t: Optional[torch.Tensor], name: str):
    if t is None:
        return None
    if t.dtype != torch.float32 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous float32 tensor")
    return t


# ---------------------------------------------------------------------------
def ssd_conv1d_silu(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
                    seq_idx: Optional[torch.Tensor] = None, num_seqs: Optional[int] = None,
                    conv_state_in: Optional[torch.Tensor] = None,
                    conv_state_out: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Depthwise causal conv1d (width = weight.shape[1]) + SiLU.  x: (batch, L, channels)."""
    lib = load_library()
    batch, L, CH = x.shape
    if x.stride(2) != 1:
        raise ValueError("x must have unit channel stride")
    if out is None:
        out = torch.empty((batch, L, CH), dtype=x.dtype, device=x.device)
    a = SsdConvArgs()
    a.struct_size = ctypes.sizeof(SsdConvArgs)
    a.dtype = _dtype_code(x)
    a.batch, a.seqlen, a.channels, a.width = batch, L, CH, weight.shape[1]
    a.x, a.x_stride_batch, a.x_stride_token = _ptr(x), x.stride(0), x.stride(1)
    a.out, a.out_stride_batch, a.out_stride_token = _ptr(out), out.stride(0), out.stride(1)
    a.weight = _ptr(_f32(weight, "weight"))
    a.bias = _ptr(_f32(bias, "bias"))
    a.seq_idx = _ptr(seq_idx)
    a.num_seqs = int(num_seqs or 0)
    a.conv_state_in = _ptr(conv_state_in)
    a.conv_state_out = _ptr(conv_state_out)
    _check(lib.ssd_conv1d_silu(ctypes.byref(a), _stream(stream)))
    return out


def _scan_args(x, dt, A, B, C, dt_bias, D, seq_idx, num_seqs, initial_state, final_state, y,
               chunk_size, seg_chunks) -> SsdScanArgs:
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if L > 0:
        for t, name, inner in ((x, "x", P), (y, "y", P), (B, "B", N), (C, "C", N)):
            if t is not None and (t.stride(3) != 1 or t.stride(2) != inner):
                raise ValueError(f"{name}: the last two dims must be packed (strides ({inner}, 1))")
        if dt.stride(2) != 1:
            raise ValueError("dt: head dim must be unit-stride")
    a = SsdScanArgs()
    a.struct_size = ctypes.sizeof(SsdScanArgs)
    a.dtype = _dtype_code(x)
    a.batch, a.seqlen, a.nheads, a.headdim = batch, L, H, P
    a.dstate, a.ngroups, a.chunk_size, a.seg_chunks = N, G, chunk_size, seg_chunks
    a.x, a.x_stride_batch, a.x_stride_token = _ptr(x), x.stride(0), x.stride(1)
    a.B, a.B_stride_batch, a.B_stride_token = _ptr(B), B.stride(0), B.stride(1)
    a.C, a.C_stride_batch, a.C_stride_token = _ptr(C), C.stride(0), C.stride(1)
    a.dt, a.dt_stride_batch, a.dt_stride_token = _ptr(dt), dt.stride(0), dt.stride(1)
    a.dt_bias = _ptr(_f32(dt_bias, "dt_bias"))
    a.A = _ptr(_f32(A, "A"))
    a.D = _ptr(_f32(D, "D"))
    a.seq_idx = _ptr(seq_idx)
    a.num_seqs = int(num_seqs or 0)
    a.initial_state = _ptr(_f32(initial_state, "initial_state"))
    a.final_state = _ptr(_f32(final_state, "final_state"))
    if y is not None:
        a.y, a.y_stride_batch, a.y_stride_token = _ptr(y), y.stride(0), y.stride(1)
    return a


def ssd_chunk_scan_workspace_size(x, dt, A, B, C, seq_idx=None, num_seqs=None, chunk_size=128,
                                  seg_chunks=0) -> int:
    lib = load_library()
    a = _scan_args(x, dt, A, B, C, None, None, seq_idx, num_seqs, None, None, x, chunk_size,
                   seg_chunks)
    n = lib.ssd_chunk_scan_workspace_size(ctypes.byref(a))
    if n == ctypes.c_size_t(-1).value:
        raise SsdError(1, lib.ssd_last_error().decode())
    return int(n)


def ssd_chunk_scan_fwd(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                       C: torch.Tensor, dt_bias: Optional[torch.Tensor] = None,
                       D: Optional[torch.Tensor] = None, seq_idx: Optional[torch.Tensor] = None,
                       num_seqs: Optional[int] = None,
                       initial_state: Optional[torch.Tensor] = None,
                       final_state: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                       chunk_size: int = 128, seg_chunks: int = 0,
                       workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Chunked SSD prefill.  x (batch,L,H,P), dt (batch,L,H) raw, B/C (batch,L,G,N).

    Writes y (allocated if not given) and, if `final_state` is given, the final
    states into it.  Returns y.
    """
    lib = load_library()
    if y is None:
        y = torch.empty(x.shape, dtype=x.dtype, device=x.device)
    a = _scan_args(x, dt, A, B, C, dt_bias, D, seq_idx, num_seqs, initial_state, final_state, y,
                   chunk_size, seg_chunks)
    need = lib.ssd_chunk_scan_workspace_size(ctypes.byref(a))
    if need == ctypes.c_size_t(-1).value:
        raise SsdError(1, lib.ssd_last_error().decode())
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.ssd_chunk_scan_fwd(ctypes.byref(a), _ptr(workspace), ws_bytes, _stream(stream)))
    return y


def ssd_decode_step(xBC: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, ssm_state: torch.Tensor,
                    nheads: int, ngroups: int, headdim: int = 64, dstate: int = 128,
                    dt_bias: Optional[torch.Tensor] = None, D: Optional[torch.Tensor] = None,
                    conv_state: Optional[torch.Tensor] = None,
                    conv_weight: Optional[torch.Tensor] = None,
                    conv_bias: Optional[torch.Tensor] = None,
                    y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One decode token; updates ssm_state (and conv_state) in place.  Returns y (batch,H,P)."""
    lib = load_library()
    batch = xBC.shape[0]
    if xBC.stride(1) != 1 or dt.stride(1) != 1:
        raise ValueError("xBC and dt rows must be contiguous")
    if not ssm_state.is_contiguous() or ssm_state.dtype != torch.float32:
        raise TypeError("ssm_state must be a contiguous float32 tensor")
    if conv_state is not None and not conv_state.is_contiguous():
        raise TypeError("conv_state must be contiguous")
    if y is None:
        y = torch.empty((batch, nheads, headdim), dtype=xBC.dtype, device=xBC.device)
    if y.stride(2) != 1 or y.stride(1) != headdim:
        raise ValueError("y must have packed (H, P) rows")
    a = SsdDecodeArgs()
    a.struct_size = ctypes.sizeof(SsdDecodeArgs)
    a.dtype = _dtype_code(xBC)
    a.batch, a.nheads, a.headdim, a.dstate, a.ngroups = batch, nheads, headdim, dstate, ngroups
    a.conv_width = conv_weight.shape[1] if conv_weight is not None else 0
    a.xBC, a.xBC_stride_batch = _ptr(xBC), xBC.stride(0)
    a.dt, a.dt_stride_batch = _ptr(dt), dt.stride(0)
    a.dt_bias = _ptr(_f32(dt_bias, "dt_bias"))
    a.A = _ptr(_f32(A, "A"))
    a.D = _ptr(_f32(D, "D"))
    a.conv_weight = _ptr(_f32(conv_weight, "conv_weight"))
    a.conv_bias = _ptr(_f32(conv_bias, "conv_bias"))
    a.conv_state = _ptr(conv_state)
    a.ssm_state = _ptr(ssm_state)
    a.y, a.y_stride_batch = _ptr(y), y.stride(0)
    _check(lib.ssd_decode_step(ctypes.byref(a), _stream(stream)))
    return y
