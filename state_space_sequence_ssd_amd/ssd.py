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


_SCAN_ARGS_SIZE = ctypes.sizeof(SsdScanArgs)


class SsdLinearArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("dtype", _i32), ("M", _i32), ("N", _i32), ("K", _i32),
                ("x", _vp), ("x_stride", _i64), ("w", _vp), ("w_stride", _i64), ("y", _vp), ("y_stride", _i64)]


class SsdConvScanArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("dtype", _i32),
                ("batch", _i32), ("seqlen", _i32), ("nheads", _i32), ("headdim", _i32),
                ("dstate", _i32), ("ngroups", _i32), ("chunk_size", _i32), ("seg_chunks", _i32),
                ("conv_width", _i32),
                ("xBC", _vp), ("xBC_stride_batch", _i64), ("xBC_stride_token", _i64),
                ("conv_weight", _vp), ("conv_bias", _vp),
                ("dt", _vp), ("dt_stride_batch", _i64), ("dt_stride_token", _i64),
                ("dt_bias", _vp), ("A", _vp), ("D", _vp), ("seq_idx", _vp), ("num_seqs", _i32),
                ("conv_state_in", _vp), ("conv_state_out", _vp),
                ("initial_state", _vp), ("final_state", _vp),
                ("y", _vp), ("y_stride_batch", _i64), ("y_stride_token", _i64)]


class SsdDecodeArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("dtype", _i32),
                ("batch", _i32), ("nheads", _i32), ("headdim", _i32), ("dstate", _i32),
                ("ngroups", _i32), ("conv_width", _i32),
                ("xBC", _vp), ("xBC_stride_batch", _i64), ("dt", _vp), ("dt_stride_batch", _i64),
                ("dt_bias", _vp), ("A", _vp), ("D", _vp), ("conv_weight", _vp), ("conv_bias", _vp),
                ("conv_state", _vp), ("ssm_state", _vp), ("y", _vp), ("y_stride_batch", _i64)]


class SsdNormArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("dtype", _i32),
                ("batch", _i32), ("seqlen", _i32), ("channels", _i32), ("group_size", _i32),
                ("norm_before_gate", _i32), ("eps", ctypes.c_float),
                ("y", _vp), ("y_stride_batch", _i64), ("y_stride_token", _i64),
                ("z", _vp), ("z_stride_batch", _i64), ("z_stride_token", _i64),
                ("weight", _vp),
                ("out", _vp), ("out_stride_batch", _i64), ("out_stride_token", _i64)]


class SsdMimoDecodeArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("dtype", _i32),
                ("batch", _i32), ("nheads", _i32), ("headdim", _i32), ("dstate", _i32),
                ("ngroups", _i32), ("rank", _i32), ("trapezoid", _i32),
                ("x", _vp), ("x_stride_batch", _i64), ("B", _vp), ("B_stride_batch", _i64),
                ("C", _vp), ("C_stride_batch", _i64), ("dt", _vp), ("dt_stride_batch", _i64),
                ("lam", _vp), ("lam_stride_batch", _i64),
                ("dt_bias", _vp), ("A", _vp), ("D", _vp), ("ssm_state", _vp),
                ("prev_x", _vp), ("prev_B", _vp), ("y", _vp), ("y_stride_batch", _i64)]


class SsdScanBwdArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("dtype", _i32),
                ("batch", _i32), ("seqlen", _i32), ("nheads", _i32), ("headdim", _i32),
                ("dstate", _i32), ("ngroups", _i32),
                ("x", _vp), ("dt", _vp), ("B", _vp), ("C", _vp), ("dy", _vp),
                ("dt_bias", _vp), ("A", _vp), ("D", _vp), ("initial_state", _vp), ("d_final_state", _vp),
                ("dx", _vp), ("ddt", _vp), ("dB", _vp), ("dC", _vp),
                ("d_dt_bias", _vp), ("dA", _vp), ("dD", _vp), ("d_initial_state", _vp)]


EXPORTS = ["ssd_conv1d_silu", "ssd_chunk_scan_workspace_size", "ssd_chunk_scan_fwd",
           "ssd_chunk_scan_fwd_noalloc", "ssd_conv_scan_workspace_size", "ssd_conv_scan_fwd", "ssd_linear", "ssd_chunk_scan_bwd_workspace_size", "ssd_chunk_scan_bwd",
           "ssd_gated_rmsnorm", "ssd_decode_step", "ssd_decode_step_mimo", "ssd_last_error", "ssd_version"]
NOALLOC_SCRATCH_BYTES = 96 * 1024 * 1024   # SSD_NOALLOC_SCRATCH_BYTES

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
    lib.ssd_chunk_scan_fwd_noalloc.argtypes = [ctypes.POINTER(SsdScanArgs), _vp]
    lib.ssd_chunk_scan_fwd_noalloc.restype = ctypes.c_int
    lib.ssd_conv_scan_workspace_size.argtypes = [ctypes.POINTER(SsdConvScanArgs)]
    lib.ssd_conv_scan_workspace_size.restype = ctypes.c_size_t
    lib.ssd_conv_scan_fwd.argtypes = [ctypes.POINTER(SsdConvScanArgs), _vp, ctypes.c_size_t, _vp]
    lib.ssd_conv_scan_fwd.restype = ctypes.c_int
    lib.ssd_linear.argtypes = [ctypes.POINTER(SsdLinearArgs), _vp]
    lib.ssd_linear.restype = ctypes.c_int
    lib.ssd_gated_rmsnorm.argtypes = [ctypes.POINTER(SsdNormArgs), _vp]
    lib.ssd_gated_rmsnorm.restype = ctypes.c_int
    lib.ssd_chunk_scan_bwd_workspace_size.argtypes = [ctypes.POINTER(SsdScanBwdArgs)]
    lib.ssd_chunk_scan_bwd_workspace_size.restype = ctypes.c_size_t
    lib.ssd_chunk_scan_bwd.argtypes = [ctypes.POINTER(SsdScanBwdArgs), _vp, ctypes.c_size_t, _vp]
    lib.ssd_chunk_scan_bwd.restype = ctypes.c_int
    lib.ssd_decode_step_mimo.argtypes = [ctypes.POINTER(SsdMimoDecodeArgs), _vp]
    lib.ssd_decode_step_mimo.restype = ctypes.c_int
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


def _empty(stream, *shape_args, **kw) -> torch.Tensor:
    """torch.empty on the stream the call launches on (the current one when
    none is given): the caching allocator then ties the block to that stream,
    so a temporary freed when the call returns is not handed to another
    stream while this one's kernels still use it."""
    if stream is None:
        return torch.empty(*shape_args, **kw)
    with torch.cuda.stream(stream):
        return torch.empty(*shape_args, **kw)


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _f32(t: Optional[torch.Tensor], name: str, numel: Optional[int] = None,
         shape: Optional[tuple] = None):
    """A contiguous float32 tensor (or None), of `numel` elements / `shape` if given."""
    if t is None:
        return None
    if t.dtype != torch.float32 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous float32 tensor")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements (got {t.numel()})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t


def _same_dtype(ref: torch.Tensor, **tensors):
    """Every given tensor has ref's dtype (the one dtype code the ABI carries)."""
    for name, t in tensors.items():
        if t is not None and t.dtype != ref.dtype:
            raise TypeError(f"{name} is {t.dtype}, but the call's tensors are {ref.dtype}")


def _shape(t: Optional[torch.Tensor], name: str, shape: tuple):
    if t is not None and t.shape != shape:
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def _seq_idx(seq_idx: Optional[torch.Tensor], L: int, num_seqs: Optional[int]):
    if seq_idx is None:
        return
    if seq_idx.dtype != torch.int32 or not seq_idx.is_contiguous() or tuple(seq_idx.shape) != (L,):
        raise TypeError(f"seq_idx must be a contiguous int32 tensor of shape ({L},)")
    if num_seqs is None or int(num_seqs) < 1:
        raise ValueError("num_seqs (>= 1) is required with seq_idx")


def _on_gpu(ref: torch.Tensor, **tensors):
    """Every tensor lives on ref's GPU: the library dereferences device pointers
    only.  Checked last, after every dtype and shape check."""
    if not ref.is_cuda:
        raise ValueError("tensors must be on a GPU (the HIP path has no CPU fallback)")
    for name, t in tensors.items():
        if t is not None and (not t.is_cuda or t.device != ref.device):
            raise ValueError(f"{name} must be on {ref.device} (got {t.device})")


# ---------------------------------------------------------------------------
def ssd_conv1d_silu(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
                    seq_idx: Optional[torch.Tensor] = None, num_seqs: Optional[int] = None,
                    conv_state_in: Optional[torch.Tensor] = None,
                    conv_state_out: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Depthwise causal conv1d (width = weight.shape[1]) + SiLU.  x: (batch, L, channels)."""
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be (batch, L, channels)")
    batch, L, CH = x.shape
    if x.stride(2) != 1:
        raise ValueError("x must have unit channel stride")
    _dtype_code(x)
    if weight.dim() != 2 or weight.shape[0] != CH:
        raise ValueError(f"weight must be (channels={CH}, width)")
    K = weight.shape[1]
    _f32(weight, "weight")
    _f32(bias, "bias", numel=CH)
    _seq_idx(seq_idx, L, num_seqs)
    rows = int(num_seqs) if seq_idx is not None else batch
    _same_dtype(x, out=out, conv_state_in=conv_state_in, conv_state_out=conv_state_out)
    _shape(out, "out", (batch, L, CH))
    for name, t in (("conv_state_in", conv_state_in), ("conv_state_out", conv_state_out)):
        _shape(t, name, (rows, K - 1, CH))
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if out is not None and out.stride(2) != 1:
        raise ValueError("out must have unit channel stride")
    _on_gpu(x, out=out, weight=weight, bias=bias, seq_idx=seq_idx, conv_state_in=conv_state_in,
            conv_state_out=conv_state_out)
    if out is None:
        out = _empty(stream, (batch, L, CH), dtype=x.dtype, device=x.device)
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
    # Per-call host cost matters for short sequences (the kernel then runs
    # for tens of microseconds): every tensor's metadata is read once and the
    # struct is built in one constructor call.
    if x.dim() != 4 or B.dim() != 4 or C.dim() != 4 or dt.dim() != 3:
        raise ValueError("x (batch,L,H,P), B/C (batch,L,G,N) and dt (batch,L,H) expected")
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    code = _dtype_code(x)
    _same_dtype(x, dt=dt, B=B, C=C, y=y)
    _shape(B, "B", (batch, L, G, N))
    _shape(C, "C", (batch, L, G, N))
    _shape(dt, "dt", (batch, L, H))
    _shape(y, "y", (batch, L, H, P))
    _f32(A, "A", numel=H)
    _f32(dt_bias, "dt_bias", numel=H)
    _f32(D, "D", numel=H)
    _seq_idx(seq_idx, L, num_seqs)
    rows = int(num_seqs) if seq_idx is not None else batch
    _f32(initial_state, "initial_state", shape=(rows, H, P, N))
    _f32(final_state, "final_state", shape=(rows, H, P, N))
    _on_gpu(x, dt=dt, A=A, B=B, C=C, y=y, dt_bias=dt_bias, D=D, seq_idx=seq_idx,
            initial_state=initial_state, final_state=final_state)
    xs, bs, cs, ds = x.stride(), B.stride(), C.stride(), dt.stride()
    ys = y.stride() if y is not None else (0, 0, P, 1)
    if L > 0:
        for st, name, inner in ((xs, "x", P), (ys, "y", P), (bs, "B", N), (cs, "C", N)):
            if st[3] != 1 or st[2] != inner:
                raise ValueError(f"{name}: the last two dims must be packed (strides ({inner}, 1))")
        if ds[2] != 1:
            raise ValueError("dt: head dim must be unit-stride")
    return SsdScanArgs(_SCAN_ARGS_SIZE, code, batch, L, H, P, N, G, chunk_size, seg_chunks,
                       x.data_ptr(), xs[0], xs[1], B.data_ptr(), bs[0], bs[1],
                       C.data_ptr(), cs[0], cs[1], dt.data_ptr(), ds[0], ds[1],
                       _ptr(dt_bias), A.data_ptr(), _ptr(D), _ptr(seq_idx), int(num_seqs or 0),
                       _ptr(initial_state), _ptr(final_state),
                       _ptr(y), ys[0], ys[1])


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
        y = _empty(stream, x.shape, dtype=x.dtype, device=x.device)
    a = _scan_args(x, dt, A, B, C, dt_bias, D, seq_idx, num_seqs, initial_state, final_state, y,
                   chunk_size, seg_chunks)
    if workspace is None:
        # (a caller workspace is checked by the library: too small is an error)
        need = lib.ssd_chunk_scan_workspace_size(ctypes.byref(a))
        if need == ctypes.c_size_t(-1).value:
            raise SsdError(1, lib.ssd_last_error().decode())
        if need > 0:
            workspace = _empty(stream, need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.ssd_chunk_scan_fwd(ctypes.byref(a), _ptr(workspace), ws_bytes, _stream(stream)))
    return y


def ssd_chunk_scan_fwd_noalloc(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                               C: torch.Tensor, y: torch.Tensor, dt_bias: Optional[torch.Tensor] = None,
                               D: Optional[torch.Tensor] = None, seq_idx: Optional[torch.Tensor] = None,
                               num_seqs: Optional[int] = None,
                               initial_state: Optional[torch.Tensor] = None,
                               final_state: Optional[torch.Tensor] = None,
                               chunk_size: int = 128, seg_chunks: int = 0, stream=None) -> torch.Tensor:
    """ssd_chunk_scan_fwd with the library's own workspace array: nothing is
    allocated (y is required).  Calls that overlap on one GPU race on that
    array; the current device must be the stream's.  Returns y."""
    lib = load_library()
    if y is None:
        raise ValueError("y is required (this entry point allocates nothing)")
    a = _scan_args(x, dt, A, B, C, dt_bias, D, seq_idx, num_seqs, initial_state, final_state, y,
                   chunk_size, seg_chunks)
    _check(lib.ssd_chunk_scan_fwd_noalloc(ctypes.byref(a), _stream(stream)))
    return y


def _conv_scan_args(xBC, conv_weight, dt, A, nheads, ngroups, headdim, dstate, conv_bias, dt_bias, D,
                    seq_idx, num_seqs, conv_state_in, conv_state_out, initial_state, final_state, y,
                    chunk_size, seg_chunks) -> SsdConvScanArgs:
    if xBC.dim() != 3 or dt.dim() != 3:
        raise ValueError("xBC (batch, L, conv_dim) and dt (batch, L, nheads) expected")
    batch, L, CH = xBC.shape
    H, G, P, N = int(nheads), int(ngroups), int(headdim), int(dstate)
    if CH != H * P + 2 * G * N:
        raise ValueError(f"xBC has {CH} channels; nheads*headdim + 2*ngroups*dstate = {H * P + 2 * G * N}")
    code = _dtype_code(xBC)
    _same_dtype(xBC, dt=dt, y=y, conv_state_in=conv_state_in, conv_state_out=conv_state_out)
    if conv_weight.dim() != 2 or conv_weight.shape[0] != CH:
        raise ValueError(f"conv_weight must be (conv_dim={CH}, width)")
    K = conv_weight.shape[1]
    _f32(conv_weight, "conv_weight")
    _f32(conv_bias, "conv_bias", numel=CH)
    _shape(dt, "dt", (batch, L, H))
    _shape(y, "y", (batch, L, H, P))
    _f32(A, "A", numel=H)
    _f32(dt_bias, "dt_bias", numel=H)
    _f32(D, "D", numel=H)
    _seq_idx(seq_idx, L, num_seqs)
    rows = int(num_seqs) if seq_idx is not None else batch
    for name, t in (("conv_state_in", conv_state_in), ("conv_state_out", conv_state_out)):
        _shape(t, name, (rows, K - 1, CH))
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    _f32(initial_state, "initial_state", shape=(rows, H, P, N))
    _f32(final_state, "final_state", shape=(rows, H, P, N))
    _on_gpu(xBC, conv_weight=conv_weight, conv_bias=conv_bias, dt=dt, A=A, y=y, dt_bias=dt_bias, D=D,
            seq_idx=seq_idx, conv_state_in=conv_state_in, conv_state_out=conv_state_out,
            initial_state=initial_state, final_state=final_state)
    xs, ds = xBC.stride(), dt.stride()
    ys = y.stride() if y is not None else (0, 0, P, 1)
    if L > 0:
        if xs[2] != 1:
            raise ValueError("xBC must have unit channel stride")
        if ys[3] != 1 or ys[2] != P:
            raise ValueError(f"y: the last two dims must be packed (strides ({P}, 1))")
        if ds[2] != 1:
            raise ValueError("dt: head dim must be unit-stride")
    return SsdConvScanArgs(ctypes.sizeof(SsdConvScanArgs), code, batch, L, H, P, N, G, chunk_size, seg_chunks, K,
                           xBC.data_ptr(), xs[0], xs[1], conv_weight.data_ptr(), _ptr(conv_bias),
                           dt.data_ptr(), ds[0], ds[1], _ptr(dt_bias), A.data_ptr(), _ptr(D),
                           _ptr(seq_idx), int(num_seqs or 0), _ptr(conv_state_in), _ptr(conv_state_out),
                           _ptr(initial_state), _ptr(final_state), _ptr(y), ys[0], ys[1])


def ssd_conv_scan_workspace_size(xBC, conv_weight, dt, A, nheads, ngroups, headdim=64, dstate=128,
                                 seq_idx=None, num_seqs=None, chunk_size=128, seg_chunks=0) -> int:
    lib = load_library()
    y = torch.empty((xBC.shape[0], xBC.shape[1], nheads, headdim), dtype=xBC.dtype, device=xBC.device)
    a = _conv_scan_args(xBC, conv_weight, dt, A, nheads, ngroups, headdim, dstate, None, None, None,
                        seq_idx, num_seqs, None, None, None, None, y, chunk_size, seg_chunks)
    n = lib.ssd_conv_scan_workspace_size(ctypes.byref(a))
    if n == ctypes.c_size_t(-1).value:
        raise SsdError(1, lib.ssd_last_error().decode())
    return int(n)


def ssd_conv_scan_fwd(xBC: torch.Tensor, conv_weight: torch.Tensor, dt: torch.Tensor, A: torch.Tensor,
                      nheads: int, ngroups: int, headdim: int = 64, dstate: int = 128,
                      conv_bias: Optional[torch.Tensor] = None, dt_bias: Optional[torch.Tensor] = None,
                      D: Optional[torch.Tensor] = None, seq_idx: Optional[torch.Tensor] = None,
                      num_seqs: Optional[int] = None, conv_state_in: Optional[torch.Tensor] = None,
                      conv_state_out: Optional[torch.Tensor] = None,
                      initial_state: Optional[torch.Tensor] = None,
                      final_state: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                      chunk_size: int = 128, seg_chunks: int = 0,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """conv1d(4) + SiLU of xBC (batch, L, nheads*headdim + 2*ngroups*dstate; columns
    x | B | C) and the chunked scan of its output, in one call (the x channels'
    conv runs inside the bf16 scan kernel).  Returns y (batch, L, nheads, headdim)."""
    lib = load_library()
    if y is None:
        y = _empty(stream, (xBC.shape[0], xBC.shape[1], nheads, headdim), dtype=xBC.dtype, device=xBC.device)
    a = _conv_scan_args(xBC, conv_weight, dt, A, nheads, ngroups, headdim, dstate, conv_bias, dt_bias, D,
                        seq_idx, num_seqs, conv_state_in, conv_state_out, initial_state, final_state, y,
                        chunk_size, seg_chunks)
    if workspace is None:
        need = lib.ssd_conv_scan_workspace_size(ctypes.byref(a))
        if need == ctypes.c_size_t(-1).value:
            raise SsdError(1, lib.ssd_last_error().decode())
        if need > 0:
            workspace = _empty(stream, need, dtype=torch.uint8, device=xBC.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.ssd_conv_scan_fwd(ctypes.byref(a), _ptr(workspace), ws_bytes, _stream(stream)))
    return y


def ssd_linear(x: torch.Tensor, w: torch.Tensor, y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y = x w^T (a projection of the mixer).  x (..., K) with packed leading dims
    and a unit-stride last dim, w (N, K) (a torch Linear weight), bf16.
    Returns y (..., N)."""
    lib = load_library()
    if x.dim() < 1 or w.dim() != 2:
        raise ValueError("x (..., K) and w (N, K) expected")
    K = x.shape[-1]
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError(f"w must be (N, K={K})")
    _dtype_code(x)
    _same_dtype(x, w=w, y=y)
    x2 = x.reshape(-1, K) if x.dim() != 2 else x
    if x2.data_ptr() != x.data_ptr():
        raise ValueError("x's leading dims must be packed (a view, not a copy)")
    M = x2.shape[0]
    if y is None:
        y = _empty(stream, (*x.shape[:-1], N), dtype=x.dtype, device=x.device)
    _shape(y, "y", (*x.shape[:-1], N))
    y2 = y.reshape(-1, N) if y.dim() != 2 else y
    if y2.data_ptr() != y.data_ptr():
        raise ValueError("y's leading dims must be packed")
    for t, name in ((x2, "x"), (w, "w"), (y2, "y")):
        if t.shape[1] > 1 and t.stride(1) != 1:
            raise ValueError(f"{name} must have a unit-stride last dim")
    _on_gpu(x, w=w, y=y)
    a = SsdLinearArgs(ctypes.sizeof(SsdLinearArgs), _dtype_code(x), M, N, K,
                      x2.data_ptr(), x2.stride(0), w.data_ptr(), w.stride(0), y2.data_ptr(), y2.stride(0))
    _check(lib.ssd_linear(ctypes.byref(a), _stream(stream)))
    return y


def mamba2_mixer_fwd(hidden: torch.Tensor, in_proj_w: torch.Tensor, conv_w: torch.Tensor,
                     dt_bias: torch.Tensor, A: torch.Tensor, D: torch.Tensor, norm_w: torch.Tensor,
                     out_proj_w: torch.Tensor, nheads: int, ngroups: int, headdim: int = 64,
                     dstate: int = 128, norm_group_size: Optional[int] = None, eps: float = 1e-5,
                     conv_bias: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The whole Mamba-2 mixer forward as a sequence of this library's calls:
    in_proj -> [z | xBC | dt] column views -> conv1d + SiLU fused into the
    chunked scan -> gated RMSNorm(y, z), norm after the gate -> out_proj.
    hidden (batch, L, d_model) bf16.  Only views and the calls' outputs are
    made here; every step is a libssd call.  Returns (batch, L, d_model)."""
    batch, L, _ = hidden.shape
    d_inner = nheads * headdim
    conv_dim = d_inner + 2 * ngroups * dstate
    d_in_proj = 2 * d_inner + 2 * ngroups * dstate + nheads
    if in_proj_w.shape[0] != d_in_proj:
        raise ValueError(f"in_proj_w must have {d_in_proj} rows (z, x, B, C, dt)")
    zxbcdt = ssd_linear(hidden, in_proj_w, stream=stream)
    z = zxbcdt[..., :d_inner]
    xBC = zxbcdt[..., d_inner:d_inner + conv_dim]
    dt = zxbcdt[..., d_inner + conv_dim:]
    y = ssd_conv_scan_fwd(xBC, conv_w, dt, A, nheads, ngroups, headdim, dstate, conv_bias=conv_bias,
                          dt_bias=dt_bias, D=D, final_state=final_state, workspace=workspace, stream=stream)
    gs = norm_group_size or d_inner // ngroups
    yn = ssd_gated_rmsnorm(y.flatten(2), norm_w, gs, z=z, eps=eps, stream=stream)
    return ssd_linear(yn, out_proj_w, stream=stream)


def _flat3(t: torch.Tensor, name: str):
    """(batch, seqlen, channels) view of a (batch, seqlen, ..., ) tensor whose
    trailing dims are packed; returns (tensor3, batch stride, token stride)."""
    if t.dim() < 3:
        raise ValueError(f"{name} must be (batch, seqlen, channels...)")
    inner = 1
    for d in range(t.dim() - 1, 1, -1):
        if t.stride(d) != inner:
            raise ValueError(f"{name}: the channel dims must be packed")
        inner *= t.shape[d]
    return t.shape[0], t.shape[1], inner, t.stride(0), t.stride(1)


def ssd_gated_rmsnorm(y: torch.Tensor, weight: torch.Tensor, group_size: int,
                      z: Optional[torch.Tensor] = None, norm_before_gate: bool = False,
                      eps: float = 1e-5, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Gated RMSNorm of the mixer output.  y, z (batch, seqlen, ...channels),
    weight (channels) fp32.  Returns out (y's shape, allocated if not given)."""
    lib = load_library()
    batch, L, CH, y_sb, y_st = _flat3(y, "y")
    _dtype_code(y)
    _same_dtype(y, z=z, out=out)
    _f32(weight, "weight", numel=CH)
    if z is not None:
        zb, zl, zc, z_sb, z_st = _flat3(z, "z")
        if (zb, zl, zc) != (batch, L, CH):
            raise ValueError(f"z must match y's (batch, seqlen, channels) = {(batch, L, CH)}")
    if out is not None:
        ob, ol, oc, o_sb, o_st = _flat3(out, "out")
        if (ob, ol, oc) != (batch, L, CH):
            raise ValueError(f"out must match y's (batch, seqlen, channels) = {(batch, L, CH)}")
    _on_gpu(y, z=z, weight=weight, out=out)
    if out is None:
        out = _empty(stream, y.shape, dtype=y.dtype, device=y.device)
        _, _, _, o_sb, o_st = _flat3(out, "out")
    a = SsdNormArgs()
    a.struct_size = ctypes.sizeof(SsdNormArgs)
    a.dtype = _dtype_code(y)
    a.batch, a.seqlen, a.channels, a.group_size = batch, L, CH, int(group_size)
    a.norm_before_gate, a.eps = int(bool(norm_before_gate)), float(eps)
    a.y, a.y_stride_batch, a.y_stride_token = _ptr(y), y_sb, y_st
    if z is not None:
        a.z, a.z_stride_batch, a.z_stride_token = _ptr(z), z_sb, z_st
    a.weight = _ptr(weight)
    a.out, a.out_stride_batch, a.out_stride_token = _ptr(out), o_sb, o_st
    _check(lib.ssd_gated_rmsnorm(ctypes.byref(a), _stream(stream)))
    return out


def ssd_decode_step(xBC: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, ssm_state: torch.Tensor,
                    nheads: int, ngroups: int, headdim: int = 64, dstate: int = 128,
                    dt_bias: Optional[torch.Tensor] = None, D: Optional[torch.Tensor] = None,
                    conv_state: Optional[torch.Tensor] = None,
                    conv_weight: Optional[torch.Tensor] = None,
                    conv_bias: Optional[torch.Tensor] = None,
                    y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One decode token; updates ssm_state (and conv_state) in place.  Returns y (batch,H,P)."""
    lib = load_library()
    if xBC.dim() != 2 or dt.dim() != 2:
        raise ValueError("xBC (batch, conv_dim) and dt (batch, nheads) expected")
    batch = xBC.shape[0]
    conv_dim = nheads * headdim + 2 * ngroups * dstate
    if xBC.stride(1) != 1 or dt.stride(1) != 1:
        raise ValueError("xBC and dt rows must be contiguous")
    _dtype_code(xBC)
    _same_dtype(xBC, dt=dt, conv_state=conv_state, y=y)
    _shape(xBC, "xBC", (batch, conv_dim))
    _shape(dt, "dt", (batch, nheads))
    _f32(ssm_state, "ssm_state", shape=(batch, nheads, headdim, dstate))
    _f32(A, "A", numel=nheads)
    _f32(dt_bias, "dt_bias", numel=nheads)
    _f32(D, "D", numel=nheads)
    if conv_state is not None:
        if conv_weight is None:
            raise ValueError("conv_state needs conv_weight")
        if conv_weight.dim() != 2 or conv_weight.shape[0] != conv_dim:
            raise ValueError(f"conv_weight must be (conv_dim={conv_dim}, width)")
        _f32(conv_weight, "conv_weight")
        _f32(conv_bias, "conv_bias", numel=conv_dim)
        _shape(conv_state, "conv_state", (batch, conv_weight.shape[1] - 1, conv_dim))
        if not conv_state.is_contiguous():
            raise TypeError("conv_state must be contiguous")
    _shape(y, "y", (batch, nheads, headdim))
    _on_gpu(xBC, dt=dt, A=A, ssm_state=ssm_state, dt_bias=dt_bias, D=D, conv_state=conv_state,
            conv_weight=conv_weight, conv_bias=conv_bias, y=y)
    if y is None:
        y = _empty(stream, (batch, nheads, headdim), dtype=xBC.dtype, device=xBC.device)
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


def ssd_decode_step_mimo(x: torch.Tensor, B: torch.Tensor, C: torch.Tensor, dt: torch.Tensor,
                         A: torch.Tensor, ssm_state: torch.Tensor, dt_bias: Optional[torch.Tensor] = None,
                         D: Optional[torch.Tensor] = None, trapezoid: bool = False,
                         lam: Optional[torch.Tensor] = None, prev_x: Optional[torch.Tensor] = None,
                         prev_B: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    """One MIMO decode token.  x (batch,H,P,R), B/C (batch,G,N,R), dt (and lam)
    (batch,H); ssm_state (batch,H,P,N) fp32 updated in place, and with the
    trapezoidal form prev_x / prev_B replaced by x / B.  Returns y (batch,H,P,R)."""
    lib = load_library()
    if x.dim() != 4 or B.dim() != 4 or C.dim() != 4 or dt.dim() != 2:
        raise ValueError("x (batch,H,P,R), B/C (batch,G,N,R) and dt (batch,H) expected")
    batch, H, P, R = x.shape
    G, N = B.shape[1], B.shape[2]
    _dtype_code(x)
    _same_dtype(x, B=B, C=C, dt=dt, lam=lam, prev_x=prev_x, prev_B=prev_B, y=y)
    _shape(B, "B", (batch, G, N, R))
    _shape(C, "C", (batch, G, N, R))
    _shape(dt, "dt", (batch, H))
    _shape(lam, "lam", (batch, H))
    _shape(y, "y", (batch, H, P, R))
    _shape(prev_x, "prev_x", (batch, H, P, R))
    _shape(prev_B, "prev_B", (batch, G, N, R))
    for name, t in (("x", x), ("B", B), ("C", C), ("y", y)):
        if t is not None and t.shape[0] > 0 and not t[0].is_contiguous():
            raise ValueError(f"{name}: each batch row must be contiguous")
    for name, t in (("dt", dt), ("lam", lam)):
        if t is not None and t.stride(1) != 1:
            raise ValueError(f"{name}: rows must be unit-stride")
    for name, t in (("prev_x", prev_x), ("prev_B", prev_B)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if trapezoid and (prev_x is None or prev_B is None):
        raise ValueError("the trapezoidal form needs prev_x and prev_B")
    _f32(ssm_state, "ssm_state", shape=(batch, H, P, N))
    _f32(A, "A", numel=H)
    _f32(dt_bias, "dt_bias", numel=H)
    _f32(D, "D", numel=H)
    _on_gpu(x, B=B, C=C, dt=dt, lam=lam, A=A, ssm_state=ssm_state, dt_bias=dt_bias, D=D,
            prev_x=prev_x, prev_B=prev_B, y=y)
    if y is None:
        y = _empty(stream, (batch, H, P, R), dtype=x.dtype, device=x.device)
    a = SsdMimoDecodeArgs()
    a.struct_size = ctypes.sizeof(SsdMimoDecodeArgs)
    a.dtype = _dtype_code(x)
    a.batch, a.nheads, a.headdim, a.dstate, a.ngroups, a.rank = batch, H, P, N, G, R
    a.trapezoid = int(bool(trapezoid))
    a.x, a.x_stride_batch = _ptr(x), x.stride(0)
    a.B, a.B_stride_batch = _ptr(B), B.stride(0)
    a.C, a.C_stride_batch = _ptr(C), C.stride(0)
    a.dt, a.dt_stride_batch = _ptr(dt), dt.stride(0)
    if lam is not None:
        a.lam, a.lam_stride_batch = _ptr(lam), lam.stride(0)
    a.dt_bias, a.A, a.D = _ptr(dt_bias), _ptr(A), _ptr(D)
    a.ssm_state = _ptr(ssm_state)
    a.prev_x, a.prev_B = _ptr(prev_x), _ptr(prev_B)
    a.y, a.y_stride_batch = _ptr(y), y.stride(0)
    _check(lib.ssd_decode_step_mimo(ctypes.byref(a), _stream(stream)))
    return y


def ssd_chunk_scan_bwd(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                       dy: torch.Tensor, dt_bias: Optional[torch.Tensor] = None,
                       D: Optional[torch.Tensor] = None, initial_state: Optional[torch.Tensor] = None,
                       d_final_state: Optional[torch.Tensor] = None, want_d_initial_state: bool = False,
                       workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Backward of ssd_chunk_scan_fwd (batch rows).  Contiguous x, dy
    (batch,L,H,P), dt (batch,L,H), B, C (batch,L,G,N).  Returns a dict of
    dx, ddt (w.r.t. dt raw), dB, dC (x's dtype), d_dt_bias, dA, dD (fp32) and
    d_initial_state (fp32, if asked)."""
    lib = load_library()
    if x.dim() != 4 or B.dim() != 4 or C.dim() != 4 or dt.dim() != 3:
        raise ValueError("x (batch,L,H,P), B/C (batch,L,G,N) and dt (batch,L,H) expected")
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    _dtype_code(x)
    _same_dtype(x, dt=dt, B=B, C=C, dy=dy)
    _shape(B, "B", (batch, L, G, N))
    _shape(C, "C", (batch, L, G, N))
    _shape(dt, "dt", (batch, L, H))
    _shape(dy, "dy", (batch, L, H, P))
    for name, t in (("x", x), ("dt", dt), ("B", B), ("C", C), ("dy", dy)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    _f32(A, "A", numel=H)
    _f32(dt_bias, "dt_bias", numel=H)
    _f32(D, "D", numel=H)
    _f32(initial_state, "initial_state", shape=(batch, H, P, N))
    _f32(d_final_state, "d_final_state", shape=(batch, H, P, N))
    _on_gpu(x, dt=dt, A=A, B=B, C=C, dy=dy, dt_bias=dt_bias, D=D, initial_state=initial_state,
            d_final_state=d_final_state, workspace=workspace)
    dev = x.device
    out = {"dx": _empty(stream, x.shape, dtype=x.dtype, device=dev),
           "ddt": _empty(stream, dt.shape, dtype=dt.dtype, device=dev),
           "dB": _empty(stream, B.shape, dtype=B.dtype, device=dev),
           "dC": _empty(stream, C.shape, dtype=C.dtype, device=dev), "d_dt_bias": _empty(stream, H, device=dev),
           "dA": _empty(stream, H, device=dev), "dD": _empty(stream, H, device=dev),
           "d_initial_state": _empty(stream, (batch, H, P, N), device=dev) if want_d_initial_state else None}
    a = SsdScanBwdArgs()
    a.struct_size = ctypes.sizeof(SsdScanBwdArgs)
    a.dtype = _dtype_code(x)
    a.batch, a.seqlen, a.nheads, a.headdim, a.dstate, a.ngroups = batch, L, H, P, N, G
    a.x, a.dt, a.B, a.C, a.dy = _ptr(x), _ptr(dt), _ptr(B), _ptr(C), _ptr(dy)
    a.dt_bias, a.A, a.D = _ptr(dt_bias), _ptr(A), _ptr(D)
    a.initial_state, a.d_final_state = _ptr(initial_state), _ptr(d_final_state)
    a.dx, a.ddt, a.dB, a.dC = _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dB"]), _ptr(out["dC"])
    a.d_dt_bias, a.dA, a.dD = _ptr(out["d_dt_bias"]), _ptr(out["dA"]), _ptr(out["dD"])
    a.d_initial_state = _ptr(out["d_initial_state"])
    need = lib.ssd_chunk_scan_bwd_workspace_size(ctypes.byref(a))
    if need == ctypes.c_size_t(-1).value:
        raise SsdError(1, lib.ssd_last_error().decode())
    if workspace is None:
        workspace = _empty(stream, max(need, 1), dtype=torch.uint8, device=dev)
    if workspace.dtype != torch.uint8 or workspace.numel() < need:
        raise ValueError(f"workspace must be a uint8 tensor of at least {need} bytes")
    _check(lib.ssd_chunk_scan_bwd(ctypes.byref(a), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out
