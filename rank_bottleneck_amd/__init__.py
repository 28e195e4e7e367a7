"""Python binding of the low-rank bottleneck block's HIP library (liblrblock.so).

Argument marshalling only: every step of the block runs in the library's HIP
kernels; torch supplies device memory and the current stream.  There is no CPU
or PyTorch fallback: if the library is missing or no GPU is present, the calls
raise.

The functions carry the C entry points' names (rmsnorm_online, lr_block_fwd,
lr_block_bwd, lr_down_partial, lr_up_finish, lr_block_workspace_size,
lr_mlp_fwd, lr_mlp_bwd, lr_status_str, ...) and take torch tensors;
``fwd``/``bwd``/``down_partial``/``up_finish``/``mlp_fwd``/``mlp_bwd``
additionally allocate the outputs and the workspace.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import torch  # loads the HIP runtime first, so the library binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblrblock.so")

LR_OK, LR_EINVAL, LR_EUNSUPPORTED, LR_EWORKSPACE, LR_EHIP = range(5)
LR_F32, LR_BF16 = 0, 1
ACTS = {"identity": 0, "silu": 1, "swiglu": 2}
DTYPES = {"f32": LR_F32, "bf16": LR_BF16}
TORCH_DTYPE = {LR_F32: torch.float32, LR_BF16: torch.bfloat16}


class LrDims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int64), ("r", ctypes.c_int64), ("g", ctypes.c_int64),
                ("d_norm", ctypes.c_int64), ("eps", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("act", ctypes.c_int32)]


class LrMlpDims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int64), ("f", ctypes.c_int64), ("r", ctypes.c_int64),
                ("eps", ctypes.c_float), ("dtype", ctypes.c_int32)]


class LrError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {lr_status_str(status)} ({status})")
        self.status = status


_lib = None
ENTRY_POINTS = ("rmsnorm_online", "lr_block_fwd", "lr_block_fwd_rstd", "lr_block_bwd", "lr_block_bwd_rstd",
                "lr_block_fwd_residual", "lr_block_bwd_residual", "lr_block_fwd_noalloc", "lr_down_partial",
                "lr_up_finish", "lr_block_workspace_size", "lr_mlp_fwd", "lr_mlp_bwd", "lr_mlp_workspace_size",
                "lr_status_str", "lr_trace_begin", "lr_trace_count", "lr_trace_elapsed", "lr_trace_end")


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load liblrblock.so (once): the in-tree build, or the file named by the
    LR_BLOCK_LIBRARY environment variable.  Raises if it does not exist."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("LR_BLOCK_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m rank_bottleneck_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i64, f32p, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(ctypes.c_float), ctypes.c_size_t
    dims = ctypes.POINTER(LrDims)
    lib.rmsnorm_online.argtypes = [dims, vp, vp, vp, vp, vp, vp]
    lib.lr_block_fwd.argtypes = [dims, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.lr_block_fwd_rstd.argtypes = [dims, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.lr_block_bwd.argtypes = [dims, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.lr_block_bwd_rstd.argtypes = [dims, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.lr_block_fwd_residual.argtypes = [dims, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.lr_block_bwd_residual.argtypes = [dims, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.lr_block_fwd_noalloc.argtypes = [dims, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.lr_down_partial.argtypes = [dims, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.lr_up_finish.argtypes = [dims, vp, vp, vp, vp, vp, vp, sz, vp]
    mdims = ctypes.POINTER(LrMlpDims)
    lib.lr_mlp_fwd.argtypes = [mdims] + [vp] * 13 + [sz, vp]
    lib.lr_mlp_bwd.argtypes = [mdims] + [vp] * 20 + [sz, vp]
    lib.lr_mlp_workspace_size.argtypes = [mdims, ctypes.c_int]
    lib.lr_mlp_workspace_size.restype = sz
    for f in ("rmsnorm_online", "lr_block_fwd", "lr_block_fwd_rstd", "lr_block_bwd", "lr_block_bwd_rstd",
              "lr_block_fwd_residual", "lr_block_bwd_residual", "lr_block_fwd_noalloc", "lr_down_partial",
              "lr_up_finish", "lr_mlp_fwd", "lr_mlp_bwd"):
        getattr(lib, f).restype = ctypes.c_int
    lib.lr_block_workspace_size.argtypes = [dims, ctypes.c_int]
    lib.lr_block_workspace_size.restype = sz
    lib.lr_status_str.argtypes = [ctypes.c_int]
    lib.lr_status_str.restype = ctypes.c_char_p
    lib.lr_trace_begin.argtypes = [ctypes.c_char_p, ctypes.c_int]
    lib.lr_trace_begin.restype = ctypes.c_int
    lib.lr_trace_count.argtypes = []
    lib.lr_trace_count.restype = ctypes.c_int
    lib.lr_trace_elapsed.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float)]
    lib.lr_trace_elapsed.restype = ctypes.c_int
    lib.lr_trace_end.argtypes = []
    lib.lr_trace_end.restype = ctypes.c_int
    _lib = lib
    return lib


def lr_status_str(status: int) -> str:
    return load().lr_status_str(int(status)).decode()


def make_dims(T: int, d: int, r: int, g: int, act: str = "silu", dtype: str = "bf16", eps: float = 1e-6,
              d_norm: int = 0) -> LrDims:
    return LrDims(T, d, r, g, d_norm, eps, DTYPES[dtype], ACTS[act])


def n_up(dims: LrDims) -> int:
    return 1 if dims.act == ACTS["swiglu"] else dims.g


def lr_block_workspace_size(dims: LrDims, backward: bool) -> int:
    return int(load().lr_block_workspace_size(ctypes.byref(dims), 1 if backward else 0))


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor is not on a GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _ptr_array(ts: Sequence[torch.Tensor]):
    arr = (ctypes.c_void_p * max(1, len(ts)))()
    for i, t in enumerate(ts):
        arr[i] = _ptr(t)
    return arr


def _stream(stream) -> Optional[int]:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(fn: str, st: int):
    if st != LR_OK:
        raise LrError(fn, st)


def _ws_nbytes(ws: Optional[torch.Tensor]) -> int:
    return 0 if ws is None else ws.numel() * ws.element_size()


# ----------------------------------------------------------------------- raw entry points
def rmsnorm_online(dims: LrDims, x, gamma=None, y=None, sumsq=None, rstd=None, stream=None) -> None:
    _check("rmsnorm_online", load().rmsnorm_online(ctypes.byref(dims), _ptr(x), _ptr(gamma), _ptr(y), _ptr(sumsq),
                                                    _ptr(rstd), _stream(stream)))


def lr_block_fwd(dims: LrDims, x, gamma, A, B: Sequence, y: Sequence, h_save, ws, stream=None) -> None:
    _check("lr_block_fwd", load().lr_block_fwd(ctypes.byref(dims), _ptr(x), _ptr(gamma), _ptr(A), _ptr_array(B),
                                                _ptr_array(y), _ptr(h_save), _ptr(ws), _ws_nbytes(ws),
                                                _stream(stream)))


def lr_block_fwd_rstd(dims: LrDims, x, gamma, A, B: Sequence, y: Sequence, h_save, rstd_save, ws,
                      stream=None) -> None:
    _check("lr_block_fwd_rstd", load().lr_block_fwd_rstd(ctypes.byref(dims), _ptr(x), _ptr(gamma), _ptr(A),
                                                          _ptr_array(B), _ptr_array(y), _ptr(h_save),
                                                          _ptr(rstd_save), _ptr(ws), _ws_nbytes(ws),
                                                          _stream(stream)))


def lr_block_bwd(dims: LrDims, x, gamma, A, B: Sequence, h_saved, dy: Sequence, dx, dgamma, dA, dB: Sequence, ws,
                 stream=None) -> None:
    _check("lr_block_bwd", load().lr_block_bwd(ctypes.byref(dims), _ptr(x), _ptr(gamma), _ptr(A), _ptr_array(B),
                                                _ptr(h_saved), _ptr_array(dy), _ptr(dx), _ptr(dgamma), _ptr(dA),
                                                _ptr_array(dB), _ptr(ws), _ws_nbytes(ws), _stream(stream)))


def lr_block_bwd_rstd(dims: LrDims, x, gamma, A, B: Sequence, h_saved, rstd_saved, dy: Sequence, dx, dgamma, dA,
                      dB: Sequence, ws, stream=None) -> None:
    _check("lr_block_bwd_rstd", load().lr_block_bwd_rstd(ctypes.byref(dims), _ptr(x), _ptr(gamma), _ptr(A),
                                                          _ptr_array(B), _ptr(h_saved), _ptr(rstd_saved),
                                                          _ptr_array(dy), _ptr(dx), _ptr(dgamma), _ptr(dA),
                                                          _ptr_array(dB), _ptr(ws), _ws_nbytes(ws),
                                                          _stream(stream)))


def lr_block_fwd_residual(dims: LrDims, x, gamma, A, B: Sequence, residual: Sequence, y: Sequence, h_save,
                          rstd_save, ws, stream=None) -> None:
    _check("lr_block_fwd_residual", load().lr_block_fwd_residual(
        ctypes.byref(dims), _ptr(x), _ptr(gamma), _ptr(A), _ptr_array(B), _ptr_array(residual), _ptr_array(y),
        _ptr(h_save), _ptr(rstd_save), _ptr(ws), _ws_nbytes(ws), _stream(stream)))


def lr_block_bwd_residual(dims: LrDims, x, gamma, A, B: Sequence, h_saved, rstd_saved, dy: Sequence, dx_residual,
                          dx, dgamma, dA, dB: Sequence, ws, stream=None) -> None:
    _check("lr_block_bwd_residual", load().lr_block_bwd_residual(
        ctypes.byref(dims), _ptr(x), _ptr(gamma), _ptr(A), _ptr_array(B), _ptr(h_saved), _ptr(rstd_saved),
        _ptr_array(dy), _ptr(dx_residual), _ptr(dx), _ptr(dgamma), _ptr(dA), _ptr_array(dB), _ptr(ws),
        _ws_nbytes(ws), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 128 << 20   # LR_NOALLOC_SCRATCH_BYTES


def lr_block_fwd_noalloc(dims: LrDims, x, gamma, A, B: Sequence, y: Sequence, h_save, rstd_save,
                         stream=None) -> None:
    """The forward with the library's per-GPU device scratch as its workspace
    (no allocation by the library; the outputs are the caller's)."""
    _check("lr_block_fwd_noalloc", load().lr_block_fwd_noalloc(
        ctypes.byref(dims), _ptr(x), _ptr(gamma), _ptr(A), _ptr_array(B), _ptr_array(y), _ptr(h_save),
        _ptr(rstd_save), _stream(stream)))


def lr_down_partial(dims: LrDims, x, gamma, A, partial, sumsq, ws, stream=None) -> None:
    _check("lr_down_partial", load().lr_down_partial(ctypes.byref(dims), _ptr(x), _ptr(gamma), _ptr(A),
                                                      _ptr(partial), _ptr(sumsq), _ptr(ws), _ws_nbytes(ws),
                                                      _stream(stream)))


def lr_up_finish(dims: LrDims, partial, sumsq, B: Sequence, y: Sequence, h_save, ws, stream=None) -> None:
    _check("lr_up_finish", load().lr_up_finish(ctypes.byref(dims), _ptr(partial), _ptr(sumsq), _ptr_array(B),
                                                _ptr_array(y), _ptr(h_save), _ptr(ws), _ws_nbytes(ws),
                                                _stream(stream)))


def make_mlp_dims(T: int, d: int, f: int, r: int, dtype: str = "bf16", eps: float = 1e-6) -> LrMlpDims:
    return LrMlpDims(T, d, f, r, eps, DTYPES[dtype])


def lr_mlp_workspace_size(dims: LrMlpDims, backward: bool) -> int:
    return int(load().lr_mlp_workspace_size(ctypes.byref(dims), 1 if backward else 0))


def lr_mlp_fwd(dims: LrMlpDims, x, gamma, A_in, B_g, B_u, A_o, B_o, residual, out, h_in_save, h_out_save,
               rstd_save, ws, stream=None) -> None:
    _check("lr_mlp_fwd", load().lr_mlp_fwd(
        ctypes.byref(dims), _ptr(x), _ptr(gamma), _ptr(A_in), _ptr(B_g), _ptr(B_u), _ptr(A_o), _ptr(B_o),
        _ptr(residual), _ptr(out), _ptr(h_in_save), _ptr(h_out_save), _ptr(rstd_save), _ptr(ws), _ws_nbytes(ws),
        _stream(stream)))


def lr_mlp_bwd(dims: LrMlpDims, x, gamma, A_in, B_g, B_u, A_o, B_o, h_in_saved, h_out_saved, rstd_saved, dout,
               dx_residual, dx, dgamma, dA_in, dB_g, dB_u, dA_o, dB_o, ws, stream=None) -> None:
    _check("lr_mlp_bwd", load().lr_mlp_bwd(
        ctypes.byref(dims), _ptr(x), _ptr(gamma), _ptr(A_in), _ptr(B_g), _ptr(B_u), _ptr(A_o), _ptr(B_o),
        _ptr(h_in_saved), _ptr(h_out_saved), _ptr(rstd_saved), _ptr(dout), _ptr(dx_residual), _ptr(dx),
        _ptr(dgamma), _ptr(dA_in), _ptr(dB_g), _ptr(dB_u), _ptr(dA_o), _ptr(dB_o), _ptr(ws), _ws_nbytes(ws),
        _stream(stream)))


def lr_trace_begin(kernel: Optional[str] = None, max_launches: int = 1024) -> None:
    _check("lr_trace_begin", load().lr_trace_begin(None if kernel is None else kernel.encode(), max_launches))


def lr_trace_count() -> int:
    return int(load().lr_trace_count())


def lr_trace_elapsed(i: int):
    """(kernel name, milliseconds) of traced launch i; waits for it to finish."""
    name, ms = ctypes.c_char_p(), ctypes.c_float()
    _check("lr_trace_elapsed", load().lr_trace_elapsed(i, ctypes.byref(name), ctypes.byref(ms)))
    return name.value.decode(), float(ms.value)


def lr_trace_end() -> None:
    _check("lr_trace_end", load().lr_trace_end())


# ----------------------------------------------------------------------- allocating helpers
def workspace(dims: LrDims, backward: bool, device="cuda") -> torch.Tensor:
    n = lr_block_workspace_size(dims, backward)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def fwd(dims: LrDims, x, gamma, A, B: Sequence, save_h: bool = True, ws=None, stream=None, rstd=None,
        residual: Optional[Sequence] = None):
    """Allocating forward: returns (list of y_i, h or None).  rstd: an fp32 [T]
    tensor that receives the rows' rstd, or None.  residual: n_up [T, d]
    tensors added to the y_i (lr_block_fwd_residual), or None."""
    dt = TORCH_DTYPE[dims.dtype]
    y = [torch.empty((dims.T, dims.d), dtype=dt, device=x.device) for _ in range(n_up(dims))]
    h = torch.empty((dims.T, dims.g * dims.r), dtype=dt, device=x.device) if save_h else None
    ws = workspace(dims, False, x.device) if ws is None else ws
    if residual is not None:
        lr_block_fwd_residual(dims, x, gamma, A, B, residual, y, h, rstd, ws, stream)
    elif rstd is None:
        lr_block_fwd(dims, x, gamma, A, B, y, h, ws, stream)
    else:
        lr_block_fwd_rstd(dims, x, gamma, A, B, y, h, rstd, ws, stream)
    return y, h


def bwd(dims: LrDims, x, gamma, A, B: Sequence, h, dy: Sequence, ws=None, stream=None, rstd=None,
        dx_residual=None):
    """Allocating backward: returns dict(dx, dgamma, dA, dB).  rstd: the forward's
    saved rstd, or None to recompute it from x.  dx_residual: a [T, d] tensor
    added to dx (lr_block_bwd_residual), or None."""
    dt = TORCH_DTYPE[dims.dtype]
    dev = x.device
    dx = torch.empty((dims.T, dims.d), dtype=dt, device=dev)
    dgamma = torch.empty(dims.d, dtype=torch.float32, device=dev)
    dA = torch.empty((dims.d, dims.g * dims.r), dtype=torch.float32, device=dev)
    dB = [torch.empty((dims.r, dims.d), dtype=torch.float32, device=dev) for _ in range(n_up(dims))]
    ws = workspace(dims, True, dev) if ws is None else ws
    if dx_residual is not None:
        lr_block_bwd_residual(dims, x, gamma, A, B, h, rstd, dy, dx_residual, dx, dgamma, dA, dB, ws, stream)
    elif rstd is None:
        lr_block_bwd(dims, x, gamma, A, B, h, dy, dx, dgamma, dA, dB, ws, stream)
    else:
        lr_block_bwd_rstd(dims, x, gamma, A, B, h, rstd, dy, dx, dgamma, dA, dB, ws, stream)
    return {"dx": dx, "dgamma": dgamma, "dA": dA, "dB": dB}


def down_partial(dims: LrDims, x, gamma, A, ws=None, stream=None):
    dev = x.device
    partial = torch.empty((dims.T, dims.g * dims.r), dtype=torch.float32, device=dev)
    sumsq = torch.empty(dims.T, dtype=torch.float32, device=dev)
    ws = workspace(dims, False, dev) if ws is None else ws
    lr_down_partial(dims, x, gamma, A, partial, sumsq, ws, stream)
    return partial, sumsq


def up_finish(dims: LrDims, partial, sumsq, B: Sequence, save_h: bool = True, ws=None, stream=None):
    dt = TORCH_DTYPE[dims.dtype]
    dev = partial.device
    y = [torch.empty((dims.T, dims.d), dtype=dt, device=dev) for _ in range(n_up(dims))]
    h = torch.empty((dims.T, dims.g * dims.r), dtype=dt, device=dev) if save_h else None
    ws = workspace(dims, False, dev) if ws is None else ws
    lr_up_finish(dims, partial, sumsq, B, y, h, ws, stream)
    return y, h


def mlp_workspace(dims: LrMlpDims, backward: bool, device="cuda") -> torch.Tensor:
    n = lr_mlp_workspace_size(dims, backward)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def mlp_fwd(dims: LrMlpDims, x, gamma, A_in, B_g, B_u, A_o, B_o, residual=None, save: bool = True, rstd=None,
            ws=None, stream=None):
    """Allocating MLP forward: returns (out, h_in or None, h_out or None).  rstd:
    an fp32 [T] tensor that receives the rows' rstd, or None."""
    dt = TORCH_DTYPE[dims.dtype]
    dev = x.device
    out = torch.empty((dims.T, dims.d), dtype=dt, device=dev)
    h_in = torch.empty((dims.T, 2 * dims.r), dtype=dt, device=dev) if save else None
    h_out = torch.empty((dims.T, dims.r), dtype=dt, device=dev) if save else None
    ws = mlp_workspace(dims, False, dev) if ws is None else ws
    lr_mlp_fwd(dims, x, gamma, A_in, B_g, B_u, A_o, B_o, residual, out, h_in, h_out, rstd, ws, stream)
    return out, h_in, h_out


def mlp_bwd(dims: LrMlpDims, x, gamma, A_in, B_g, B_u, A_o, B_o, h_in, h_out, dout, rstd=None, dx_residual=None,
            ws=None, stream=None):
    """Allocating MLP backward: returns dict(dx, dgamma, dA_in, dB_g, dB_u, dA_o, dB_o)."""
    dt = TORCH_DTYPE[dims.dtype]
    dev = x.device
    f32 = dict(dtype=torch.float32, device=dev)
    g = {"dx": torch.empty((dims.T, dims.d), dtype=dt, device=dev), "dgamma": torch.empty(dims.d, **f32),
         "dA_in": torch.empty((dims.d, 2 * dims.r), **f32), "dB_g": torch.empty((dims.r, dims.f), **f32),
         "dB_u": torch.empty((dims.r, dims.f), **f32), "dA_o": torch.empty((dims.f, dims.r), **f32),
         "dB_o": torch.empty((dims.r, dims.d), **f32)}
    ws = mlp_workspace(dims, True, dev) if ws is None else ws
    lr_mlp_bwd(dims, x, gamma, A_in, B_g, B_u, A_o, B_o, h_in, h_out, rstd, dout, dx_residual, g["dx"], g["dgamma"],
               g["dA_in"], g["dB_g"], g["dB_u"], g["dA_o"], g["dB_o"], ws, stream)
    return g
