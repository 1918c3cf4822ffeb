"""Python binding of libdsc, the gfx950 causal dynamic short convolution library.

Argument marshalling only: each function below takes torch tensors that
already live on the GPU, reads their shapes, data pointers and the current
HIP stream, and calls the C-ABI entry point of the same name (declared in
include/dsc.h). Every step of the computation runs in the library's HIP
kernels; nothing here computes. PyTorch only supplies device memory and
streams.

The library must have been built (``python -m dynamic_short_convolutions_amd.build``);
importing works without it, but every call raises if libdsc.so is missing.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# DSC_LIBRARY names another build of the library (launch-shape sweeps); default: in-tree
LIB_PATH = os.environ.get("DSC_LIBRARY") or os.path.join(PKG_DIR, "libdsc.so")

DSC_F32, DSC_BF16 = 0, 1
STATUS_NAMES = {
    0: "DSC_SUCCESS",
    1: "DSC_ERROR_INVALID_VALUE",
    2: "DSC_ERROR_MISALIGNED",
    3: "DSC_ERROR_ALIASING",
    4: "DSC_ERROR_NOT_SUPPORTED",
    5: "DSC_ERROR_WORKSPACE",
    6: "DSC_ERROR_HIP",
}
EXPORTED = (
    "dsc_fwd",
    "dsc_bwd",
    "dsc_lowrank_fwd",
    "dsc_lowrank_bwd_workspace_bytes",
    "dsc_lowrank_bwd",
    "dsc_lowrank_bwd_noalloc",
    "dsc_fwd_varlen",
    "dsc_bwd_varlen",
    "dsc_fwd_rope",
    "dsc_bwd_rope",
    "dsc_fwd_gen",
    "dsc_fwd_gen_varlen",
    "dsc_bwd_gen",
    "dsc_bwd_gen_varlen",
    "dsc_lowrank_fwd_varlen",
    "dsc_lowrank_bwd_varlen",
    "dsc_decode_step",
    "dsc_lowrank_decode_step",
    "dsc_decode_state_from_prefill",
    "dsc_status_string",
    "dsc_abi_version",
)


class DscRope(ctypes.Structure):
    """dsc_rope_t: rotary tables (device float32 [n_pos, head_dim/2]) and the rotated channels."""
    _fields_ = [("cos", ctypes.c_void_p), ("sin", ctypes.c_void_p), ("n_pos", ctypes.c_int64),
                ("d_rot", ctypes.c_int64), ("head_dim", ctypes.c_int32), ("interleaved", ctypes.c_int32)]


class DscError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {dsc_status_string(status)}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library with argument types declared (loads it on first use)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m dynamic_short_convolutions_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        L.dsc_fwd.argtypes = [vp, vp, vp, i64, i64, i64, i64, i32, i32, ctypes.c_int, vp]
        L.dsc_bwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, ctypes.c_int, vp]
        L.dsc_lowrank_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, ctypes.c_int, vp]
        L.dsc_lowrank_bwd_workspace_bytes.argtypes = [i64, i64, i64, i32, i32, ctypes.c_int]
        L.dsc_lowrank_bwd_workspace_bytes.restype = sz
        L.dsc_lowrank_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i64, i32, i32, i32,
                                      ctypes.c_int, vp]
        L.dsc_fwd_varlen.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, ctypes.c_int, vp]
        L.dsc_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, ctypes.c_int, vp]
        L.dsc_fwd_gen.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i32, i64, i32, ctypes.c_int, vp]
        L.dsc_fwd_gen_varlen.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i64, i32, ctypes.c_int, vp]
        L.dsc_bwd_gen.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i64, i32, ctypes.c_int, vp]
        L.dsc_bwd_gen_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i64, i32,
                                         ctypes.c_int, vp]
        L.dsc_fwd_rope.argtypes = [vp, vp, vp, ctypes.POINTER(DscRope), vp, i64, i64, i64, i64, i32, i32,
                                   ctypes.c_int, vp]
        L.dsc_bwd_rope.argtypes = [vp, vp, vp, ctypes.POINTER(DscRope), vp, vp, vp, i64, i64, i64, i64, i32, i32,
                                   ctypes.c_int, vp]
        L.dsc_lowrank_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, ctypes.c_int, vp]
        L.dsc_lowrank_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i64, i32, i32, i32,
                                             ctypes.c_int, vp]
        L.dsc_lowrank_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32,
                                              ctypes.c_int, vp]
        L.dsc_decode_step.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, ctypes.c_int, vp]
        L.dsc_lowrank_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, ctypes.c_int, vp]
        L.dsc_decode_state_from_prefill.argtypes = [vp, vp, vp, i64, i64, i64, i32, ctypes.c_int, vp]
        for f in ("dsc_fwd", "dsc_bwd", "dsc_lowrank_fwd", "dsc_lowrank_bwd", "dsc_lowrank_bwd_noalloc",
                  "dsc_fwd_varlen", "dsc_bwd_varlen",
                  "dsc_lowrank_fwd_varlen", "dsc_lowrank_bwd_varlen", "dsc_fwd_rope", "dsc_bwd_rope",
                  "dsc_fwd_gen", "dsc_fwd_gen_varlen", "dsc_bwd_gen", "dsc_bwd_gen_varlen", "dsc_decode_step",
                  "dsc_lowrank_decode_step", "dsc_decode_state_from_prefill"):
            getattr(L, f).restype = ctypes.c_int
        L.dsc_status_string.argtypes = [ctypes.c_int]
        L.dsc_status_string.restype = ctypes.c_char_p
        L.dsc_abi_version.argtypes = []
        L.dsc_abi_version.restype = ctypes.c_int32
        _lib = L
    return _lib


def dsc_status_string(status: int) -> str:
    return lib().dsc_status_string(int(status)).decode()


def dsc_abi_version() -> int:
    return int(lib().dsc_abi_version())


# ----------------------------------------------------------------------------- torch marshalling

def _dtype_code(*tensors) -> int:
    import torch

    kinds = {t.dtype for t in tensors}
    if kinds == {torch.bfloat16}:
        return DSC_BF16
    if kinds == {torch.float32}:
        return DSC_F32
    raise TypeError(f"all tensors must be bfloat16 or all float32, got {kinds}")


def _ptr(t) -> int:
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(status: int, where: str) -> None:
    if status != 0:
        raise DscError(status, where)


def dsc_fwd(x, w, y, residual: bool, stream=None) -> None:
    """y = residual*x + head-wise dynamic conv of x with w. x, y [B,T,D]; w [B,T,G,W]."""
    B, T, D = x.shape
    _, _, G, W = w.shape
    st = lib().dsc_fwd(_ptr(x), _ptr(w), _ptr(y), B, T, D, G, W, int(residual), _dtype_code(x, w, y),
                       _stream(stream))
    _check(st, "dsc_fwd")


def dsc_bwd(x, w, dy, dx, dw, residual: bool, stream=None) -> None:
    """Gradients dx [B,T,D] and dw [B,T,G,W] of dsc_fwd given dy."""
    B, T, D = x.shape
    _, _, G, W = w.shape
    st = lib().dsc_bwd(_ptr(x), _ptr(w), _ptr(dy), _ptr(dx), _ptr(dw), B, T, D, G, W, int(residual),
                       _dtype_code(x, w, dy, dx, dw), _stream(stream))
    _check(st, "dsc_bwd")


def dsc_lowrank_fwd(x, z, U, y, W: int, residual: bool, stream=None) -> None:
    """y = residual*x + dynamic conv of x with filters z.U. x, y [B,T,D]; z [B,T,R]; U [R,D*W]."""
    B, T, D = x.shape
    R = z.shape[2]
    st = lib().dsc_lowrank_fwd(_ptr(x), _ptr(z), _ptr(U), _ptr(y), B, T, D, R, W, int(residual),
                               _dtype_code(x, z, U, y), _stream(stream))
    _check(st, "dsc_lowrank_fwd")


def dsc_lowrank_bwd_workspace_bytes(B: int, T: int, D: int, R: int, W: int, dtype_code: int) -> int:
    return int(lib().dsc_lowrank_bwd_workspace_bytes(B, T, D, R, W, dtype_code))


def dsc_lowrank_bwd(x, z, U, dy, dx, dz, dU, workspace, W: int, residual: bool, stream=None) -> None:
    """Gradients dx, dz, dU of dsc_lowrank_fwd given dy. workspace: a uint8 GPU tensor (or None)
    of at least dsc_lowrank_bwd_workspace_bytes bytes."""
    B, T, D = x.shape
    R = z.shape[2]
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().dsc_lowrank_bwd(_ptr(x), _ptr(z), _ptr(U), _ptr(dy), _ptr(dx), _ptr(dz), _ptr(dU), ws_ptr,
                               ws_bytes, B, T, D, R, W, int(residual), _dtype_code(x, z, U, dy, dx, dz, dU),
                               _stream(stream))
    _check(st, "dsc_lowrank_bwd")


NOALLOC_SCRATCH_BYTES = 128 << 20  # DSC_NOALLOC_SCRATCH_BYTES


def dsc_lowrank_bwd_noalloc(x, z, U, dy, dx, dz, dU, W: int, residual: bool, stream=None) -> None:
    """dsc_lowrank_bwd without a workspace: the library's own per-GPU scratch array holds the
    partial sums (problems needing more than NOALLOC_SCRATCH_BYTES are refused). Calls that
    overlap on one GPU race."""
    B, T, D = x.shape
    R = z.shape[2]
    st = lib().dsc_lowrank_bwd_noalloc(_ptr(x), _ptr(z), _ptr(U), _ptr(dy), _ptr(dx), _ptr(dz), _ptr(dU), B, T, D,
                                       R, W, int(residual), _dtype_code(x, z, U, dy, dx, dz, dU), _stream(stream))
    _check(st, "dsc_lowrank_bwd_noalloc")


# ----------------------------------------------------------------------------- packed sequences

def dsc_fwd_varlen(x, w, pos, y, residual: bool, stream=None) -> None:
    """dsc_fwd with pos [B,T] int32: each token's index within its packed sequence."""
    B, T, D = x.shape
    _, _, G, W = w.shape
    st = lib().dsc_fwd_varlen(_ptr(x), _ptr(w), _int32_ptr(pos), _ptr(y), B, T, D, G, W, int(residual),
                              _dtype_code(x, w, y), _stream(stream))
    _check(st, "dsc_fwd_varlen")


def dsc_bwd_varlen(x, w, pos, dy, dx, dw, residual: bool, stream=None) -> None:
    """Gradients of dsc_fwd_varlen."""
    B, T, D = x.shape
    _, _, G, W = w.shape
    st = lib().dsc_bwd_varlen(_ptr(x), _ptr(w), _int32_ptr(pos), _ptr(dy), _ptr(dx), _ptr(dw), B, T, D, G, W,
                              int(residual), _dtype_code(x, w, dy, dx, dw), _stream(stream))
    _check(st, "dsc_bwd_varlen")


def dsc_lowrank_fwd_varlen(x, z, U, pos, y, W: int, residual: bool, stream=None) -> None:
    """dsc_lowrank_fwd with pos [B,T] int32 positions within packed sequences."""
    B, T, D = x.shape
    R = z.shape[2]
    st = lib().dsc_lowrank_fwd_varlen(_ptr(x), _ptr(z), _ptr(U), _int32_ptr(pos), _ptr(y), B, T, D, R, W,
                                      int(residual), _dtype_code(x, z, U, y), _stream(stream))
    _check(st, "dsc_lowrank_fwd_varlen")


def dsc_lowrank_bwd_varlen(x, z, U, pos, dy, dx, dz, dU, workspace, W: int, residual: bool, stream=None) -> None:
    """Gradients of dsc_lowrank_fwd_varlen (workspace as for dsc_lowrank_bwd)."""
    B, T, D = x.shape
    R = z.shape[2]
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().dsc_lowrank_bwd_varlen(_ptr(x), _ptr(z), _ptr(U), _int32_ptr(pos), _ptr(dy), _ptr(dx), _ptr(dz),
                                      _ptr(dU), ws_ptr, ws_bytes, B, T, D, R, W, int(residual),
                                      _dtype_code(x, z, U, dy, dx, dz, dU), _stream(stream))
    _check(st, "dsc_lowrank_bwd_varlen")


# ----------------------------------------------------------------------------- rotary epilogue

def rope_args(cos, sin, d_rot: int, head_dim: int, interleaved: bool) -> DscRope:
    """dsc_rope_t for float32 GPU tables cos, sin [n_pos, head_dim/2]."""
    import torch

    for t in (cos, sin):
        if t.dtype != torch.float32:
            raise TypeError("rotary tables must be float32")
    if tuple(cos.shape) != tuple(sin.shape) or cos.dim() != 2:
        raise ValueError("rotary tables must both be [n_pos, head_dim/2]")
    return DscRope(_ptr(cos), _ptr(sin), cos.shape[0], int(d_rot), int(head_dim), int(interleaved))


def dsc_fwd_rope(x, w, pos, rope: DscRope, y, residual: bool, stream=None) -> None:
    """y = rotary embedding (channels [0, d_rot)) of residual*x + head-wise conv of x with w.
    pos: [B,T] int32 positions within packed sequences, or None (position t)."""
    B, T, D = x.shape
    _, _, G, W = w.shape
    st = lib().dsc_fwd_rope(_ptr(x), _ptr(w), _int32_ptr(pos) if pos is not None else None, ctypes.byref(rope),
                            _ptr(y), B, T, D, G, W, int(residual), _dtype_code(x, w, y), _stream(stream))
    _check(st, "dsc_fwd_rope")


def dsc_bwd_rope(x, w, pos, rope: DscRope, dy, dx, dw, residual: bool, stream=None) -> None:
    """Gradients dx, dw of dsc_fwd_rope given dy."""
    B, T, D = x.shape
    _, _, G, W = w.shape
    st = lib().dsc_bwd_rope(_ptr(x), _ptr(w), _int32_ptr(pos) if pos is not None else None, ctypes.byref(rope),
                            _ptr(dy), _ptr(dx), _ptr(dw), B, T, D, G, W, int(residual), _dtype_code(x, w, dy, dx, dw),
                            _stream(stream))
    _check(st, "dsc_bwd_rope")


# ----------------------------------------------------------------------------- generator in the kernel

def dsc_fwd_gen(x, h, Wg, y, W: int, residual: bool, stream=None) -> None:
    """Head-wise forward with filters w = h . Wg^T formed in the kernel. x, y [B,T,D]; h [B,T,K];
    Wg [G*W, K] (a linear layer's weight)."""
    B, T, D = x.shape
    K = h.shape[2]
    G = Wg.shape[0] // W
    if Wg.shape[0] != G * W or Wg.shape[1] != K:
        raise ValueError("Wg must be [G*W, K]")
    st = lib().dsc_fwd_gen(_ptr(x), _ptr(h), _ptr(Wg), _ptr(y), B, T, D, G, W, K, int(residual),
                           _dtype_code(x, h, Wg, y), _stream(stream))
    _check(st, "dsc_fwd_gen")


def dsc_fwd_gen_varlen(x, h, Wg, pos, y, W: int, residual: bool, stream=None) -> None:
    """dsc_fwd_gen with pos [B,T] int32: each token's index within its packed sequence."""
    B, T, D = x.shape
    K = h.shape[2]
    G = Wg.shape[0] // W
    if Wg.shape[0] != G * W or Wg.shape[1] != K:
        raise ValueError("Wg must be [G*W, K]")
    st = lib().dsc_fwd_gen_varlen(_ptr(x), _ptr(h), _ptr(Wg), _int32_ptr(pos), _ptr(y), B, T, D, G, W, K,
                                  int(residual), _dtype_code(x, h, Wg, y), _stream(stream))
    _check(st, "dsc_fwd_gen_varlen")


def _gen_dims(x, h, Wg, W):
    B, T, D = x.shape
    K = h.shape[2]
    G = Wg.shape[0] // W
    if Wg.shape[0] != G * W or Wg.shape[1] != K:
        raise ValueError("Wg must be [G*W, K]")
    return B, T, D, G, K


def dsc_bwd_gen(x, h, Wg, dy, dx, dw, W: int, residual: bool, stream=None) -> None:
    """Gradients of dsc_fwd_gen: dx [B,T,D] and dw [B,T,G,W] (the generated filters'
    gradient), with the filters regenerated in the kernel."""
    B, T, D, G, K = _gen_dims(x, h, Wg, W)
    st = lib().dsc_bwd_gen(_ptr(x), _ptr(h), _ptr(Wg), _ptr(dy), _ptr(dx), _ptr(dw), B, T, D, G, W, K,
                           int(residual), _dtype_code(x, h, Wg, dy, dx, dw), _stream(stream))
    _check(st, "dsc_bwd_gen")


def dsc_bwd_gen_varlen(x, h, Wg, pos, dy, dx, dw, W: int, residual: bool, stream=None) -> None:
    """dsc_bwd_gen with pos [B,T] int32: each token's index within its packed sequence."""
    B, T, D, G, K = _gen_dims(x, h, Wg, W)
    st = lib().dsc_bwd_gen_varlen(_ptr(x), _ptr(h), _ptr(Wg), _int32_ptr(pos), _ptr(dy), _ptr(dx), _ptr(dw), B, T,
                                  D, G, W, K, int(residual), _dtype_code(x, h, Wg, dy, dx, dw), _stream(stream))
    _check(st, "dsc_bwd_gen_varlen")


# ----------------------------------------------------------------------------- decoding

def _int32_ptr(t) -> int:
    import torch

    if t.dtype != torch.int32:
        raise TypeError("positions and lengths must be int32")
    return _ptr(t)


def _ring_ptr(state, W: int):
    """The ring's pointer; W == 1 keeps no ring (None or an empty tensor)."""
    if W == 1 and (state is None or state.numel() == 0):
        return None
    return _ptr(state)


def dsc_decode_step(x, w, pos, state, y, residual: bool, stream=None) -> None:
    """One decode step, head-wise filters. x, y [B,D]; w [B,G,W]; pos [B] int32, the index of
    each row's token in its sequence (negative: idle row); state [B,W-1,D] ring, updated in place."""
    B, D = x.shape
    _, G, W = w.shape
    tensors = [x, w, y] + ([state] if _ring_ptr(state, W) is not None else [])
    st = lib().dsc_decode_step(_ptr(x), _ptr(w), _int32_ptr(pos), _ring_ptr(state, W), _ptr(y), B, D, G, W,
                               int(residual), _dtype_code(*tensors), _stream(stream))
    _check(st, "dsc_decode_step")


def dsc_lowrank_decode_step(x, z, U, pos, state, y, W: int, residual: bool, stream=None) -> None:
    """One decode step, low-rank filters z.U. x, y [B,D]; z [B,R]; U [R,D*W]; pos, state as
    for dsc_decode_step."""
    B, D = x.shape
    R = z.shape[1]
    tensors = [x, z, U, y] + ([state] if _ring_ptr(state, W) is not None else [])
    st = lib().dsc_lowrank_decode_step(_ptr(x), _ptr(z), _ptr(U), _int32_ptr(pos), _ring_ptr(state, W), _ptr(y),
                                       B, D, R, W, int(residual), _dtype_code(*tensors), _stream(stream))
    _check(st, "dsc_lowrank_decode_step")


def dsc_decode_state_from_prefill(x, lengths, state, W: int, stream=None) -> None:
    """Fill each row's ring from its prompt: x [B,T,D], lengths [B] int32 (tokens consumed),
    state [B,W-1,D] updated in place."""
    B, T, D = x.shape
    tensors = [x] + ([state] if _ring_ptr(state, W) is not None else [])
    st = lib().dsc_decode_state_from_prefill(_ptr(x), _int32_ptr(lengths), _ring_ptr(state, W), B, T, D, W,
                                             _dtype_code(*tensors), _stream(stream))
    _check(st, "dsc_decode_state_from_prefill")
