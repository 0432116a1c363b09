"""MI355X-native LVSA frame-block-sparse attention: Python binding.

A thin ctypes layer over ``liblvsa.so`` (C ABI declared in ``include/lvsa.h``).
Every step of the computation runs in the library: the host mask builder in
C++, the attention in the gfx950 HIP kernel.  This module only marshals
arguments: torch tensors become (pointer, sizes, strides) records, the
current HIP stream is passed through, and negative status codes become
exceptions.  There is no fallback path: if the library is missing or the
device is not a gfx950, calls raise.

Functions with the ABI's names:

  lvsa_version()                      -> int
  lvsa_last_error()                   -> str
  lvsa_mask_nnz(T, C, W)              -> int
  lvsa_build_mask(T, C, W, step, flags=LVSA_ROT_MOD_TPER) -> Mask (host int32)
  lvsa_build_mask_steps(T, C, W, step0, n_steps, flags=...) -> MaskSteps (host int32)
  lvsa_validate_mask(T, row_ptr, col_idx)
  lvsa_attention(q, k, v, mask_dev, out=None, scale=None, stream=None, workspace=None) -> out
      (with a workspace: the C ABI's lvsa_attention_ws)
  lvsa_attention_workspace_bytes(B, H, N, D, T) -> int
  lvsa_attention_ws_static(q, k, v, mask_dev, out, scale=None, stream=None) -> out
      (the workspace path on the library's static device scratch; allocates nothing)

``Mask.to(device)`` copies the CSR arrays (``non_blocking`` on the current
stream) for ``lvsa_attention``.  ``MaskSteps`` holds the masks of a run of
steps in one buffer: ``.to(device)`` copies them all at once and
``.mask(i)`` is the ``Mask`` of step step0+i (views, no copy).
"""

from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

LVSA_OK = 0
LVSA_ERR_ARG = -1
LVSA_ERR_CAPACITY = -2
LVSA_ERR_SHAPE = -3
LVSA_ERR_DTYPE = -4
LVSA_ERR_HIP = -5
LVSA_ERR_MASK = -6

LVSA_ROT_MOD_TPER = 0
LVSA_ROT_MOD_T = 1
LVSA_FIXED_GRID = 2
LVSA_WINDOW_ONLY = 3

LVSA_DTYPE_BF16 = 1
LVSA_STATIC_SCRATCH_BYTES = 16 << 20

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblvsa.so")


class LvsaError(Exception):
    def __init__(self, code: int, msg: str):
        super().__init__(f"lvsa error {code}: {msg}")
        self.code = code


class LvsaValueError(LvsaError, ValueError):
    """Argument, shape, dtype, capacity or mask error (nothing was launched)."""


class LvsaDeviceError(LvsaError, RuntimeError):
    """No gfx950 device, or a HIP launch failure."""


class LvsaMaskInfo(ctypes.Structure):
    _fields_ = [("c_eff", ctypes.c_int32), ("t_per", ctypes.c_int32),
                ("n_anchor", ctypes.c_int32), ("offset", ctypes.c_int32),
                ("nnz", ctypes.c_int32)]


class LvsaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p),
                ("B", ctypes.c_int64), ("H", ctypes.c_int64), ("N", ctypes.c_int64), ("D", ctypes.c_int64),
                ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64),
                ("dtype", ctypes.c_int32)]


_LIB = None
_I32P = ctypes.POINTER(ctypes.c_int32)


def library() -> ctypes.CDLL:
    """Loads liblvsa.so once (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m block_sparse_attention_lvsa_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        lib.lvsa_version.restype = ctypes.c_int
        lib.lvsa_version.argtypes = []
        lib.lvsa_last_error.restype = ctypes.c_char_p
        lib.lvsa_last_error.argtypes = []
        lib.lvsa_mask_nnz.restype = ctypes.c_int
        lib.lvsa_mask_nnz.argtypes = [ctypes.c_int32] * 3 + [_I32P]
        lib.lvsa_build_mask.restype = ctypes.c_int
        lib.lvsa_build_mask.argtypes = [ctypes.c_int32] * 5 + [_I32P, _I32P, ctypes.c_int32,
                                                                ctypes.POINTER(LvsaMaskInfo)]
        lib.lvsa_build_mask_steps.restype = ctypes.c_int
        lib.lvsa_build_mask_steps.argtypes = [ctypes.c_int32] * 6 + [_I32P, _I32P, ctypes.c_int64,
                                                                      ctypes.POINTER(LvsaMaskInfo)]
        lib.lvsa_validate_mask.restype = ctypes.c_int
        lib.lvsa_validate_mask.argtypes = [ctypes.c_int32, _I32P, _I32P, ctypes.c_int32]
        lib.lvsa_attention.restype = ctypes.c_int
        lib.lvsa_attention.argtypes = [ctypes.POINTER(LvsaTensor)] * 3 + [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
            ctypes.POINTER(LvsaTensor), ctypes.c_float, ctypes.c_void_p]
        lib.lvsa_attention_ws.restype = ctypes.c_int
        lib.lvsa_attention_ws.argtypes = [ctypes.POINTER(LvsaTensor)] * 3 + [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
            ctypes.POINTER(LvsaTensor), ctypes.c_float, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        lib.lvsa_attention_ws_static.restype = ctypes.c_int
        lib.lvsa_attention_ws_static.argtypes = [ctypes.POINTER(LvsaTensor)] * 3 + [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
            ctypes.POINTER(LvsaTensor), ctypes.c_float, ctypes.c_void_p]
        lib.lvsa_attention_workspace_bytes.restype = ctypes.c_int
        lib.lvsa_attention_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                       ctypes.c_int64, ctypes.c_int32,
                                                       ctypes.POINTER(ctypes.c_int64)]
        _LIB = lib
    return _LIB


def _check(rc: int) -> None:
    if rc == LVSA_OK:
        return
    msg = lvsa_last_error()
    if rc == LVSA_ERR_HIP:
        raise LvsaDeviceError(rc, msg)
    raise LvsaValueError(rc, msg)


def lvsa_version() -> int:
    return library().lvsa_version()


def lvsa_last_error() -> str:
    return library().lvsa_last_error().decode("utf-8", "replace")


def lvsa_mask_nnz(T: int, C: int, W: int) -> int:
    n = ctypes.c_int32(0)
    _check(library().lvsa_mask_nnz(T, C, W, ctypes.byref(n)))
    return n.value


class Mask(NamedTuple):
    """CSR frame mask: row_ptr [T+1], col_idx [nnz] (int32), plus metadata."""
    row_ptr: "object"
    col_idx: "object"
    T: int
    c_eff: int
    t_per: int
    n_anchor: int
    offset: int
    nnz: int

    def to(self, device, non_blocking: bool = True) -> "Mask":
        return self._replace(row_ptr=self.row_ptr.to(device, non_blocking=non_blocking),
                             col_idx=self.col_idx.to(device, non_blocking=non_blocking))

    def rows(self):
        rp = self.row_ptr.tolist()
        ci = self.col_idx.tolist()
        return [ci[rp[t]:rp[t + 1]] for t in range(self.T)]


def _i32ptr(t) -> "ctypes.POINTER(ctypes.c_int32)":
    return ctypes.cast(ctypes.c_void_p(t.data_ptr()), _I32P)


def lvsa_build_mask(T: int, C: int, W: int, step: int, flags: int = LVSA_ROT_MOD_TPER,
                    pin_memory: bool = False) -> Mask:
    """Host CSR mask of one denoising step (C++ builder; see include/lvsa.h)."""
    import torch
    nnz = lvsa_mask_nnz(T, C, W)
    row_ptr = torch.empty(T + 1, dtype=torch.int32, pin_memory=pin_memory)
    col_idx = torch.empty(max(nnz, 1), dtype=torch.int32, pin_memory=pin_memory)
    info = LvsaMaskInfo()
    _check(library().lvsa_build_mask(T, C, W, step, flags, _i32ptr(row_ptr), _i32ptr(col_idx),
                                     nnz, ctypes.byref(info)))
    return Mask(row_ptr, col_idx[:nnz], T, info.c_eff, info.t_per, info.n_anchor, info.offset, info.nnz)


class MaskSteps(NamedTuple):
    """CSR masks of steps step0 .. step0+n_steps-1 sharing one row_ptr [T+1];
    col_idx is [n_steps, nnz] (int32).  ``info[i]`` = (c_eff, t_per,
    n_anchor, offset) of step step0+i."""
    row_ptr: "object"
    col_idx: "object"
    T: int
    step0: int
    n_steps: int
    nnz: int
    info: tuple

    def to(self, device, non_blocking: bool = True) -> "MaskSteps":
        return self._replace(row_ptr=self.row_ptr.to(device, non_blocking=non_blocking),
                             col_idx=self.col_idx.to(device, non_blocking=non_blocking))

    def mask(self, i: int) -> Mask:
        if not 0 <= i < self.n_steps:
            raise IndexError(f"step index {i} outside [0, {self.n_steps})")
        c_eff, t_per, n_anchor, offset = self.info[i]
        return Mask(self.row_ptr, self.col_idx[i], self.T, c_eff, t_per, n_anchor, offset, self.nnz)


def lvsa_build_mask_steps(T: int, C: int, W: int, step0: int, n_steps: int,
                          flags: int = LVSA_ROT_MOD_TPER, pin_memory: bool = False) -> MaskSteps:
    """Host CSR masks of n_steps consecutive denoising steps in one buffer
    (C++ builder; see include/lvsa.h)."""
    import torch
    nnz = lvsa_mask_nnz(T, C, W)
    if n_steps < 1:
        raise LvsaValueError(LVSA_ERR_ARG, f"n_steps={n_steps}: need n_steps >= 1")
    row_ptr = torch.empty(T + 1, dtype=torch.int32, pin_memory=pin_memory)
    col_idx = torch.empty(n_steps, nnz, dtype=torch.int32, pin_memory=pin_memory)
    infos = (LvsaMaskInfo * n_steps)()
    _check(library().lvsa_build_mask_steps(T, C, W, step0, n_steps, flags, _i32ptr(row_ptr), _i32ptr(col_idx),
                                           n_steps * nnz, infos))
    info = tuple((x.c_eff, x.t_per, x.n_anchor, x.offset) for x in infos)
    return MaskSteps(row_ptr, col_idx, T, step0, n_steps, nnz, info)


def lvsa_validate_mask(T: int, row_ptr, col_idx) -> None:
    """Host check of a CSR mask held in CPU int32 tensors; raises on a defect."""
    import torch
    rp = row_ptr.to(dtype=torch.int32, device="cpu").contiguous()
    ci = col_idx.to(dtype=torch.int32, device="cpu").contiguous()
    if rp.numel() != T + 1:
        raise LvsaValueError(LVSA_ERR_MASK, f"row_ptr has {rp.numel()} entries, expected T+1={T + 1}")
    ci_buf = ci if ci.numel() else torch.zeros(1, dtype=torch.int32)
    _check(library().lvsa_validate_mask(T, _i32ptr(rp), _i32ptr(ci_buf), ci.numel()))


def _tensor_record(x, name: str) -> LvsaTensor:
    import torch
    if x.dim() != 4:
        raise LvsaValueError(LVSA_ERR_SHAPE, f"{name}: expected [B, H, N, D], got {tuple(x.shape)}")
    if not x.is_cuda:
        raise LvsaValueError(LVSA_ERR_ARG, f"{name}: must be a device tensor")
    if x.shape[3] > 1 and x.stride(3) != 1:
        raise LvsaValueError(LVSA_ERR_SHAPE, f"{name}: innermost dimension must be contiguous")
    B, H, N, D = x.shape
    return LvsaTensor(x.data_ptr(), B, H, N, D, x.stride(0), x.stride(1), x.stride(2),
                      LVSA_DTYPE_BF16 if x.dtype == torch.bfloat16 else 0)


def lvsa_attention_workspace_bytes(B: int, H: int, N: int, D: int, T: int) -> int:
    """Device workspace bytes lvsa_attention needs when given a workspace, for
    [B, H, N, D] tensors of T frames."""
    n = ctypes.c_int64(0)
    _check(library().lvsa_attention_workspace_bytes(B, H, N, D, T, ctypes.byref(n)))
    return n.value


def lvsa_attention(q, k, v, mask: Mask, out=None, scale: Optional[float] = None, stream=None, workspace=None):
    """Frame-block-sparse attention on the GPU (see include/lvsa.h).

    q, k, v, out: [B, H, T·P, D] bf16 CUDA tensors; mask: a Mask whose
    arrays are already on q's device.  ``workspace``: optional device tensor
    of at least lvsa_attention_workspace_bytes(B, H, N, D, T) bytes (then the call
    is the ABI's lvsa_attention_ws).  Launches on ``stream`` (default: the
    current stream) and returns ``out`` without synchronising.
    """
    import torch
    if out is None:
        out = torch.empty_like(q)
    if mask.row_ptr.numel() != mask.T + 1:
        raise LvsaValueError(LVSA_ERR_ARG, f"mask.row_ptr has {mask.row_ptr.numel()} entries, need T+1")
    for name, t in (("row_ptr", mask.row_ptr), ("col_idx", mask.col_idx)):
        if t.device != q.device or t.dtype != torch.int32 or not t.is_contiguous():
            raise LvsaValueError(LVSA_ERR_ARG, f"mask.{name}: need contiguous int32 on {q.device}")
    rq, rk, rv, ro = (_tensor_record(x, n) for x, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")))
    for name, t in (("k", k), ("v", v), ("out", out)):
        if t.device != q.device:
            raise LvsaValueError(LVSA_ERR_ARG, f"{name}: on {t.device}, q on {q.device}")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    sp = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    args = (ctypes.byref(rq), ctypes.byref(rk), ctypes.byref(rv),
            ctypes.c_void_p(mask.row_ptr.data_ptr()), ctypes.c_void_p(mask.col_idx.data_ptr()),
            mask.T, mask.col_idx.numel(), ctypes.byref(ro), 0.0 if scale is None else float(scale))
    if workspace is not None and (not workspace.is_cuda or workspace.device != q.device):
        raise LvsaValueError(LVSA_ERR_ARG, f"workspace: need a device tensor on {q.device}")
    with torch.cuda.device(q.device):  # the library launches on the current device
        if workspace is None:
            _check(library().lvsa_attention(*args, ctypes.c_void_p(sp)))
        else:
            nbytes = workspace.numel() * workspace.element_size()
            _check(library().lvsa_attention_ws(*args, ctypes.c_void_p(workspace.data_ptr()), nbytes,
                                               ctypes.c_void_p(sp)))
    return out


def lvsa_attention_ws_static(q, k, v, mask: Mask, out, scale: Optional[float] = None, stream=None):
    """lvsa_attention with the library's static device scratch as its
    workspace (the C ABI's lvsa_attention_ws_static): nothing is allocated,
    here or in the library, so ``out`` must be given.  Calls that can overlap
    on one GPU race on the shared scratch (see include/lvsa.h)."""
    import torch
    if out is None:
        raise LvsaValueError(LVSA_ERR_ARG, "out: required (this entry point allocates nothing)")
    if mask.row_ptr.numel() != mask.T + 1:
        raise LvsaValueError(LVSA_ERR_ARG, f"mask.row_ptr has {mask.row_ptr.numel()} entries, need T+1")
    for name, t in (("row_ptr", mask.row_ptr), ("col_idx", mask.col_idx)):
        if t.device != q.device or t.dtype != torch.int32 or not t.is_contiguous():
            raise LvsaValueError(LVSA_ERR_ARG, f"mask.{name}: need contiguous int32 on {q.device}")
    rq, rk, rv, ro = (_tensor_record(x, n) for x, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")))
    for name, t in (("k", k), ("v", v), ("out", out)):
        if t.device != q.device:
            raise LvsaValueError(LVSA_ERR_ARG, f"{name}: on {t.device}, q on {q.device}")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    sp = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        _check(library().lvsa_attention_ws_static(
            ctypes.byref(rq), ctypes.byref(rk), ctypes.byref(rv),
            ctypes.c_void_p(mask.row_ptr.data_ptr()), ctypes.c_void_p(mask.col_idx.data_ptr()),
            mask.T, mask.col_idx.numel(), ctypes.byref(ro), 0.0 if scale is None else float(scale),
            ctypes.c_void_p(sp)))
    return out
