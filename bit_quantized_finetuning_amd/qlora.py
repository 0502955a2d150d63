"""Thin Python binding over libqlora.so (ctypes).

Argument marshalling only: every step of the layer runs in the HIP library.
PyTorch supplies device memory and the current HIP stream; the library itself
allocates nothing. If the library is missing this module raises at import --
there is no fallback path.

Function names follow the C ABI in include/qlora.h:
    qlora_quantize, qlora_dequantize, qlora_merge, qlora_forward, qlora_backward,
    qlora_adamw_step, qlora_storage_bytes, qlora_storage_bytes_absmax, qlora_workspace_bytes, qlora_nf4_codebook,
    qlora_nf4_thresholds, qlora_status_string
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

BLOCK = 64
GROUP = 256
MAX_RANK = 256
# The workspace starts with a counter region (u32 words) that must be zero before
# the first call and that every call leaves zero; its last word is set only if a
# bounded wait of the skinny-token forward timed out.
COUNTER_BYTES = 16384 * 4

F32, BF16 = 0, 1

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqlora.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -m bit_quantized_finetuning_amd.build` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)


class _Nf4Weight(ctypes.Structure):
    _fields_ = [("d_out", ctypes.c_int64), ("d_in", ctypes.c_int64), ("codes", ctypes.c_void_p),
                ("qscale", ctypes.c_void_p), ("smax", ctypes.c_void_p)]


_vp, _i64, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_W = ctypes.POINTER(_Nf4Weight)

_lib.qlora_quantize.argtypes = [_vp, ctypes.c_int, _W, _vp, _vp]
_lib.qlora_quantize.restype = ctypes.c_int
_lib.qlora_dequantize.argtypes = [_W, ctypes.c_int, _vp, _vp]
_lib.qlora_dequantize.restype = ctypes.c_int
_lib.qlora_merge.argtypes = [_W, _vp, _vp, _i32, _f32, _vp, _vp]
_lib.qlora_merge.restype = ctypes.c_int
_lib.qlora_adamw_step.argtypes = [ctypes.c_void_p, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.qlora_adamw_step.restype = ctypes.c_int
_lib.qlora_forward.argtypes = [_W, _vp, _i64, _vp, _vp, _i32, _f32, _vp, _vp, _vp, _sz, _vp]
_lib.qlora_forward.restype = ctypes.c_int
_lib.qlora_backward.argtypes = [_W, _vp, _vp, _i64, _vp, _vp, _i32, _f32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.qlora_backward.restype = ctypes.c_int
_lib.qlora_storage_bytes.argtypes = [_i64, _i64]
_lib.qlora_storage_bytes.restype = _sz
_lib.qlora_storage_bytes_absmax.argtypes = [_i64, _i64]
_lib.qlora_storage_bytes_absmax.restype = _sz
_lib.qlora_workspace_bytes.argtypes = [_i64, _i64, _i64, _i32]
_lib.qlora_workspace_bytes.restype = _sz
_lib.qlora_nf4_codebook.argtypes = [ctypes.POINTER(ctypes.c_float)]
_lib.qlora_nf4_codebook.restype = None
_lib.qlora_nf4_thresholds.argtypes = [ctypes.POINTER(ctypes.c_float)]
_lib.qlora_nf4_thresholds.restype = None
_lib.qlora_status_string.argtypes = [ctypes.c_int]
_lib.qlora_status_string.restype = ctypes.c_char_p

lib = _lib  # raw handle, for tests of the C ABI itself


class QloraError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {_lib.qlora_status_string(status).decode()} (status {status})")
        self.status = status


def _check(status: int, where: str):
    if status != 0:
        raise QloraError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


# ---------------------------------------------------------------------------
# host helpers (no GPU needed)
# ---------------------------------------------------------------------------

def qlora_nf4_codebook():
    buf = (ctypes.c_float * 16)()
    _lib.qlora_nf4_codebook(buf)
    return list(buf)


def qlora_nf4_thresholds():
    buf = (ctypes.c_float * 15)()
    _lib.qlora_nf4_thresholds(buf)
    return list(buf)


def qlora_storage_bytes(d_out: int, d_in: int) -> int:
    return int(_lib.qlora_storage_bytes(d_out, d_in))


def qlora_storage_bytes_absmax(d_out: int, d_in: int) -> int:
    return int(_lib.qlora_storage_bytes_absmax(d_out, d_in))


def qlora_workspace_bytes(d_out: int, d_in: int, T: int, r: int) -> int:
    return int(_lib.qlora_workspace_bytes(d_out, d_in, T, r))


def qlora_status_string(status: int) -> str:
    return _lib.qlora_status_string(status).decode()


# ---------------------------------------------------------------------------
# device entry points
# ---------------------------------------------------------------------------

@dataclass
class NF4Weight:
    """A quantized frozen weight: the three buffers of qlora_nf4_weight plus its shape.

    qscale None is the absmax-only storage (4.5 bits per weight): smax then holds the float32 absmax of
    every 64-weight block instead of one maximum per group of 256 blocks.
    """
    d_out: int
    d_in: int
    codes: torch.Tensor           # uint8 [d_out*d_in/2]
    qscale: torch.Tensor | None   # uint8 [d_out*d_in/64], or None
    smax: torch.Tensor            # float32 [ceil(d_out*d_in/64/256)], or [d_out*d_in/64] without qscale

    @property
    def double_quant(self) -> bool:
        return self.qscale is not None

    def _c(self):
        return _Nf4Weight(self.d_out, self.d_in, self.codes.data_ptr(),
                          None if self.qscale is None else self.qscale.data_ptr(), self.smax.data_ptr())

    @staticmethod
    def empty(d_out: int, d_in: int, device, double_quant: bool = True) -> "NF4Weight":
        n = d_out * d_in
        nb = n // BLOCK
        ng = (nb + GROUP - 1) // GROUP
        # 16-byte aligned allocations (torch's caching allocator aligns to >= 512 bytes)
        return NF4Weight(d_out, d_in,
                         torch.empty(n // 2, dtype=torch.uint8, device=device),
                         torch.empty(nb, dtype=torch.uint8, device=device) if double_quant else None,
                         torch.empty(ng if double_quant else nb, dtype=torch.float32, device=device))


_workspaces: dict = {}


def workspace(device, nbytes: int) -> torch.Tensor:
    """A zero-initialised workspace cached per device (the library leaves its counters zero after each call).

    The cached workspace is shared by every call on the device that does not pass its own: calls that may run
    concurrently (on different streams) must pass distinct workspaces (`ws=`), each zeroed once, e.g. with
    `torch.zeros(qlora_workspace_bytes(...), dtype=torch.uint8, device=...)`.
    """
    dev = torch.device(device)
    key = (dev.type, dev.index)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        size = max(nbytes, 1 << 20)
        if ws is not None:
            size = max(size, 2 * ws.numel())
        torch.cuda.synchronize(dev)
        ws = torch.zeros(size, dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def _own_workspace(ws: torch.Tensor, nbytes: int) -> torch.Tensor:
    if ws.dtype != torch.uint8 or not ws.is_contiguous() or ws.numel() < nbytes:
        raise ValueError(f"ws must be a contiguous uint8 tensor of at least {nbytes} bytes")
    return ws


def _bits(t: torch.Tensor) -> torch.Tensor:
    if t.dtype != torch.bfloat16:
        raise TypeError(f"expected a bfloat16 tensor, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t


def qlora_quantize(W: torch.Tensor, out: NF4Weight | None = None, flags: torch.Tensor | None = None,
                   double_quant: bool = True) -> NF4Weight:
    """NF4-quantize W; double_quant=False keeps each block's float32 absmax (ignored when `out` is given)."""
    if W.dim() != 2 or not W.is_contiguous():
        raise ValueError("W must be a contiguous 2-D tensor")
    if W.dtype == torch.float32:
        dt = F32
    elif W.dtype == torch.bfloat16:
        dt = BF16
    else:
        raise TypeError(f"W must be float32 or bfloat16, got {W.dtype}")
    d_out, d_in = W.shape
    if out is None:
        out = NF4Weight.empty(d_out, d_in, W.device, double_quant)
    cw = out._c()
    _check(_lib.qlora_quantize(_ptr(W), dt, ctypes.byref(cw), _ptr(flags), _stream(W.device)), "qlora_quantize")
    return out


def qlora_dequantize(w: NF4Weight, dtype=torch.bfloat16) -> torch.Tensor:
    out = torch.empty(w.d_out, w.d_in, dtype=dtype, device=w.codes.device)
    dt = BF16 if dtype == torch.bfloat16 else F32
    cw = w._c()
    _check(_lib.qlora_dequantize(ctypes.byref(cw), dt, _ptr(out), _stream(out.device)), "qlora_dequantize")
    return out


def qlora_merge(w: NF4Weight, A: torch.Tensor | None, B: torch.Tensor | None, alpha: float,
                out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 [d_out, d_in] = bf16(W_hat + (alpha/r) B A): the adapter merged into the restored weight."""
    r = 0 if A is None else A.shape[0]
    if A is not None:
        _bits(A), _bits(B)
    if out is None:
        out = torch.empty(w.d_out, w.d_in, dtype=torch.bfloat16, device=w.codes.device)
    cw = w._c()
    _check(_lib.qlora_merge(ctypes.byref(cw), _ptr(A), _ptr(B), r, alpha, _ptr(out), _stream(out.device)),
           "qlora_merge")
    return out


class AdamWHparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float)]


def qlora_adamw_step(step: int, grad: torch.Tensor, master: torch.Tensor, m: torch.Tensor, v: torch.Tensor,
                     param: torch.Tensor | None = None, lr: float = 1e-4, beta1: float = 0.9, beta2: float = 0.999,
                     eps: float = 1e-8, weight_decay: float = 0.0, stream: torch.cuda.Stream | None = None):
    """One AdamW step over float32 master/m/v (device or pinned host tensors, updated in place) from a device
    float32 gradient; param (device bf16, optional) receives bf16(master). Enqueued on `stream` (default: the
    current stream of grad's device)."""
    for t in (grad, master, m, v):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise TypeError("grad, master, m and v must be contiguous float32 tensors")
    n = grad.numel()
    if any(t.numel() != n for t in (master, m, v)) or (param is not None and param.numel() != n):
        raise ValueError("all tensors must have the same number of elements")
    if param is not None:
        _bits(param)
    hp = AdamWHparams(lr, beta1, beta2, eps, weight_decay)
    st = ctypes.c_void_p((stream or torch.cuda.current_stream(grad.device)).cuda_stream)
    _check(_lib.qlora_adamw_step(ctypes.byref(hp), step, n, _ptr(grad), _ptr(master), _ptr(m), _ptr(v),
                                 _ptr(param), st), "qlora_adamw_step")


def qlora_forward(w: NF4Weight, x: torch.Tensor, A: torch.Tensor | None, B: torch.Tensor | None, alpha: float,
                  save_u: bool = False, h: torch.Tensor | None = None, u: torch.Tensor | None = None,
                  ws: torch.Tensor | None = None):
    """h = x W_hat^T + (alpha/r) (x A^T) B^T. Returns (h, u); u is float32 [T, r] when save_u or given, else None.

    h and u may be passed in (preallocated outputs); otherwise they are allocated here.
    """
    x = _bits(x)
    T = x.shape[0]
    r = 0 if A is None else A.shape[0]
    if A is not None:
        _bits(A), _bits(B)
    if h is None:
        h = torch.empty(T, w.d_out, dtype=torch.bfloat16, device=x.device)
    if u is None and save_u and r > 0:
        u = torch.empty(T, r, dtype=torch.float32, device=x.device)
    nbytes = qlora_workspace_bytes(w.d_out, w.d_in, T, r)
    ws = workspace(x.device, nbytes) if ws is None else _own_workspace(ws, nbytes)
    cw = w._c()
    _check(_lib.qlora_forward(ctypes.byref(cw), _ptr(x), T, _ptr(A), _ptr(B), r, alpha, _ptr(h), _ptr(u),
                              _ptr(ws), ws.numel(), _stream(x.device)), "qlora_forward")
    return h, u


def qlora_backward(w: NF4Weight, x: torch.Tensor | None, dY: torch.Tensor, A: torch.Tensor | None,
                   B: torch.Tensor | None, alpha: float, u_saved: torch.Tensor | None = None,
                   need_dx: bool = True, need_dA: bool = True, need_dB: bool = True,
                   dX: torch.Tensor | None = None, dA: torch.Tensor | None = None, dB: torch.Tensor | None = None,
                   ws: torch.Tensor | None = None):
    """Returns (dX bf16 [T, d_in] | None, dA f32 [r, d_in] | None, dB f32 [d_out, r] | None).

    Outputs passed in are written in place (and count as needed); the others are allocated when needed.
    """
    dY = _bits(dY)
    T = dY.shape[0]
    r = 0 if A is None else A.shape[0]
    dev = dY.device
    if dX is None and need_dx:
        dX = torch.empty(T, w.d_in, dtype=torch.bfloat16, device=dev)
    if dA is None and need_dA and r > 0:
        dA = torch.empty(r, w.d_in, dtype=torch.float32, device=dev)
    if dB is None and need_dB and r > 0:
        dB = torch.empty(w.d_out, r, dtype=torch.float32, device=dev)
    nbytes = qlora_workspace_bytes(w.d_out, w.d_in, T, r)
    ws = workspace(dev, nbytes) if ws is None else _own_workspace(ws, nbytes)
    cw = w._c()
    _check(_lib.qlora_backward(ctypes.byref(cw), _ptr(x), _ptr(dY), T, _ptr(A), _ptr(B), r, alpha, _ptr(u_saved),
                               _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws), ws.numel(), _stream(dev)), "qlora_backward")
    return dX, dA, dB
