"""Thin Python binding over libqlora.so (ctypes).

Argument marshalling only: every step of the layer runs in the HIP library.
PyTorch supplies device memory and the current HIP stream; the library itself
allocates nothing. If the library is missing this module raises at import --
there is no fallback path.

Function names follow the C ABI in include/qlora.h:
    qlora_quantize, qlora_dequantize, qlora_merge, qlora_forward, qlora_forward_noalloc, qlora_backward,
    qlora_adamw_step, qlora_adamw_step_host, qlora_workspace_fallbacks, qlora_workspace_set_wait_limit, qlora_storage_bytes,
    qlora_storage_bytes_absmax,
    qlora_workspace_bytes, qlora_nf4_codebook, qlora_nf4_thresholds, qlora_status_string

The C ABI sees only pointers, so every tensor argument is checked here before the call: its shape against the
weight and the other operands, its dtype, contiguity, and that it lives on the weight's GPU. A mismatch raises
TypeError (dtype) or ValueError (shape, layout, device) and nothing is launched.
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
# the first call and that every call leaves zero, except its last word, which
# counts the waits that ran out of time (qlora_workspace_fallbacks).
COUNTER_BYTES = 16384 * 4
STATIC_SCRATCH_BYTES = 1 << 20  # QLORA_STATIC_SCRATCH_BYTES: scratch of qlora_forward_noalloc per GPU

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
_lib.qlora_quantize_many.argtypes = [ctypes.POINTER(_vp), ctypes.c_int, _W, _i32, _vp, _vp]
_lib.qlora_quantize_many.restype = ctypes.c_int
_lib.qlora_dequantize.argtypes = [_W, ctypes.c_int, _vp, _vp]
_lib.qlora_dequantize.restype = ctypes.c_int
_lib.qlora_merge.argtypes = [_W, _vp, _vp, _i32, _f32, _vp, _vp]
_lib.qlora_merge.restype = ctypes.c_int
_lib.qlora_adamw_step.argtypes = [ctypes.c_void_p, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.qlora_adamw_step.restype = ctypes.c_int
_lib.qlora_adamw_step_host.argtypes = [ctypes.c_void_p, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _i32]
_lib.qlora_adamw_step_host.restype = ctypes.c_int
_lib.qlora_forward.argtypes = [_W, _vp, _i64, _vp, _vp, _i32, _f32, _vp, _vp, _vp, _sz, _vp]
_lib.qlora_forward.restype = ctypes.c_int


class _ForwardJob(ctypes.Structure):
    _fields_ = [("W", _W), ("x", _vp), ("T", _i64), ("A", _vp), ("B", _vp), ("r", _i32), ("alpha", _f32),
                ("h", _vp), ("u_out", _vp)]


_lib.qlora_forward_many.argtypes = [ctypes.POINTER(_ForwardJob), _i32, _vp, _sz, _vp]
_lib.qlora_forward_many.restype = ctypes.c_int
_lib.qlora_forward_many_workspace_bytes.argtypes = [_i32]
_lib.qlora_forward_many_workspace_bytes.restype = _sz
_lib.qlora_forward_noalloc.argtypes = [_W, _vp, _i64, _vp, _vp, _i32, _f32, _vp, _vp, _vp]
_lib.qlora_forward_noalloc.restype = ctypes.c_int
_lib.qlora_workspace_fallbacks.argtypes = [_vp, ctypes.POINTER(ctypes.c_uint32), _vp]
_lib.qlora_workspace_fallbacks.restype = ctypes.c_int
_lib.qlora_workspace_set_wait_limit.argtypes = [_vp, ctypes.c_uint32, _vp]
_lib.qlora_workspace_set_wait_limit.restype = ctypes.c_int
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


def _arg(t, name: str, dtype, shape):
    """dtype, shape and contiguity of one tensor argument (None passes)."""
    if t is None:
        return
    if not torch.is_tensor(t):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_weight(w: "NF4Weight"):
    n = w.d_out * w.d_in
    if w.d_in % BLOCK or n <= 0:
        raise ValueError(f"weight shape {w.d_out}x{w.d_in}: d_in must be a positive multiple of {BLOCK}")
    nb = n // BLOCK
    _arg(w.codes, "codes", torch.uint8, (n // 2,))
    if w.qscale is not None:
        _arg(w.qscale, "qscale", torch.uint8, (nb,))
        _arg(w.smax, "smax", torch.float32, ((nb + GROUP - 1) // GROUP,))
    else:
        _arg(w.smax, "smax", torch.float32, (nb,))


def _check_devices(device, **tensors):
    """Every given tensor on `device`, a GPU (the checks that come last, so that the shape rules can be
    exercised without one)."""
    if device.type != "cuda":
        raise ValueError(f"the weight must be on a GPU, got {device}")
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, the weight on {device}")


def _adapter_rank(w: "NF4Weight", A, B) -> int:
    if (A is None) != (B is None):
        raise ValueError("give both A and B, or neither")
    if A is None:
        return 0
    if A.dim() != 2:
        raise ValueError(f"A must be [r, d_in], got shape {tuple(A.shape)}")
    r = A.shape[0]
    if r < 0 or r > MAX_RANK or r % 8:
        raise ValueError(f"rank {r} outside 0..{MAX_RANK} or not a multiple of 8")
    _arg(A, "A", torch.bfloat16, (r, w.d_in))
    _arg(B, "B", torch.bfloat16, (w.d_out, r))
    return r


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
    if (out.d_out, out.d_in) != (d_out, d_in):
        raise ValueError(f"out is {out.d_out}x{out.d_in}, W is {d_out}x{d_in}")
    _check_weight(out)
    if flags is not None and (flags.dtype not in (torch.int32, torch.uint32) or flags.numel() < 1):
        raise TypeError("flags must be a 32-bit integer tensor of at least one element")
    _check_devices(W.device, codes=out.codes, qscale=out.qscale, smax=out.smax, flags=flags)
    cw = out._c()
    _check(_lib.qlora_quantize(_ptr(W), dt, ctypes.byref(cw), _ptr(flags), _stream(W.device)), "qlora_quantize")
    return out


def qlora_quantize_many(Ws, outs=None, flags: torch.Tensor | None = None,
                        double_quant: bool = True) -> list:
    """NF4-quantize several weights of one dtype in shared launches (the results equal one qlora_quantize per
    weight); `outs` (optional) names each weight's output buffers."""
    Ws = list(Ws)
    if not Ws:
        return []
    dtypes = {W.dtype for W in Ws}
    if len(dtypes) != 1 or dtypes.pop() not in (torch.float32, torch.bfloat16):
        raise TypeError("all weights must be float32, or all bfloat16")
    dt = F32 if Ws[0].dtype == torch.float32 else BF16
    if outs is None:
        outs = [None] * len(Ws)
    outs = list(outs)
    if len(outs) != len(Ws):
        raise ValueError(f"{len(Ws)} weights but {len(outs)} outputs")
    if flags is not None and (flags.dtype not in (torch.int32, torch.uint32) or flags.numel() < 1):
        raise TypeError("flags must be a 32-bit integer tensor of at least one element")
    for i, W in enumerate(Ws):
        if W.dim() != 2 or not W.is_contiguous():
            raise ValueError("every W must be a contiguous 2-D tensor")
        if outs[i] is None:
            outs[i] = NF4Weight.empty(W.shape[0], W.shape[1], W.device, double_quant)
        o = outs[i]
        if (o.d_out, o.d_in) != tuple(W.shape):
            raise ValueError(f"out {i} is {o.d_out}x{o.d_in}, W is {W.shape[0]}x{W.shape[1]}")
        _check_weight(o)
        _check_devices(Ws[0].device, W=W, codes=o.codes, qscale=o.qscale, smax=o.smax, flags=flags)
    wp = (_vp * len(Ws))(*[W.data_ptr() for W in Ws])
    cw = (_Nf4Weight * len(Ws))(*[o._c() for o in outs])
    _check(_lib.qlora_quantize_many(wp, dt, cw, len(Ws), _ptr(flags), _stream(Ws[0].device)),
           "qlora_quantize_many")
    return outs


def qlora_dequantize(w: NF4Weight, dtype=torch.bfloat16) -> torch.Tensor:
    if dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"dtype must be bfloat16 or float32, got {dtype}")
    _check_weight(w)
    _check_devices(w.codes.device, qscale=w.qscale, smax=w.smax)
    out = torch.empty(w.d_out, w.d_in, dtype=dtype, device=w.codes.device)
    dt = BF16 if dtype == torch.bfloat16 else F32
    cw = w._c()
    _check(_lib.qlora_dequantize(ctypes.byref(cw), dt, _ptr(out), _stream(out.device)), "qlora_dequantize")
    return out


def qlora_merge(w: NF4Weight, A: torch.Tensor | None, B: torch.Tensor | None, alpha: float,
                out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 [d_out, d_in] = bf16(W_hat + (alpha/r) B A): the adapter merged into the restored weight."""
    _check_weight(w)
    r = _adapter_rank(w, A, B)
    _arg(out, "out", torch.bfloat16, (w.d_out, w.d_in))
    dev = w.codes.device
    _check_devices(dev, qscale=w.qscale, smax=w.smax, A=A, B=B, out=out)
    if out is None:
        out = torch.empty(w.d_out, w.d_in, dtype=torch.bfloat16, device=dev)
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
    if grad.device.type != "cuda":
        raise ValueError(f"grad must be on a GPU, got {grad.device}")
    _check_devices(grad.device, param=param)
    for name, t in (("master", master), ("m", m), ("v", v)):
        if t.device != grad.device and not (t.device.type == "cpu" and t.is_pinned()):
            raise ValueError(f"{name} must be on the gradient's GPU or in pinned host memory, got {t.device}")
    hp = AdamWHparams(lr, beta1, beta2, eps, weight_decay)
    st = ctypes.c_void_p((stream or torch.cuda.current_stream(grad.device)).cuda_stream)
    _check(_lib.qlora_adamw_step(ctypes.byref(hp), step, n, _ptr(grad), _ptr(master), _ptr(m), _ptr(v),
                                 _ptr(param), st), "qlora_adamw_step")


def qlora_adamw_step_host(step: int, grad: torch.Tensor, master: torch.Tensor, m: torch.Tensor, v: torch.Tensor,
                          param: torch.Tensor | None = None, lr: float = 1e-4, beta1: float = 0.9,
                          beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 0.0, threads: int = 0):
    """The same AdamW step run by the host CPU: every tensor in host memory (pinned, so that the caller's copies
    to and from the device are DMA copies); param (bf16, optional) receives bf16(master). Blocks until done."""
    for t in (grad, master, m, v):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise TypeError("grad, master, m and v must be contiguous float32 tensors")
    n = grad.numel()
    if any(t.numel() != n for t in (master, m, v)) or (param is not None and param.numel() != n):
        raise ValueError("all tensors must have the same number of elements")
    if param is not None:
        _bits(param)
    for name, t in (("grad", grad), ("master", master), ("m", m), ("v", v), ("param", param)):
        if t is not None and t.device.type != "cpu":
            raise ValueError(f"{name} must be in host memory, got {t.device}")
    hp = AdamWHparams(lr, beta1, beta2, eps, weight_decay)
    _check(_lib.qlora_adamw_step_host(ctypes.byref(hp), step, n, _ptr(grad), _ptr(master), _ptr(m), _ptr(v),
                                      _ptr(param), int(threads)), "qlora_adamw_step_host")


def _check_no_overlap(inputs: dict, outputs: dict):
    """The kernels read their inputs while they write their outputs and workspace: no output may overlap an
    input or another output (in-place calls are not supported)."""
    named = [(n, _span(t), False) for n, t in inputs.items()] + [(n, _span(t), True) for n, t in outputs.items()]
    for i, (n1, s1, out1) in enumerate(named):
        if not out1 or s1 is None:
            continue
        for k, (n2, s2, _) in enumerate(named):
            if k != i and s2 is not None and s1[0] < s2[1] and s2[0] < s1[1]:
                raise ValueError(f"{n1} overlaps {n2}: outputs and workspace must not share memory with any "
                                 "other argument")


def _forward_args(w, x, A, B, h, u, save_u, ws=None):
    _check_weight(w)
    if not torch.is_tensor(x) or x.dim() != 2:
        raise ValueError("x must be a 2-D [T, d_in] tensor")
    T = x.shape[0]
    _arg(x, "x", torch.bfloat16, (T, w.d_in))
    r = _adapter_rank(w, A, B)
    _arg(h, "h", torch.bfloat16, (T, w.d_out))
    if u is not None and r == 0:
        raise ValueError("u is given but there is no adapter")
    _arg(u, "u", torch.float32, (T, r))
    if ws is not None:
        _own_workspace(ws, qlora_workspace_bytes(w.d_out, w.d_in, T, r))
    _check_no_overlap({"x": x, "A": A, "B": B, "codes": w.codes, "qscale": w.qscale, "smax": w.smax},
                      {"h": h, "u": u, "ws": ws})
    dev = w.codes.device
    _check_devices(dev, qscale=w.qscale, smax=w.smax, x=x, A=A, B=B, h=h, u=u, ws=ws)
    if h is None:
        h = torch.empty(T, w.d_out, dtype=torch.bfloat16, device=dev)
    if u is None and save_u and r > 0:
        u = torch.empty(T, r, dtype=torch.float32, device=dev)
    return T, r, h, u


def qlora_forward(w: NF4Weight, x: torch.Tensor, A: torch.Tensor | None, B: torch.Tensor | None, alpha: float,
                  save_u: bool = False, h: torch.Tensor | None = None, u: torch.Tensor | None = None,
                  ws: torch.Tensor | None = None):
    """h = x W_hat^T + (alpha/r) (x A^T) B^T. Returns (h, u); u is float32 [T, r] when save_u or given, else None.

    h and u may be passed in (preallocated outputs); otherwise they are allocated here.
    """
    T, r, h, u = _forward_args(w, x, A, B, h, u, save_u, ws)
    if ws is None:
        ws = workspace(x.device, qlora_workspace_bytes(w.d_out, w.d_in, T, r))
    cw = w._c()
    _check(_lib.qlora_forward(ctypes.byref(cw), _ptr(x), T, _ptr(A), _ptr(B), r, alpha, _ptr(h), _ptr(u),
                              _ptr(ws), ws.numel(), _stream(x.device)), "qlora_forward")
    return h, u


MAX_FORWARD_JOBS = 64  # QLORA_MAX_FORWARD_JOBS


def _span(t):
    return None if t is None or t.numel() == 0 else (t.data_ptr(), t.data_ptr() + t.numel() * t.element_size())


def _check_independent(args):
    """The jobs of one grouped launch run at the same time: no output may overlap an input or output of any job
    (its own inputs included)."""
    spans = []
    for i, (w, x, T, A, B, r, alpha, h, u) in enumerate(args):
        for name, t in (("x", x), ("A", A), ("B", B), ("codes", w.codes), ("qscale", w.qscale), ("smax", w.smax)):
            spans.append((i, name, False, _span(t)))
        for name, t in (("h", h), ("u", u)):
            spans.append((i, name, True, _span(t)))
    for i, n1, out1, s1 in spans:
        if not out1 or s1 is None:
            continue
        for k, n2, out2, s2 in spans:
            if s2 is None or (k == i and n2 == n1):
                continue
            if s1[0] < s2[1] and s2[0] < s1[1]:
                raise ValueError(f"job {i}'s {n1} overlaps job {k}'s {n2}: the jobs of a grouped call must be "
                                 "independent")


def qlora_forward_many_workspace_bytes(count: int) -> int:
    return int(_lib.qlora_forward_many_workspace_bytes(int(count)))


def qlora_forward_many(jobs, ws: torch.Tensor | None = None):
    """Several independent forwards of T <= 16 tokens in as few launches as possible (qlora_forward_many).

    jobs: a sequence of dicts with keys w, x, A, B, alpha and optionally h, u (preallocated outputs) and save_u,
    as for qlora_forward. Returns [(h, u), ...] in job order. No job's output may overlap another job's input
    or output.
    """
    jobs = list(jobs)
    if not 1 <= len(jobs) <= MAX_FORWARD_JOBS:
        raise ValueError(f"between 1 and {MAX_FORWARD_JOBS} jobs, got {len(jobs)}")
    args, outs = [], []
    dev = None
    for i, j in enumerate(jobs):
        w = j["w"]
        T, r, h, u = _forward_args(w, j["x"], j.get("A"), j.get("B"), j.get("h"), j.get("u"), j.get("save_u", False))
        if T > 16:
            raise ValueError(f"job {i}: T = {T}; the grouped forward takes T <= 16")
        if dev is None:
            dev = w.codes.device
        elif w.codes.device != dev:
            raise ValueError(f"job {i} is on {w.codes.device}, job 0 on {dev}")
        args.append((w, j["x"], T, j.get("A"), j.get("B"), r, float(j["alpha"]), h, u))
        outs.append((h, u))
    _check_independent(args)
    nbytes = qlora_forward_many_workspace_bytes(len(jobs))
    if ws is None:
        ws = workspace(dev, nbytes)
    else:
        _own_workspace(ws, nbytes)
        _check_devices(dev, ws=ws)
    cws = [a[0]._c() for a in args]  # kept alive for the call
    arr = (_ForwardJob * len(args))()
    for k, (a, cw) in enumerate(zip(args, cws)):
        w, x, T, A, B, r, alpha, h, u = a
        arr[k] = _ForwardJob(ctypes.pointer(cw), _ptr(x), T, _ptr(A), _ptr(B), r, alpha, _ptr(h), _ptr(u))
    _check(_lib.qlora_forward_many(arr, len(args), _ptr(ws), ws.numel(), _stream(dev)), "qlora_forward_many")
    return outs


def qlora_forward_noalloc(w: NF4Weight, x: torch.Tensor, A: torch.Tensor | None, B: torch.Tensor | None,
                          alpha: float, h: torch.Tensor, u: torch.Tensor | None = None):
    """qlora_forward for T <= 16 on the library's static per-GPU scratch array instead of a workspace: no
    allocation in the library or here (h, and u when wanted, are the caller's). Calls that overlap on one GPU
    share the array and must be serialized by the caller."""
    if h is None:
        raise ValueError("qlora_forward_noalloc writes into a given h (it allocates nothing)")
    T, r, h, u = _forward_args(w, x, A, B, h, u, False)
    cw = w._c()
    _check(_lib.qlora_forward_noalloc(ctypes.byref(cw), _ptr(x), T, _ptr(A), _ptr(B), r, alpha, _ptr(h), _ptr(u),
                                      _stream(x.device)), "qlora_forward_noalloc")
    return h, u


def qlora_workspace_fallbacks(ws: torch.Tensor) -> int:
    """How many waits on this workspace ran out of time and took their fallback path (the results are the same;
    a nonzero count means launches on other streams held the compute units). Synchronizes the current stream."""
    _own_workspace(ws, COUNTER_BYTES)
    _check_devices(ws.device)
    n = ctypes.c_uint32(0)
    _check(_lib.qlora_workspace_fallbacks(_ptr(ws), ctypes.byref(n), _stream(ws.device)), "qlora_workspace_fallbacks")
    return int(n.value)


def qlora_workspace_set_wait_limit(ws: torch.Tensor, ticks: int) -> None:
    """A testing aid: later calls on this workspace give up a wait after `ticks` ticks of the 100 MHz clock and
    take the fallback path (1 sends every wait that does not succeed at once there); 0 restores the built-in
    limit. Synchronizes the current stream."""
    _own_workspace(ws, COUNTER_BYTES)
    _check_devices(ws.device)
    if not 0 <= int(ticks) < 1 << 32:
        raise ValueError("ticks must fit in 32 bits")
    _check(_lib.qlora_workspace_set_wait_limit(_ptr(ws), int(ticks), _stream(ws.device)),
           "qlora_workspace_set_wait_limit")


def qlora_backward(w: NF4Weight, x: torch.Tensor | None, dY: torch.Tensor, A: torch.Tensor | None,
                   B: torch.Tensor | None, alpha: float, u_saved: torch.Tensor | None = None,
                   need_dx: bool = True, need_dA: bool = True, need_dB: bool = True,
                   dX: torch.Tensor | None = None, dA: torch.Tensor | None = None, dB: torch.Tensor | None = None,
                   ws: torch.Tensor | None = None):
    """Returns (dX bf16 [T, d_in] | None, dA f32 [r, d_in] | None, dB f32 [d_out, r] | None).

    Outputs passed in are written in place (and count as needed); the others are allocated when needed.
    """
    _check_weight(w)
    if not torch.is_tensor(dY) or dY.dim() != 2:
        raise ValueError("dY must be a 2-D [T, d_out] tensor")
    T = dY.shape[0]
    _arg(dY, "dY", torch.bfloat16, (T, w.d_out))
    _arg(x, "x", torch.bfloat16, (T, w.d_in))
    r = _adapter_rank(w, A, B)
    if r == 0 and (dA is not None or dB is not None or u_saved is not None):
        raise ValueError("dA, dB and u_saved need an adapter")
    _arg(u_saved, "u_saved", torch.float32, (T, r))
    _arg(dX, "dX", torch.bfloat16, (T, w.d_in))
    _arg(dA, "dA", torch.float32, (r, w.d_in))
    _arg(dB, "dB", torch.float32, (w.d_out, r))
    nbytes = qlora_workspace_bytes(w.d_out, w.d_in, T, r)
    if ws is not None:
        _own_workspace(ws, nbytes)
    _check_no_overlap({"x": x, "dY": dY, "A": A, "B": B, "u_saved": u_saved, "codes": w.codes, "qscale": w.qscale,
                       "smax": w.smax}, {"dX": dX, "dA": dA, "dB": dB, "ws": ws})
    dev = w.codes.device
    _check_devices(dev, qscale=w.qscale, smax=w.smax, x=x, dY=dY, A=A, B=B, u_saved=u_saved, dX=dX, dA=dA, dB=dB,
                   ws=ws)
    if dX is None and need_dx:
        dX = torch.empty(T, w.d_in, dtype=torch.bfloat16, device=dev)
    if dA is None and need_dA and r > 0:
        dA = torch.empty(r, w.d_in, dtype=torch.float32, device=dev)
    if dB is None and need_dB and r > 0:
        dB = torch.empty(w.d_out, r, dtype=torch.float32, device=dev)
    ws = workspace(dev, nbytes) if ws is None else ws
    cw = w._c()
    _check(_lib.qlora_backward(ctypes.byref(cw), _ptr(x), _ptr(dY), T, _ptr(A), _ptr(B), r, alpha, _ptr(u_saved),
                               _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws), ws.numel(), _stream(dev)), "qlora_backward")
    return dX, dA, dB
