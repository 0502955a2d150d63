"""The Python binding checks every tensor argument before it calls the C ABI (which sees only pointers): shape
against the weight and the other operands, dtype, contiguity, and the device last. Each case here fails one rule
and raises before anything is launched; CPU tensors with every other rule met reach the device check. No GPU is
needed. Also the layer modules' handling of dtype casts (their storage and adapters keep their dtypes)."""

import os

import pytest
import torch

from bit_quantized_finetuning_amd import build as _build

if not os.path.exists(_build.LIB):  # hipcc cross-compiles for gfx950 without a GPU
    _build.build()
from bit_quantized_finetuning_amd import layer  # noqa: E402
from bit_quantized_finetuning_amd import qlora as q  # noqa: E402

D_OUT, D_IN, T, R = 64, 128, 5, 8


def bf(*shape):
    return torch.zeros(*shape, dtype=torch.bfloat16)


def f32(*shape):
    return torch.zeros(*shape, dtype=torch.float32)


@pytest.fixture
def w():
    return q.NF4Weight.empty(D_OUT, D_IN, "cpu")


def _raises(exc, match, fn, *a, **k):
    with pytest.raises(exc, match=match):
        fn(*a, **k)


def test_forward_checks(w):
    x, A, B = bf(T, D_IN), bf(R, D_IN), bf(D_OUT, R)
    _raises(ValueError, "x must have shape", q.qlora_forward, w, bf(T, D_IN + 64), A, B, 16.0)
    _raises(TypeError, "x must be torch.bfloat16", q.qlora_forward, w, f32(T, D_IN), A, B, 16.0)
    _raises(ValueError, "x must be contiguous", q.qlora_forward, w, bf(D_IN, T).t(), A, B, 16.0)
    _raises(ValueError, "A must have shape", q.qlora_forward, w, x, bf(R, D_IN + 64), B, 16.0)
    # B given transposed has the right element count but the wrong shape
    _raises(ValueError, "B must have shape", q.qlora_forward, w, x, A, bf(R, D_OUT), 16.0)
    _raises(ValueError, "both A and B", q.qlora_forward, w, x, A, None, 16.0)
    _raises(ValueError, "rank", q.qlora_forward, w, x, bf(12, D_IN), bf(D_OUT, 12), 16.0)
    _raises(ValueError, "h must have shape", q.qlora_forward, w, x, A, B, 16.0, h=bf(T, D_OUT + 16))
    _raises(TypeError, "h must be torch.bfloat16", q.qlora_forward, w, x, A, B, 16.0, h=f32(T, D_OUT))
    _raises(ValueError, "u must have shape", q.qlora_forward, w, x, A, B, 16.0, u=f32(T, R + 8))
    _raises(TypeError, "u must be torch.float32", q.qlora_forward, w, x, A, B, 16.0, u=bf(T, R))
    _raises(ValueError, "no adapter", q.qlora_forward, w, x, None, None, 16.0, u=f32(T, 8))
    _raises(ValueError, "ws must be a contiguous uint8", q.qlora_forward, w, x, A, B, 16.0,
            ws=torch.zeros(16, dtype=torch.uint8))
    _raises(ValueError, "ws must be a contiguous uint8", q.qlora_forward, w, x, A, B, 16.0,
            ws=torch.zeros(1 << 24, dtype=torch.int8))
    # every shape right: the device rule is what stops a CPU call
    _raises(ValueError, "must be on a GPU", q.qlora_forward, w, x, A, B, 16.0)
    _raises(ValueError, "must be on a GPU", q.qlora_forward, w, x, None, None, 16.0)


def test_outputs_must_not_alias_inputs(w):
    A, B = bf(R, D_IN), bf(D_OUT, R)
    buf = bf(T * (D_IN + D_OUT))
    x, dY = buf[: T * D_IN].view(T, D_IN), buf[T * D_IN:].view(T, D_OUT)
    _raises(ValueError, "h overlaps x", q.qlora_forward, w, x, A, B, 16.0,
            h=buf[T * 64:T * (64 + D_OUT)].view(T, D_OUT))
    _raises(ValueError, "h overlaps x", q.qlora_forward_noalloc, w, x, A, B, 16.0, h=buf[:T * D_OUT].view(T, D_OUT))
    hb = bf(T * D_OUT + 8)
    _raises(ValueError, "h overlaps u|u overlaps h", q.qlora_forward, w, x, A, B, 16.0,
            h=hb[:T * D_OUT].view(T, D_OUT), u=hb.view(torch.float32)[:T * R].view(T, R))
    _raises(ValueError, "dX overlaps dY", q.qlora_backward, w, bf(T, D_IN), dY, A, B, 16.0,
            dX=buf[T * D_OUT:].view(T, D_IN))
    uf = f32(T * R + D_OUT * R)
    _raises(ValueError, "dB overlaps u_saved", q.qlora_backward, w, bf(T, D_IN), bf(T, D_OUT), A, B, 16.0,
            u_saved=uf[:T * R].view(T, R), dB=uf[T * R - 8:T * R - 8 + D_OUT * R].view(D_OUT, R))
    # disjoint views of one buffer are fine: the device rule is what stops a CPU call
    _raises(ValueError, "must be on a GPU", q.qlora_forward, w, x, A, B, 16.0, h=dY)
    _raises(ValueError, "must be on a GPU", q.qlora_backward, w, x, dY, A, B, 16.0, u_saved=uf[:T * R].view(T, R),
            dB=uf[T * R:].view(D_OUT, R))


def test_backward_checks(w):
    x, dY, A, B = bf(T, D_IN), bf(T, D_OUT), bf(R, D_IN), bf(D_OUT, R)
    _raises(ValueError, "dY must have shape", q.qlora_backward, w, x, bf(T, D_OUT + 16), A, B, 16.0)
    _raises(ValueError, "x must have shape", q.qlora_backward, w, bf(T + 1, D_IN), dY, A, B, 16.0)
    _raises(TypeError, "x must be torch.bfloat16", q.qlora_backward, w, f32(T, D_IN), dY, A, B, 16.0)
    _raises(ValueError, "x must be contiguous", q.qlora_backward, w, bf(D_IN, T).t(), dY, A, B, 16.0)
    _raises(ValueError, "B must have shape", q.qlora_backward, w, x, dY, A, bf(R, D_OUT), 16.0)
    _raises(ValueError, "u_saved must have shape", q.qlora_backward, w, x, dY, A, B, 16.0, u_saved=f32(T, R + 8))
    _raises(TypeError, "u_saved must be torch.float32", q.qlora_backward, w, x, dY, A, B, 16.0, u_saved=bf(T, R))
    _raises(ValueError, "dX must have shape", q.qlora_backward, w, x, dY, A, B, 16.0, dX=bf(T, D_OUT))
    _raises(ValueError, "dA must have shape", q.qlora_backward, w, x, dY, A, B, 16.0, dA=f32(D_IN, R))
    _raises(TypeError, "dB must be torch.float32", q.qlora_backward, w, x, dY, A, B, 16.0, dB=bf(D_OUT, R))
    _raises(ValueError, "need an adapter", q.qlora_backward, w, x, dY, None, None, 16.0, dA=f32(R, D_IN))
    _raises(ValueError, "must be on a GPU", q.qlora_backward, w, x, dY, A, B, 16.0)
    _raises(ValueError, "must be on a GPU", q.qlora_backward, w, None, dY, A, B, 16.0, u_saved=f32(T, R),
            need_dA=False)


def test_weight_and_other_entry_point_checks(w):
    bad = q.NF4Weight(D_OUT, D_IN, torch.zeros(D_OUT * D_IN // 4, dtype=torch.uint8), w.qscale, w.smax)
    _raises(ValueError, "codes must have shape", q.qlora_forward, bad, bf(T, D_IN), None, None, 16.0)
    bad = q.NF4Weight(D_OUT, D_IN, w.codes, w.qscale, w.smax.to(torch.bfloat16))
    _raises(TypeError, "smax must be torch.float32", q.qlora_dequantize, bad)
    absmax = q.NF4Weight.empty(D_OUT, D_IN, "cpu", double_quant=False)
    assert absmax.smax.numel() == D_OUT * D_IN // 64
    _raises(ValueError, "must be on a GPU", q.qlora_dequantize, absmax)
    _raises(ValueError, "out must have shape", q.qlora_merge, w, bf(R, D_IN), bf(D_OUT, R), 16.0,
            out=bf(D_IN, D_OUT))
    _raises(ValueError, "must be on a GPU", q.qlora_merge, w, bf(R, D_IN), bf(D_OUT, R), 16.0)
    _raises(ValueError, "out is", q.qlora_quantize, f32(D_OUT, D_IN + 64), out=w)
    _raises(TypeError, "flags", q.qlora_quantize, f32(D_OUT, D_IN), flags=torch.zeros(1, dtype=torch.int64))
    _raises(ValueError, "must be on a GPU", q.qlora_quantize, f32(D_OUT, D_IN))
    _raises(ValueError, "grad must be on a GPU", q.qlora_adamw_step, 1, f32(10), f32(10), f32(10), f32(10))
    _raises(ValueError, "same number", q.qlora_adamw_step, 1, f32(10), f32(10), f32(11), f32(10))
    _raises(ValueError, "ws must be a contiguous uint8", q.qlora_workspace_fallbacks, torch.zeros(8, dtype=torch.uint8))


class _Storage(layer._Bf16Module):
    def __init__(self):
        super().__init__()
        self.d_in, self.d_w_out = 64, 16
        self.register_buffer("codes", torch.arange(512, dtype=torch.int64).to(torch.uint8))
        self.register_buffer("qscale", torch.arange(16, dtype=torch.int64).to(torch.uint8))
        self.register_buffer("smax", torch.tensor([0.1234567], dtype=torch.float32))
        self.A = torch.nn.Parameter(torch.full((8, 64), 0.1, dtype=torch.bfloat16))


def test_dtype_casts_leave_storage_and_adapters_alone():
    m = _Storage()
    s0 = m.smax.clone()
    for cast in (lambda t: t.to(torch.bfloat16), lambda t: t.half(), lambda t: t.double(), lambda t: t.float()):
        cast(m)
        assert m.smax.dtype == torch.float32 and torch.equal(m.smax.view(torch.int32), s0.view(torch.int32))
        assert m.codes.dtype == torch.uint8 and m.A.dtype == torch.bfloat16
        assert isinstance(m.A, torch.nn.Parameter)
    # the weight the library is given is built from the registered buffers (so it follows moves and loads)
    w = m.w
    assert w.smax is m.smax and w.codes is m.codes and (w.d_out, w.d_in) == (16, 64)
    sd = m.state_dict()
    m2 = _Storage()
    m2.smax.fill_(0.5)
    m2.load_state_dict(sd)
    assert torch.equal(m2.w.smax, s0)


def test_grouped_forward_checks(w):
    x, A, B = bf(T, D_IN), bf(R, D_IN), bf(D_OUT, R)
    _raises(ValueError, "between 1 and", q.qlora_forward_many, [])
    _raises(ValueError, "between 1 and", q.qlora_forward_many, [{}] * (q.MAX_FORWARD_JOBS + 1))
    # the jobs of one launch run at the same time: outputs may not overlap any job's inputs or outputs
    x1 = bf(T, D_IN)
    ok = [(w, x, T, A, B, R, 16.0, bf(T, D_OUT), f32(T, R)), (w, x1, T, A, B, R, 16.0, bf(T, D_OUT), None)]
    q._check_independent(ok)  # a weight and adapters shared between jobs are inputs only
    over_x = x1.view(-1)[:T * D_OUT].view(T, D_OUT)  # job 0's h inside job 1's x
    _raises(ValueError, "overlaps job 1's x", q._check_independent,
            [(w, x, T, A, B, R, 16.0, over_x, None), (w, x1, T, A, B, R, 16.0, bf(T, D_OUT), None)])
    hh = bf(2 * T, D_OUT)
    _raises(ValueError, "overlaps job 1's h", q._check_independent,
            [(w, x, T, A, B, R, 16.0, hh[:T], None), (w, x1, T, A, B, R, 16.0, hh[T - 1:2 * T - 1], None)])
    own = x.view(-1)[:T * D_OUT].view(T, D_OUT)  # a job's h over its own x
    _raises(ValueError, "overlaps job 0's x", q._check_independent, [(w, x, T, A, B, R, 16.0, own, None)])
