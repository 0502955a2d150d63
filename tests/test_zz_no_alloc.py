"""qlora_forward_noalloc: the T <= 16 forward on the library's static per-GPU scratch array, for callers that
cannot allocate. Through the C ABI, two calls in a row (the second smaller) give bit for bit what qlora_forward
gives with a workspace; a call with T > 16 is refused before anything is enqueued."""

import ctypes
import os

import pytest
import torch

from bit_quantized_finetuning_amd import build as _build

if not os.path.exists(_build.LIB):  # hipcc cross-compiles for gfx950 without a GPU
    _build.build()
from bit_quantized_finetuning_amd import qlora as q  # noqa: E402

ERR_SCRATCH = -10


def test_call_beyond_the_static_array_is_refused_before_launch():
    # T > 16 (the tiled path) is refused; fake, aligned, never dereferenced pointers: validation runs on the
    # host and returns before any HIP call.
    fake = 1 << 20
    for d_out, d_in, T, r in ((1024, 1024, 17, 8), (8192, 22016, 4096, 64)):
        w = q._Nf4Weight(d_out, d_in, fake, fake, fake)
        st = q.lib.qlora_forward_noalloc(ctypes.byref(w), ctypes.c_void_p(fake), T, ctypes.c_void_p(fake),
                                         ctypes.c_void_p(fake), r, 16.0, ctypes.c_void_p(fake), None, None)
        assert st == ERR_SCRATCH
    assert "static" in q.qlora_status_string(ERR_SCRATCH)
    # a bad argument is reported as for qlora_forward
    w = q._Nf4Weight(1024, 1024, fake, fake, fake)
    assert q.lib.qlora_forward_noalloc(ctypes.byref(w), None, 4, None, None, 0, 16.0, ctypes.c_void_p(fake), None,
                                       None) == -1


def _inputs(gen, d_out, d_in, T, r):
    W = torch.randn(d_out, d_in, device="cuda", generator=gen) * 0.02
    w = q.qlora_quantize(W)
    x = torch.randn(T, d_in, device="cuda", generator=gen).to(torch.bfloat16)
    A = (torch.randn(r, d_in, device="cuda", generator=gen) * 0.02).to(torch.bfloat16) if r else None
    B = (torch.randn(d_out, r, device="cuda", generator=gen) * 0.02).to(torch.bfloat16) if r else None
    return w, x, A, B


@pytest.mark.gpu
@pytest.mark.parametrize("first,second", [
    ((4096, 4096, 16, 64), (1024, 1024, 4, 8)),       # a LLaMA-7B projection, then a smaller call
])
def test_noalloc_forward_matches_workspace_forward(first, second):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(21)
    for d_out, d_in, T, r in (first, second):
        print(f"noalloc forward {d_out}x{d_in} T={T} r={r}", flush=True)
        w, x, A, B = _inputs(gen, d_out, d_in, T, r)
        h_ref, u_ref = q.qlora_forward(w, x, A, B, 16.0, save_u=True)
        h = torch.full((T, d_out), float("nan"), dtype=torch.bfloat16, device="cuda")
        u = torch.full((T, r), float("nan"), dtype=torch.float32, device="cuda")
        q.qlora_forward_noalloc(w, x, A, B, 16.0, h, u)
        torch.cuda.synchronize()
        assert torch.equal(h.view(torch.int16), h_ref.view(torch.int16))
        assert torch.equal(u, u_ref)
        # base only (no adapter) through the same array
        h0_ref, _ = q.qlora_forward(w, x, None, None, 16.0)
        h0 = torch.empty_like(h0_ref)
        q.qlora_forward_noalloc(w, x, None, None, 16.0, h0)
        torch.cuda.synchronize()
        assert torch.equal(h0.view(torch.int16), h0_ref.view(torch.int16))
