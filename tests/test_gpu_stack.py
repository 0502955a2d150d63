"""Chained decoder layers of QLoRA projections under gradient checkpointing (needs an MI355X).

The setting of "8GB, 12GB, 16GB, 24GB GPU에서 몇 B 모델까지 LoRA 학습이 될까", section "무엇을 돌렸나": the
14B-style stack (40 layers, hidden 5120, MLP 17408, k/v 1024 wide), LoRA r=8 alpha=16 on q and v, 2048 tokens,
gradient checkpointing. One forward + backward runs through the whole chain; for chosen layers, hooks keep each
library call's actual bf16 input and output and the upstream gradient of the q/k/v call, and the oracle recomputes
from exactly those:
  * packed codes, scale codes and group maxima of the stacked q/k/v weight, bit for bit (o, gate/up and down on
    row slices that start on a double-quant group boundary);
  * q/k/v outputs (each projection with its own adapter or none), and the o, gate/up and down outputs;
  * dX of the q/k/v call (the sum over the three projections), and the float32 dA, dB of the q and v adapters;
  * the recomputed forward of the backward pass gives the first forward's q/k/v output bit for bit.
A small stack (3 layers, ragged token count) is checked in full; the 40-layer stack on sampled blocks.
"""

import numpy as np
import pytest
import torch

import oracle
from bit_quantized_finetuning_amd import synth
from gpu_common import assert_close, say, product

pytestmark = pytest.mark.gpu

stack_mod = product("stack")

R, ALPHA = 8, 16.0
SMALL = {"q": (256, 256), "k": (64, 256), "v": (64, 256), "o": (256, 256), "gate": (384, 256), "up": (384, 256),
         "down": (256, 384)}


def _np(t):
    return t.detach().float().cpu().numpy()


def _build(layers, shapes, head, T, seed):
    dev = torch.device("cuda:0")
    st = stack_mod.DecoderStack(layers=layers, shapes=shapes, r=R, alpha=ALPHA, seed=seed, device=dev,
                                checkpoint=True, head=head)
    gen = torch.Generator(device=dev)
    gen.manual_seed(4242 + seed)
    with torch.no_grad():  # B starts at zero; give it values so that the adapter term is exercised
        for layer in st.layers:
            for B in layer.qkv.B:
                B.copy_((torch.randn(B.shape, device=dev, generator=gen) * 0.02).to(torch.bfloat16))
    x0 = (torch.randn(T, shapes["q"][1], device=dev, generator=gen)).to(torch.bfloat16).requires_grad_(True)
    dy = (torch.randn(T, shapes["q"][1], device=dev, generator=gen)).to(torch.bfloat16)
    return st, x0, dy


def _capture(st, idx):
    """Forward hooks that keep, on each chosen layer's first forward, every call's input and output, and register
    gradient hooks on the q/k/v call's input and outputs; the recomputed q/k/v output is kept apart."""
    rec = {i: {"dy": [None, None, None]} for i in idx}
    handles = []
    for i in idx:
        r = rec[i]
        lay = st.layers[i]
        for name in ("qkv", "o", "gate_up", "down"):
            def hook(m, inp, out, name=name, r=r):
                outs = out if isinstance(out, tuple) else (out,)
                h = torch.cat([o.detach() for o in outs], 1).clone()
                if name + "_x" in r:
                    if name == "qkv":
                        r["qkv_h_again"] = h
                    return
                r[name + "_x"] = inp[0].detach().clone()
                r[name + "_h"] = h
                if name == "qkv":
                    for j, o in enumerate(outs):
                        o.register_hook(lambda g, j=j: r["dy"].__setitem__(j, g.detach().clone()))
                    inp[0].register_hook(lambda g: r.__setitem__("dx", g.detach().clone()))
            handles.append(getattr(lay, name).register_forward_hook(hook))
    return rec, handles


def _rows_quantized(W_np, rows):
    """Oracle quantize of the row slice [rows.start, rows.stop) (aligned to whole double-quant groups)."""
    Ws = W_np[rows]
    codes, q2, S = oracle.quantize(Ws)
    return (codes, q2, S), oracle.dequantize(codes, q2, S, Ws.shape[0], Ws.shape[1])[1]


def _check_slice_codes(mod, rows, d_in, ref):
    codes, q2, S = ref
    n0, n1 = rows.start * d_in, rows.stop * d_in
    assert n0 % (64 * 256) == 0 and n1 % (64 * 256) == 0, "slice must cover whole groups"
    assert np.array_equal(mod.codes.cpu().numpy()[n0 // 2:n1 // 2], codes), "packed codes differ"
    assert np.array_equal(mod.qscale.cpu().numpy()[n0 // 64:n1 // 64], q2), "scale codes differ"
    assert np.array_equal(mod.smax.cpu().numpy().view(np.uint32)[n0 // 16384:n1 // 16384], S.view(np.uint32)), \
        "group maxima differ"


def _check_layer(st, i, r, shapes, rng, full):
    lay = st.layers[i]
    ws = synth.stack_layer_weights(i, torch.device("cuda:0"), shapes, st.seed)
    W = {k: _np(v) for k, v in ws.items()}
    del ws
    T = r["qkv_x"].shape[0]
    ts = np.arange(T) if full else np.sort(rng.choice(T, 64, replace=False))

    # q/k/v: the whole stacked weight bit for bit
    Wqkv = np.concatenate([W["q"], W["k"], W["v"]], 0)
    codes, q2, S = oracle.quantize(Wqkv)
    assert np.array_equal(lay.qkv.codes.cpu().numpy(), codes), f"layer {i}: q/k/v packed codes differ"
    assert np.array_equal(lay.qkv.qscale.cpu().numpy(), q2), f"layer {i}: q/k/v scale codes differ"
    assert np.array_equal(lay.qkv.smax.cpu().numpy().view(np.uint32), S.view(np.uint32)), \
        f"layer {i}: q/k/v group maxima differ"
    _, wb = oracle.dequantize(codes, q2, S, *Wqkv.shape)
    dq, dk = W["q"].shape[0], W["k"].shape[0]
    spans = {"q": (0, dq), "k": (dq, dq + dk), "v": (dq + dk, Wqkv.shape[0])}
    ad = {"q": (_np(lay.qkv.A[0]), _np(lay.qkv.B[0]), lay.qkv.A[0], lay.qkv.B[0]),
          "v": (_np(lay.qkv.A[1]), _np(lay.qkv.B[1]), lay.qkv.A[1], lay.qkv.B[1])}

    x = _np(r["qkv_x"])
    h = _np(r["qkv_h"])
    dys = [_np(g) for g in r["dy"]]
    assert all(g is not None for g in r["dy"]), "q/k/v upstream gradients were not captured"
    assert torch.equal(r["qkv_h_again"].view(torch.int16), r["qkv_h"].view(torch.int16)), \
        f"layer {i}: the recomputed q/k/v output differs from the first forward's"
    d_in = x.shape[1]
    is_ = np.arange(d_in) if full else np.sort(rng.choice(d_in, 64, replace=False))
    dX_ref = np.zeros((ts.size, is_.size))
    for j, name in enumerate(("q", "k", "v")):
        a0, a1 = spans[name]
        wbp, dyp = wb[a0:a1], dys[j]
        os_ = np.arange(a1 - a0) if full else np.sort(rng.choice(a1 - a0, 64, replace=False))
        A, B, Ap, Bp = ad.get(name, (None, None, None, None))
        rr = R if A is not None else 0
        h_ref, _ = oracle.lora_forward(wbp[os_], x[ts], A, None if B is None else B[os_], ALPHA, rr)
        assert_close(f"layer {i} {name} output", h[ts][:, a0 + os_], h_ref)
        dX_ref += oracle.lora_backward(wbp[:, is_], x[ts][:, is_], dyp[ts], None if A is None else A[:, is_], B,
                                       ALPHA, rr)[0]
        if A is not None:
            _, dA_ref, _ = oracle.lora_backward(wbp[:, is_], x[:, is_], dyp, A[:, is_], B, ALPHA, rr)
            assert_close(f"layer {i} dA_{name}", Ap.grad_fp32[:, is_], dA_ref)
            _, _, dB_ref = oracle.lora_backward(wbp[os_], x, dyp[:, os_], A, B[os_], ALPHA, rr)
            assert_close(f"layer {i} dB_{name}", Bp.grad_fp32[os_], dB_ref)
            assert torch.equal(Ap.grad_fp32.to(torch.bfloat16).view(torch.int16), Ap.grad.view(torch.int16))
    assert_close(f"layer {i} q/k/v dX", r["dx"][ts][:, is_], dX_ref)

    # o, gate/up, down: frozen, base term only
    for name, parts in (("o", ("o",)), ("gate_up", ("gate", "up")), ("down", ("down",))):
        Wm = np.concatenate([W[p] for p in parts], 0)
        mod = getattr(lay, name)
        xm, hm = _np(r[name + "_x"]), _np(r[name + "_h"])
        if full:
            rows = slice(0, Wm.shape[0])
        else:
            n0 = 16 * int(rng.integers(0, (Wm.shape[0] - 64) // 16 + 1))
            rows = slice(n0, n0 + 64)
        ref, wbm = _rows_quantized(Wm, rows)
        if full:
            assert np.array_equal(mod.codes.cpu().numpy(), ref[0]), f"layer {i}: {name} codes differ"
            assert np.array_equal(mod.qscale.cpu().numpy(), ref[1]), f"layer {i}: {name} scale codes differ"
            assert np.array_equal(mod.smax.cpu().numpy().view(np.uint32), ref[2].view(np.uint32))
        else:
            _check_slice_codes(mod, rows, Wm.shape[1], ref)
        h_ref, _ = oracle.lora_forward(wbm, xm[ts], None, None, ALPHA, 0)
        assert_close(f"layer {i} {name} output", hm[ts][:, rows], h_ref)


def _run(layers, shapes, head, T, idx, full, seed):
    st, x0, dy = _build(layers, shapes, head, T, seed)
    rec, handles = _capture(st, idx)
    out = st(x0)
    out.backward(dy)
    torch.cuda.synchronize()
    for hd in handles:
        hd.remove()
    assert torch.isfinite(out.float()).all(), "non-finite output at the end of the stack"
    rng = np.random.default_rng([17, layers, T])
    for i in idx:
        say(f"  layer {i}")
        _check_layer(st, i, rec[i], shapes, rng, full)
    return st


def test_small_stack_three_layers_in_full():
    """3 layers (hidden 256, k/v 64, MLP 384, head 64), 100 tokens: every value of every call."""
    say("stack 3 x 256, T=100, checkpointing")
    _run(3, SMALL, 64, 100, [0, 1, 2], full=True, seed=1)


def test_small_stack_checkpointing_changes_nothing():
    """The same stack with and without gradient checkpointing: identical outputs and adapter gradients."""
    say("stack 3 x 256, checkpointing on / off")
    res = []
    for ck in (True, False):
        st, x0, dy = _build(3, SMALL, 64, 100, seed=2)
        st.use_checkpoint = ck
        out = st(x0)
        out.backward(dy)
        torch.cuda.synchronize()
        res.append((out.detach().clone(), [p.grad_fp32.clone() for lay in st.layers for p in
                                          list(lay.qkv.A) + list(lay.qkv.B)], x0.grad.clone()))
    (o1, g1, x1), (o2, g2, x2) = res
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(x1.view(torch.int16), x2.view(torch.int16))
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_14b_stack_forty_layers_2048_tokens():
    """The 40-layer 14B-style stack, 2048 tokens: layers 0, 19 and 39 on sampled blocks."""
    say("14B-style stack, 40 layers, T=2048, checkpointing")
    _run(40, synth.STACK_SHAPES, 128, 2048, [0, 19, 39], full=False, seed=0)
