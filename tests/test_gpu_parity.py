"""GPU parity of the HIP path against the CPU oracle (needs an MI355X).

Bit-exact: packed codes, scale codes, group maxima, restored weights (float32 and
bf16). Within tolerance (see gpu_common): h, dX, dA, dB. Shapes span several
tiles and ragged tails of every kernel: T in {1, 4, 16} takes the weight-streaming
kernel, larger T the MFMA GEMM; d_out not a multiple of the 64/256 row tiles;
d_in not a multiple of the 256-wide K segments; groups of 256 blocks that straddle
rows and a short last group.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import Case, assert_close, assert_within_one_bf16_ulp, bits_to_bf16, merge_float32_slack, say, product

pytestmark = pytest.mark.gpu

q = product("qlora")


def _quantize_and_compare(case):
    d = case.device_inputs()
    w = q.qlora_quantize(d["W"])
    torch.cuda.synchronize()
    codes, q2, S, w32, wb = case.oracle_quant()
    assert np.array_equal(w.codes.cpu().numpy(), codes), "packed codes differ"
    assert np.array_equal(w.qscale.cpu().numpy(), q2), "scale codes differ"
    assert np.array_equal(w.smax.cpu().numpy().view(np.uint32), S.view(np.uint32)), "group maxima differ"
    return w, d


# ---------------------------------------------------------------------------
# quantize / dequantize: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d_out,d_in,wdtype", [
    (1024, 1024, "f32"),     # single-linear workload
    (16, 64, "f32"),         # smallest legal weight: one block per row, one short group
    (48, 192, "f32"),
    (80, 320, "f32"),        # 400 blocks: groups straddle rows, short last group
    (32, 5120, "bf16"),      # bf16 weights, 80 blocks per row
    (4096, 4096, "f32"),     # LLaMA-7B q_proj shape
])
def test_quantize_bit_exact(d_out, d_in, wdtype):
    say(f"quantize {d_out}x{d_in} {wdtype}")
    _quantize_and_compare(Case(d_out, d_in, 0, 1, cfg=101, wdtype=wdtype))


def test_quantize_adversarial_blocks():
    """Midpoint ties and their float32 neighbours, zero blocks, an outlier group, all-negative blocks."""
    say("quantize adversarial")
    mids = oracle.nf4_midpoints_f64()
    vals = []
    for m in mids:
        f = np.float32(m)
        vals += [f, np.nextafter(f, np.float32(-1)), np.nextafter(f, np.float32(1))]
        vals += [-f, np.nextafter(-f, np.float32(-1)), np.nextafter(-f, np.float32(1))]
    vals = np.array(vals, dtype=np.float32)
    rows = []
    for i in range(0, vals.size, 63):
        blk = np.zeros(64, dtype=np.float32)
        chunk = vals[i:i + 63]
        blk[:chunk.size] = chunk
        blk[63] = 1.0                       # absmax 1 -> w/s == w exactly
        rows.append(blk)
    W = np.zeros((16, 64 * 8), dtype=np.float32)
    flat = np.concatenate(rows)
    W.reshape(-1)[:flat.size] = flat
    W[5, :] = 0.0                           # zero blocks
    W[6, :64] = -np.abs(np.linspace(0.01, 0.5, 64, dtype=np.float32))
    W[9, :] = 1e-3
    W[9, 70] = 10.0                         # outlier: small blocks of the group go to q2 = 0
    W[12, :64] = np.float32(1e-30)          # tiny (near-denormal ratios stay normal)
    case = Case(16, 512, 0, 1, cfg=102)
    case.W = W
    w, d = _quantize_and_compare(case)
    out = q.qlora_dequantize(w, torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), case.oracle_quant()[3].view(np.uint32))


@pytest.mark.parametrize("d_out,d_in", [(1024, 1024), (80, 320), (272, 5120)])
def test_dequantize_bit_exact(d_out, d_in):
    say(f"dequantize {d_out}x{d_in}")
    case = Case(d_out, d_in, 0, 1, cfg=103)
    w, _ = _quantize_and_compare(case)
    o32 = q.qlora_dequantize(w, torch.float32)
    ob = q.qlora_dequantize(w, torch.bfloat16)
    torch.cuda.synchronize()
    _, _, _, w32, wb = case.oracle_quant()
    assert np.array_equal(o32.cpu().numpy().view(np.uint32), w32.view(np.uint32)), "float32 restore differs"
    assert np.array_equal(ob.float().cpu().numpy().view(np.uint32), wb.view(np.uint32)), "bf16 restore differs"


def test_quantize_flags_non_finite():
    say("quantize non-finite flag")
    W = torch.zeros(16, 64, device="cuda")
    W[3, 7] = float("inf")
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    q.qlora_quantize(W, flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) & 1
    flags.zero_()
    q.qlora_quantize(torch.ones(16, 64, device="cuda"), flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0


@pytest.mark.parametrize("wdtype", ["bf16", "f32"])
def test_quantize_many_equals_single_calls(wdtype):
    """qlora_quantize_many over 37 weights (two launches: 32 jobs, then 5) of mixed shapes, groups that straddle
    rows, short last groups, both storages mixed, gives the same bits as one qlora_quantize per weight; one
    weight is also checked against the oracle."""
    say(f"quantize_many {wdtype}")
    dt = torch.bfloat16 if wdtype == "bf16" else torch.float32
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2024)
    shapes = [(16, 64), (48, 192), (80, 320), (1024, 5120), (5120, 1024), (272, 5120), (32, 5120), (16, 16384)]
    Ws, dq = [], []
    for i in range(37):
        d_out, d_in = shapes[i % len(shapes)]
        Ws.append((torch.randn(d_out, d_in, device="cuda", generator=gen) * (0.02 * (1 + i % 3))).to(dt))
        dq.append(i % 5 != 3)  # every fifth weight in absmax-only storage
    outs = [q.NF4Weight.empty(W.shape[0], W.shape[1], W.device, d) for W, d in zip(Ws, dq)]
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = q.qlora_quantize_many(Ws, outs, flags=flags)
    ref = [q.qlora_quantize(W, double_quant=d) for W, d in zip(Ws, dq)]
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    for i, (a, b) in enumerate(zip(got, ref)):
        assert torch.equal(a.codes, b.codes), f"weight {i}: codes differ"
        assert (a.qscale is None) == (b.qscale is None)
        if a.qscale is not None:
            assert torch.equal(a.qscale, b.qscale), f"weight {i}: scale codes differ"
        assert torch.equal(a.smax.view(torch.int32), b.smax.view(torch.int32)), f"weight {i}: scales differ"
    W2 = Ws[2].float().cpu().numpy()
    codes, q2, S = oracle.quantize(W2)[:3]
    assert np.array_equal(got[2].codes.cpu().numpy(), codes)
    assert np.array_equal(got[2].qscale.cpu().numpy(), q2)
    assert np.array_equal(got[2].smax.cpu().numpy().view(np.uint32), np.asarray(S, dtype=np.float32).view(np.uint32))
    # a non-finite weight in one job sets the shared flag
    Ws[30][1, 2] = float("inf")
    q.qlora_quantize_many(Ws[28:33], flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) & 1


# ---------------------------------------------------------------------------
# forward / backward: tolerance
# ---------------------------------------------------------------------------

SHAPES = [
    # d_out, d_in, r
    (1024, 1024, 8),      # single-linear workload shape
    (80, 192, 16),        # ragged rows / K segments
    (272, 320, 64),
    (16, 64, 0),          # base only, minimal
    (528, 1344, 256),     # maximum rank
]
TOKENS = [1, 4, 16, 17, 100, 300]


@pytest.mark.parametrize("d_out,d_in,r", SHAPES)
@pytest.mark.parametrize("T", TOKENS)
def test_forward_parity(d_out, d_in, r, T):
    say(f"forward {d_out}x{d_in} r={r} T={T}")
    case = Case(d_out, d_in, r, T, cfg=104)
    w, d = _quantize_and_compare(case)
    h, u = q.qlora_forward(w, d["x"], d["A"], d["B"], case.alpha, save_u=True)
    torch.cuda.synchronize()
    h_ref, u_ref = case.oracle_forward()
    assert_close("h", h, h_ref)
    if r > 0:
        assert_close("u", u, u_ref)
    _assert_workspace_clean()


def _assert_workspace_clean():
    """After a call every counter is back to zero, and no wait ran out of time (the last word counts those)."""
    ws = q.workspace("cuda", 1 << 20)
    counters = ws[:q.COUNTER_BYTES].view(torch.int32)
    assert int(counters.abs().sum().item()) == 0, "counter region not reset (or a wait timed out)"


@pytest.mark.parametrize("d_out,d_in,r", SHAPES)
@pytest.mark.parametrize("T", [1, 16, 100, 300])
@pytest.mark.parametrize("saved_u", [True, False])
def test_backward_parity(d_out, d_in, r, T, saved_u):
    say(f"backward {d_out}x{d_in} r={r} T={T} saved_u={saved_u}")
    case = Case(d_out, d_in, r, T, cfg=105)
    w, d = _quantize_and_compare(case)
    u = None
    if saved_u and r > 0:
        _, u = q.qlora_forward(w, d["x"], d["A"], d["B"], case.alpha, save_u=True)
    dX, dA, dB = q.qlora_backward(w, d["x"], d["dY"], d["A"], d["B"], case.alpha, u_saved=u)
    torch.cuda.synchronize()
    dX_ref, dA_ref, dB_ref = case.oracle_backward()
    assert_close("dX", dX, dX_ref)
    if r > 0:
        assert_close("dA", dA, dA_ref)
        assert_close("dB", dB, dB_ref)
    else:
        assert dA is None and dB is None


@pytest.mark.parametrize("T", [4, 300])
def test_zero_B_gives_base_output_exactly(T):
    """B = 0: h is bit-identical to the adapter-free call (48GB page: B = 0 at init leaves the model unchanged)."""
    say(f"zero-B T={T}")
    case = Case(272, 320, 64, T, cfg=106)
    w, d = _quantize_and_compare(case)
    h0, _ = q.qlora_forward(w, d["x"], d["A"], torch.zeros_like(d["B"]), case.alpha)
    hb, _ = q.qlora_forward(w, d["x"], None, None, case.alpha)
    torch.cuda.synchronize()
    assert torch.equal(h0.view(torch.int16), hb.view(torch.int16))


def test_zero_weight_leaves_adapter_term():
    say("zero weight")
    case = Case(64, 128, 8, 20, cfg=107)
    case.W = np.zeros_like(case.W)
    w, d = _quantize_and_compare(case)
    assert int(w.codes.cpu().unique().numel()) == 1 and int(w.codes[0].item()) == 0x77
    h, _ = q.qlora_forward(w, d["x"], d["A"], d["B"], case.alpha)
    torch.cuda.synchronize()
    assert_close("h", h, case.oracle_forward()[0])


@pytest.mark.parametrize("T", [16, 300])
def test_no_gradient_into_weight(T):
    say(f"frozen weight T={T}")
    case = Case(272, 320, 64, T, cfg=108)
    w, d = _quantize_and_compare(case)
    before = (w.codes.clone(), w.qscale.clone(), w.smax.clone())
    q.qlora_forward(w, d["x"], d["A"], d["B"], case.alpha)
    q.qlora_backward(w, d["x"], d["dY"], d["A"], d["B"], case.alpha)
    torch.cuda.synchronize()
    assert torch.equal(before[0], w.codes) and torch.equal(before[1], w.qscale)
    assert torch.equal(before[2].view(torch.int32), w.smax.view(torch.int32))


@pytest.mark.parametrize("T", [16, 300])
def test_deterministic_reruns(T):
    say(f"determinism T={T}")
    case = Case(1024, 1024, 64, T, cfg=109)
    w, d = _quantize_and_compare(case)
    outs = []
    for _ in range(2):
        h, u = q.qlora_forward(w, d["x"], d["A"], d["B"], case.alpha, save_u=True)
        g = q.qlora_backward(w, d["x"], d["dY"], d["A"], d["B"], case.alpha, u_saved=u)
        torch.cuda.synchronize()
        outs.append([h.clone(), u.clone()] + [t.clone() for t in g])
    _assert_workspace_clean()
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def test_error_leaves_outputs_untouched():
    say("error path sentinel")
    case = Case(64, 128, 8, 4, cfg=110)
    w, d = _quantize_and_compare(case)
    h = torch.full((4, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    cw = w._c()
    import ctypes
    st = q.lib.qlora_forward(ctypes.byref(cw), d["x"].data_ptr(), 4, d["A"].data_ptr(), d["B"].data_ptr(), 8,
                             16.0, h.data_ptr(), None, q.workspace("cuda", 1 << 20).data_ptr(), 16, None)
    torch.cuda.synchronize()
    assert st == -4
    assert bool((h == 7.0).all())


def test_skinny_forward_call_sequence():
    """Back-to-back T <= 16 calls with changing adapters, ranks and shapes on one workspace: each
    result matches the oracle, so no call accepts the adapter intermediate of an earlier one."""
    seq = [(272, 320, 64, 16, 111), (272, 320, 64, 16, 112), (80, 192, 16, 4, 113), (272, 320, 64, 1, 114),
           (528, 1344, 256, 16, 115), (272, 320, 8, 16, 116)]
    for d_out, d_in, r, T, cfg in seq:
        say(f"sequence {d_out}x{d_in} r={r} T={T} cfg={cfg}")
        case = Case(d_out, d_in, r, T, cfg=cfg)
        w, d = _quantize_and_compare(case)
        h, u = q.qlora_forward(w, d["x"], d["A"], d["B"], case.alpha, save_u=True)
        torch.cuda.synchronize()
        h_ref, u_ref = case.oracle_forward()
        assert_close("h", h, h_ref)
        assert_close("u", u, u_ref)
    _assert_workspace_clean()


# ---------------------------------------------------------------------------
# LoRA-FA (A frozen): the backward without dA needs no layer input
# (GPU-fit page, "LoRA 변형을 바꿔도 답이 같은 이유": LoRA-FA keeps no layer input)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [16, 300])
def test_lora_fa_backward_needs_no_input(T):
    say(f"LoRA-FA backward T={T}")
    case = Case(272, 320, 64, T, cfg=117)
    w, d = _quantize_and_compare(case)
    _, u = q.qlora_forward(w, d["x"], d["A"], d["B"], case.alpha, save_u=True)
    dX, dA, dB = q.qlora_backward(w, None, d["dY"], d["A"], d["B"], case.alpha, u_saved=u, need_dA=False)
    torch.cuda.synchronize()
    assert dA is None
    dX_ref, _, dB_ref = case.oracle_backward()
    assert_close("dX", dX, dX_ref)
    assert_close("dB", dB, dB_ref)


# ---------------------------------------------------------------------------
# merge for export (48GB page, "QLoRA Puts the Two Methods in Different Places")
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d_out,d_in,r", [(1024, 1024, 8), (80, 320, 16), (272, 5120, 64), (528, 1344, 256),
                                          (16, 64, 8)])
def test_merge_parity(d_out, d_in, r):
    say(f"merge {d_out}x{d_in} r={r}")
    case = Case(d_out, d_in, r, 1, cfg=118)
    w, d = _quantize_and_compare(case)
    out = q.qlora_merge(w, d["A"], d["B"], case.alpha)
    torch.cuda.synchronize()
    wb = case.oracle_quant()[4]
    assert_within_one_bf16_ulp("merged", out, oracle.lora_merge(wb, case.A, case.B, case.alpha, r),
                               merge_float32_slack(wb, case.A, case.B, case.alpha, r))


def test_merge_without_adapter_is_the_restore():
    say("merge r=0 / B=0")
    case = Case(80, 320, 16, 1, cfg=119)
    w, d = _quantize_and_compare(case)
    wb = case.oracle_quant()[4]
    plain = q.qlora_merge(w, None, None, case.alpha)
    zero_b = q.qlora_merge(w, d["A"], torch.zeros_like(d["B"]), case.alpha)
    torch.cuda.synchronize()
    for t in (plain, zero_b):
        assert np.array_equal(t.float().cpu().numpy(), wb)  # values; a -0.0 restore comes back +0.0


def test_concurrent_streams_with_own_workspaces():
    """Two skinny forwards (their adapter exchange runs through the workspace) and two GEMM backwards issued on two
    streams at once, each with its own workspace, give bit for bit the results of the same calls run one after
    the other."""
    say("concurrent streams")
    cases = [Case(1024, 1024, 64, 16, cfg=127, proj=i) for i in range(2)]
    ins = []
    for c in cases:
        d = c.device_inputs()
        ins.append((q.qlora_quantize(d["W"]), d))
    torch.cuda.synchronize()

    def run(k, ws=None):
        w, d = ins[k]
        h, u = q.qlora_forward(w, d["x"], d["A"], d["B"], 16.0, save_u=True, ws=ws)
        x300 = d["x"].repeat(19, 1)[:300].contiguous()
        dy300 = torch.cat([d["dY"]] * 19)[:300].contiguous()
        g = q.qlora_backward(w, x300, dy300, d["A"], d["B"], 16.0, ws=ws)
        return (h, u) + tuple(g)

    ref = [run(0), run(1)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(2)]   # default priority
    wss = [torch.zeros(q.qlora_workspace_bytes(1024, 1024, 300, 64), dtype=torch.uint8, device="cuda")
           for _ in range(2)]
    torch.cuda.synchronize()
    out = [None, None]
    for k in range(2):
        with torch.cuda.stream(streams[k]):
            out[k] = run(k, wss[k])
    torch.cuda.synchronize()
    for k in range(2):
        for a, b in zip(out[k], ref[k]):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
    for ws in wss:
        # every counter is left zero; the last word counts waits that took their fallback (same results)
        assert int(ws[:q.COUNTER_BYTES - 4].view(torch.int32).abs().sum().item()) == 0
        say(f"    fallbacks: {q.qlora_workspace_fallbacks(ws)}")


def _rand_bf16(gen, *shape, std=1.0):
    return (torch.randn(*shape, device="cuda", generator=gen) * std).to(torch.bfloat16)


def test_concurrent_full_size_calls_from_two_threads():
    """Two host threads, each on its own stream with its own workspace, each running a LLaMA-7B-shape skinny
    forward (4096 x 4096, T = 16, r = 64; one workgroup per compute unit, producers and readers of the adapter
    exchange) and a 13B-shape backward (5120 x 5120, T = 4096, r = 64; split-K tails and token-split adapter
    gradients) three times over: every output is bit for bit that of the same calls run one after the other.
    The two launches can hold the compute units the other's waiting workgroups need; no wait depends on that
    (a wait that runs out of time takes its fallback, counted in the workspace)."""
    import threading

    say("concurrent full-size calls, two threads")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    ins = []
    for k in range(2):
        Ws = (torch.randn(4096, 4096, device="cuda", generator=gen) * 0.02)
        Wb = (torch.randn(5120, 5120, device="cuda", generator=gen) * 0.02)
        ins.append(dict(ws_=q.qlora_quantize(Ws), wb=q.qlora_quantize(Wb),
                        xs=_rand_bf16(gen, 16, 4096), As=_rand_bf16(gen, 64, 4096, std=0.02),
                        Bs=_rand_bf16(gen, 4096, 64, std=0.02),
                        xb=_rand_bf16(gen, 4096, 5120), dyb=_rand_bf16(gen, 4096, 5120),
                        Ab=_rand_bf16(gen, 64, 5120, std=0.02), Bb=_rand_bf16(gen, 5120, 64, std=0.02)))
        del Ws, Wb
    torch.cuda.synchronize()

    def run(k, ws=None):
        d = ins[k]
        h, u = q.qlora_forward(d["ws_"], d["xs"], d["As"], d["Bs"], 16.0, save_u=True, ws=ws)
        g = q.qlora_backward(d["wb"], d["xb"], d["dyb"], d["Ab"], d["Bb"], 16.0, ws=ws)
        return (h, u) + tuple(g)

    ref = [run(0), run(1)]
    torch.cuda.synchronize()
    wss = [torch.zeros(max(q.qlora_workspace_bytes(4096, 4096, 16, 64), q.qlora_workspace_bytes(5120, 5120, 4096, 64)),
                       dtype=torch.uint8, device="cuda") for _ in range(2)]
    streams = [torch.cuda.Stream() for _ in range(2)]   # default priority
    torch.cuda.synchronize()
    outs = [[], []]
    errors = []
    start = threading.Barrier(2)

    def worker(k):
        try:
            start.wait()
            with torch.cuda.stream(streams[k]):
                for _ in range(3):
                    outs[k].append(run(k, wss[k]))
            streams[k].synchronize()
        except Exception as e:  # pragma: no cover - reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for k in range(2):
        for rep, out in enumerate(outs[k]):
            for i, (a, b) in enumerate(zip(out, ref[k])):
                same = torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                                   b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
                assert same, f"thread {k}, repetition {rep}, output {i} differs from the sequential run"
    for ws in wss:
        assert int(ws[:q.COUNTER_BYTES - 4].view(torch.int32).abs().sum().item()) == 0
        say(f"    fallbacks: {q.qlora_workspace_fallbacks(ws)}")


def test_fallback_paths_give_the_same_bits():
    """With the workspace's wait limit at one tick, every wait that does not succeed at once takes its fallback
    path: a skinny forward's reader forms missing adapter partials itself (4096 x 4096, T = 1 and 16, r = 64), a
    split GEMM part (1024 x 4096 at T = 512: fewer tiles than compute units, every tile split over K) and a
    token-split adapter-gradient part leave their shares to the last arriver. Three repetitions give bit for bit
    the outputs of the same calls under the built-in limit, and the fallback count shows that the paths ran."""
    say("fallback paths")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(23)
    w1 = q.qlora_quantize(torch.randn(4096, 4096, device="cuda", generator=gen) * 0.02)
    x1 = _rand_bf16(gen, 16, 4096)
    A1, B1 = _rand_bf16(gen, 64, 4096, std=0.02), _rand_bf16(gen, 4096, 64, std=0.02)
    w2 = q.qlora_quantize(torch.randn(1024, 4096, device="cuda", generator=gen) * 0.02)
    x2, dy2 = _rand_bf16(gen, 512, 4096), _rand_bf16(gen, 512, 1024)
    A2, B2 = _rand_bf16(gen, 64, 4096, std=0.02), _rand_bf16(gen, 1024, 64, std=0.02)
    ws = torch.zeros(max(q.qlora_workspace_bytes(4096, 4096, 16, 64), q.qlora_workspace_bytes(1024, 4096, 512, 64)),
                     dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    def run():
        out = []
        for T in (1, 16):
            out += list(q.qlora_forward(w1, x1[:T].contiguous(), A1, B1, 16.0, save_u=True, ws=ws))
        h, u = q.qlora_forward(w2, x2, A2, B2, 16.0, save_u=True, ws=ws)
        out += [h, u] + list(q.qlora_backward(w2, x2, dy2, A2, B2, 16.0, u_saved=u, ws=ws))
        return out

    ref = run()
    torch.cuda.synchronize()
    assert q.qlora_workspace_fallbacks(ws) == 0
    q.qlora_workspace_set_wait_limit(ws, 1)
    try:
        got = [run() for _ in range(3)]
        torch.cuda.synchronize()
        n = q.qlora_workspace_fallbacks(ws)
    finally:
        q.qlora_workspace_set_wait_limit(ws, 0)
    say(f"    fallbacks with a one-tick limit: {n}")
    for rep, out in enumerate(got):
        for i, (a, b) in enumerate(zip(out, ref)):
            same = torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
            assert same, f"repetition {rep}, output {i} differs from the run under the built-in limit"
    assert n > 0, "no wait took its fallback path"
    # every counter is left zero (the last word counts the fallbacks, the one before it is the limit, now 0)
    assert int(ws[:q.COUNTER_BYTES - 4].view(torch.int32).abs().sum().item()) == 0
