"""GPU parity of the grouped weight-streaming forward (qlora_forward_many): several independent forwards of
T <= 16 tokens in as few launches as their kernel variants allow.

Per job: h and u within tolerance of the oracle (gpu_common); u bit for bit equal to the same job run alone
through qlora_forward; h within tolerance of it (a job's share of the compute units decides which wave sums
which K segments, so h may differ in the last float32 bits); every output bit for bit the same across repeated
calls and across the adapter exchange's fallback path. The jobs mix the kernel variants (x staged in LDS or read
from memory; blocks per row a multiple of four or not), ranks 0 to 256, ragged row tiles, both storages, and
more jobs of one variant than one launch takes.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import Case, assert_close, say, product

pytestmark = pytest.mark.gpu

q = product("qlora")


class AbsmaxCase(Case):
    def oracle_quant(self):
        if self._q is None:
            codes, s = oracle.quantize_absmax(self.W)
            w32, wb = oracle.dequantize_absmax(codes, s, self.d_out, self.d_in)
            self._q = (codes, None, s, w32, wb)
        return self._q


# d_out, d_in, r, T, storage ("dq": double quant, "am": absmax only)
MIXED = [
    (1024, 1024, 8, 1, "dq"),     # x in LDS, 16 blocks per row
    (80, 192, 16, 4, "dq"),       # 3 blocks per row, ragged row tile
    (272, 320, 64, 16, "dq"),     # 5 blocks per row
    (528, 1344, 256, 16, "am"),   # maximum rank, absmax-only storage
    (4096, 4096, 64, 1, "dq"),    # LLaMA-7B q_proj shape
    (16, 64, 0, 3, "dq"),         # base only, one block per row
    (272, 5120, 16, 16, "dq"),    # x read from memory (16 x 5120 bf16 > 136 KB), 80 blocks per row
    (64, 5184, 64, 16, "am"),     # x from memory, 81 blocks per row
    (1024, 4096, 64, 16, "dq"),
    (2048, 1024, 32, 2, "dq"),
]
# eleven jobs of one kernel variant: two launches
ELEVEN = [(256 + 64 * i, 512, 8 * (i % 4), 1 + i % 16, "dq") for i in range(11)]
# a rank-256 job needs 64 producer workgroups although it has 33 row tiles; with a large job beside it the
# shares first add up to more than the compute units and are taken back from the large job
TRIM = [(528, 1344, 256, 4, "dq"), (4096, 1344, 0, 4, "dq")]


def _cases(spec, cfg):
    out = []
    for k, (d_out, d_in, r, T, st) in enumerate(spec):
        cls = AbsmaxCase if st == "am" else Case
        c = cls(d_out, d_in, r, T, cfg=cfg, proj=k)
        d = c.device_inputs()
        w = q.qlora_quantize(d["W"], double_quant=(st == "dq"))
        del d["W"]
        out.append((c, w, d))
    torch.cuda.synchronize()
    return out


def _jobs(cases):
    return [{"w": w, "x": d["x"], "A": d["A"], "B": d["B"], "alpha": c.alpha, "save_u": c.r > 0}
            for c, w, d in cases]


def _same(a, b):
    if a is None or b is None:
        return a is None and b is None
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


@pytest.mark.parametrize("spec,cfg", [(MIXED, 140), (ELEVEN, 141), (TRIM, 144)], ids=["mixed", "eleven", "trim"])
def test_forward_many_parity(spec, cfg):
    say(f"forward_many {len(spec)} jobs")
    cases = _cases(spec, cfg)
    ws = torch.zeros(q.qlora_forward_many_workspace_bytes(len(cases)), dtype=torch.uint8, device="cuda")
    got = q.qlora_forward_many(_jobs(cases), ws=ws)
    again = q.qlora_forward_many(_jobs(cases), ws=ws)
    torch.cuda.synchronize()
    for (c, w, d), (h, u), (h2, u2) in zip(cases, got, again):
        tag = f"{c.d_out}x{c.d_in} r={c.r} T={c.T}"
        h_ref, u_ref = c.oracle_forward()
        assert_close(f"h {tag}", h, h_ref)
        hs, us = q.qlora_forward(w, d["x"], d["A"], d["B"], c.alpha, save_u=c.r > 0)
        torch.cuda.synchronize()
        assert_close(f"h {tag} against the call alone", h, hs.double().cpu().numpy())
        if c.r > 0:
            assert_close(f"u {tag}", u, u_ref)
            assert _same(u, us), f"{tag}: u differs from the call alone"
        assert _same(h, h2) and _same(u, u2), f"{tag}: a repeated call gave other bits"
    assert int(ws[:q.COUNTER_BYTES].view(torch.int32).abs().sum().item()) == 0


def test_forward_many_fallback_gives_the_same_bits():
    """With a one-tick wait limit every reader that does not find an adapter partial at once forms it itself:
    the outputs are the bits of the run under the built-in limit, and the fallback count shows the path ran."""
    say("forward_many fallback")
    cases = _cases(MIXED, 142)
    ws = torch.zeros(q.qlora_forward_many_workspace_bytes(len(cases)), dtype=torch.uint8, device="cuda")
    ref = q.qlora_forward_many(_jobs(cases), ws=ws)
    torch.cuda.synchronize()
    assert q.qlora_workspace_fallbacks(ws) == 0
    q.qlora_workspace_set_wait_limit(ws, 1)
    try:
        got = [q.qlora_forward_many(_jobs(cases), ws=ws) for _ in range(3)]
        torch.cuda.synchronize()
        n = q.qlora_workspace_fallbacks(ws)
    finally:
        q.qlora_workspace_set_wait_limit(ws, 0)
    say(f"    fallbacks with a one-tick limit: {n}")
    for rep, outs in enumerate(got):
        for k, ((h, u), (hr, ur)) in enumerate(zip(outs, ref)):
            assert _same(h, hr) and _same(u, ur), f"repetition {rep}, job {k} differs from the run under the limit"
    assert n > 0, "no wait took its fallback path"
    assert int(ws[:q.COUNTER_BYTES - 4].view(torch.int32).abs().sum().item()) == 0


def test_forward_many_rejects_a_long_job_before_launching():
    cases = _cases([(256, 512, 8, 4, "dq")], 143)
    c, w, d = cases[0]
    x17 = torch.zeros(17, 512, dtype=torch.bfloat16, device="cuda")
    h = torch.full((4, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        q.qlora_forward_many([{"w": w, "x": d["x"], "A": d["A"], "B": d["B"], "alpha": 16.0, "h": h},
                              {"w": w, "x": x17, "A": d["A"], "B": d["B"], "alpha": 16.0}])
    torch.cuda.synchronize()
    assert bool((h == 7.0).all()), "an output was written although the call was refused"
