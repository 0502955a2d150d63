"""The benchmark's flop accounting (host logic, no GPU): a stacked call (several projections of one input as one
weight, their adapters as a block-diagonal pair) is counted with the algorithmic flops of its projections called
one by one, so the zeros of the block-diagonal B never count as work. Checked against the formulas of the
forward h = x W^T + s (x A^T) B^T and the backward dX, dA, dB written out per projection."""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from bit_quantized_finetuning_amd import synth  # noqa: E402


def _direct(d_out, d_in, r, T):
    # forward: x W^T (2 T d_in d_out), u = x A^T (2 T r d_in), u B^T (2 T r d_out)
    fwd = 2 * T * d_in * d_out + 2 * T * r * d_in + 2 * T * r * d_out
    # backward: dY W (2 T d_in d_out), v = dY B and s v A (2 T r d_out + 2 T r d_in), dA = v^T x and dB = dY^T u
    bwd = 2 * T * d_in * d_out + 2 * T * r * (d_out + d_in) + 2 * T * r * (d_in + d_out)
    return fwd, bwd


def test_stacked_layers_count_the_flops_of_their_projections():
    for sep, fused in (("65b_layer", "65b_layer_fused"), ("14b_stack", "14b_stack_fused")):
        T = synth.WORKLOADS[sep].tokens[0]
        want = sum(sum(_direct(p.d_out, p.d_in, p.r, T)) for p in synth.WORKLOADS[sep].projections)
        for wl in (sep, fused):
            got = sum(bench.proj_flops(p, T, False) + bench.proj_flops(p, T, True)
                      for p in synth.WORKLOADS[wl].projections)
            assert got == want, (wl, got, want)


def test_stacked_layer_matches_its_parts():
    sep, fused = synth.WORKLOADS["65b_layer"], synth.WORKLOADS["65b_layer_fused"]
    # the same weights row for row, and one rank-64 adapter per projection
    assert sum(p.d_out * p.d_in for p in sep.projections) == sum(p.d_out * p.d_in for p in fused.projections)
    for p in fused.projections:
        if p.b_rows:
            assert p.b_rows[0][0] == 0 and p.b_rows[-1][1] == p.d_out
            assert all(a[1] == b[0] for a, b in zip(p.b_rows, p.b_rows[1:]))
            assert p.r == 64 * len(p.b_rows) and p.alpha / p.r == 16.0 / 64
            # every part holds a whole number of 256-block double-quant groups, so stacking leaves the storage alone
            assert all((r1 - r0) * p.d_in % (64 * 256) == 0 for r0, r1 in p.b_rows)
