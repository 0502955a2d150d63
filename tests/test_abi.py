"""C-ABI checks that need no GPU: exported symbols, host-side tables, sizes, and argument
validation (every case here fails validation, so nothing is enqueued)."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora.h")

from bit_quantized_finetuning_amd import build as _build  # noqa: E402

if not os.path.exists(_build.LIB):  # hipcc cross-compiles for gfx950 without a GPU
    _build.build()
from bit_quantized_finetuning_amd import qlora as q  # noqa: E402

ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_WORKSPACE, ERR_DTYPE = -1, -2, -3, -4, -5


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qlora_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert {"qlora_quantize", "qlora_forward", "qlora_backward", "qlora_dequantize"} <= set(names)
    for n in names:
        assert hasattr(q.lib, n), f"{n} declared in include/qlora.h but not exported"


def test_codebook_bit_exact_with_oracle():
    lib_c = np.array(q.qlora_nf4_codebook(), dtype=np.float32)
    assert np.array_equal(lib_c.view(np.uint32), oracle.nf4_codebook().view(np.uint32))


def test_thresholds_bit_exact_with_oracle():
    lib_t = np.array(q.qlora_nf4_thresholds(), dtype=np.float32)
    assert np.array_equal(lib_t.view(np.uint32), oracle.nf4_thresholds_f32().view(np.uint32))


@pytest.mark.parametrize("shape", [(1024, 1024), (4096, 4096), (11008, 4096), (5120, 5120), (13824, 5120),
                                   (8192, 22016), (16, 64), (48, 192)])
def test_storage_bytes_matches_oracle(shape):
    assert q.qlora_storage_bytes(*shape) == oracle.storage_bytes(*shape)


def test_workspace_bytes_positive_and_covers_buffers():
    # Not monotone in T: a tile count that leaves the last round of compute
    # units partly idle adds float32 partial tiles of a K split.
    a = q.qlora_workspace_bytes(4096, 4096, 16, 64)
    b = q.qlora_workspace_bytes(4096, 4096, 4096, 64)
    assert a >= 65536 and b >= 65536
    assert b >= 65536 + 2 * 4096 * 64 * 4  # counters + float32 u and v at T = 4096
    assert q.qlora_workspace_bytes(4096, 4096, 16, 0) > 0
    assert q.qlora_workspace_bytes(0, 4096, 16, 0) == 0


def test_status_strings():
    for s in (0, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_WORKSPACE, ERR_DTYPE, -6, -7, -8, -9):
        assert q.qlora_status_string(s)
    assert q.qlora_status_string(12345) == "unknown status"


# --- validation: fake, never-dereferenced device addresses --------------------

GOOD = 0x10000   # 16-byte aligned, never touched because validation fails first
BAD = 0x10001    # misaligned


def _w(d_out=64, d_in=128, codes=GOOD, qs=GOOD, sm=GOOD):
    return q._Nf4Weight(d_out, d_in, codes, qs, sm)


def _fwd(w, x=GOOD, T=4, A=GOOD, B=GOOD, r=8, h=GOOD, u=None, ws=GOOD, ws_bytes=1 << 40):
    return q.lib.qlora_forward(ctypes.byref(w), x, T, A, B, r, 16.0, h, u, ws, ws_bytes, None)


def _bwd(w, x=GOOD, dY=GOOD, T=4, A=GOOD, B=GOOD, r=8, u=None, dX=GOOD, dA=GOOD, dB=GOOD, ws=GOOD,
         ws_bytes=1 << 40):
    return q.lib.qlora_backward(ctypes.byref(w), x, dY, T, A, B, r, 16.0, u, dX, dA, dB, ws, ws_bytes, None)


def test_forward_rejects_bad_arguments():
    assert _fwd(_w(d_in=100)) == ERR_SHAPE          # d_in % 64
    assert _fwd(_w(d_out=40)) == ERR_SHAPE          # d_out % 16
    assert _fwd(_w(d_out=0)) == ERR_SHAPE
    assert _fwd(_w(), T=0) == ERR_SHAPE
    assert _fwd(_w(), r=12) == ERR_SHAPE            # r % 8
    assert _fwd(_w(), r=264) == ERR_SHAPE           # r > 256
    assert _fwd(_w(), r=-8) == ERR_SHAPE
    assert _fwd(_w(codes=None)) == ERR_NULL
    assert _fwd(_w(), x=None) == ERR_NULL
    assert _fwd(_w(), h=None) == ERR_NULL
    assert _fwd(_w(), A=None) == ERR_NULL           # r > 0 with only B
    assert _fwd(_w(), x=BAD) == ERR_ALIGN
    assert _fwd(_w(qs=BAD)) == ERR_ALIGN
    assert _fwd(_w(), u=BAD) == ERR_ALIGN
    assert _fwd(_w(), ws_bytes=16) == ERR_WORKSPACE
    assert _fwd(_w(), ws=None) == ERR_NULL
    need = q.qlora_workspace_bytes(64, 128, 4, 8)
    assert _fwd(_w(), ws_bytes=need - 1) == ERR_WORKSPACE


def test_backward_rejects_bad_arguments():
    assert _bwd(_w(d_in=96)) == ERR_SHAPE
    assert _bwd(_w(), dY=None) == ERR_NULL
    assert _bwd(_w(), A=None, B=None, r=0, dA=GOOD, dB=None) == ERR_SHAPE   # no adapter, dA asked
    assert _bwd(_w(), x=None, u=None, dB=GOOD, dA=None) == ERR_NULL          # dB needs x or u
    assert _bwd(_w(), x=None, dA=GOOD) == ERR_NULL                           # dA needs x
    assert _bwd(_w(), dX=BAD) == ERR_ALIGN
    assert _bwd(_w(), ws_bytes=0) == ERR_WORKSPACE


def test_quantize_and_dequantize_reject_bad_arguments():
    w = _w()
    assert q.lib.qlora_quantize(None, 0, ctypes.byref(w), None, None) == ERR_NULL
    assert q.lib.qlora_quantize(GOOD, 7, ctypes.byref(w), None, None) == ERR_DTYPE
    assert q.lib.qlora_quantize(BAD, 0, ctypes.byref(w), None, None) == ERR_ALIGN
    assert q.lib.qlora_quantize(GOOD, 0, ctypes.byref(_w(d_in=65)), None, None) == ERR_SHAPE
    assert q.lib.qlora_quantize(GOOD, 0, None, None, None) == ERR_NULL
    assert q.lib.qlora_dequantize(ctypes.byref(w), 3, GOOD, None) == ERR_DTYPE
    assert q.lib.qlora_dequantize(ctypes.byref(w), 0, None, None) == ERR_NULL
    assert q.lib.qlora_dequantize(ctypes.byref(w), 0, BAD, None) == ERR_ALIGN


def test_quantize_many_rejects_bad_arguments_before_launching():
    """A bad job anywhere in the list is found before any launch (here no GPU is there to launch on)."""
    ws = (q._Nf4Weight * 3)(_w(), _w(), _w(d_in=65))
    ptrs = (ctypes.c_void_p * 3)(GOOD, GOOD, GOOD)
    assert q.lib.qlora_quantize_many(ptrs, 0, ws, -1, None, None) == ERR_SHAPE
    assert q.lib.qlora_quantize_many(None, 0, ws, 2, None, None) == ERR_NULL
    assert q.lib.qlora_quantize_many(ptrs, 0, None, 2, None, None) == ERR_NULL
    assert q.lib.qlora_quantize_many(ptrs, 0, ws, 3, None, None) == ERR_SHAPE        # the third job
    assert q.lib.qlora_quantize_many(ptrs, 7, ws, 2, None, None) == ERR_DTYPE
    assert q.lib.qlora_quantize_many(ptrs, 0, ws, 0, None, None) == 0                # nothing to do
    bad = (ctypes.c_void_p * 2)(GOOD, BAD)
    assert q.lib.qlora_quantize_many(bad, 0, ws, 2, None, None) == ERR_ALIGN
    nul = (ctypes.c_void_p * 2)(GOOD, None)
    assert q.lib.qlora_quantize_many(nul, 0, ws, 2, None, None) == ERR_NULL


def _job(w, x=GOOD, T=4, A=GOOD, B=GOOD, r=8, h=GOOD, u=None):
    return q._ForwardJob(ctypes.pointer(w), x, T, A, B, r, 16.0, h, u)


def test_forward_many_rejects_bad_arguments_before_launching():
    """Every job is checked before any launch (here no GPU is there to launch on); the workspace covers the
    counter region and one rank-256 exchange buffer per job."""
    ws1 = q.qlora_forward_many_workspace_bytes(1)
    assert ws1 == 65536 + 4 * 16 * 256 * 8
    assert q.qlora_forward_many_workspace_bytes(3) == 65536 + 3 * 4 * 16 * 256 * 8
    assert q.qlora_forward_many_workspace_bytes(0) == 0
    assert q.qlora_forward_many_workspace_bytes(q.MAX_FORWARD_JOBS + 1) == 0
    ws_need = q.qlora_forward_many_workspace_bytes(3)
    wts = [_w(), _w(), _w()]

    def call(jobs, count=None, ws=GOOD, ws_bytes=ws_need):
        arr = (q._ForwardJob * len(jobs))(*jobs)
        return q.lib.qlora_forward_many(arr, len(jobs) if count is None else count, ws, ws_bytes, None)

    good = [_job(w) for w in wts]
    assert call(good, count=0) == ERR_SHAPE
    assert call(good, count=q.MAX_FORWARD_JOBS + 1) == ERR_SHAPE
    assert q.lib.qlora_forward_many(None, 1, GOOD, ws_need, None) == ERR_NULL
    assert call(good[:2] + [_job(wts[2], T=17)]) == ERR_SHAPE          # the third job: T > 16
    assert call(good[:2] + [_job(_w(d_in=100))]) == ERR_SHAPE         # d_in % 64
    assert call([good[0], _job(wts[1], r=12), good[2]]) == ERR_SHAPE   # r % 8
    assert call([good[0], _job(wts[1], x=None), good[2]]) == ERR_NULL
    assert call([good[0], _job(wts[1], h=None), good[2]]) == ERR_NULL
    assert call([good[0], _job(wts[1], A=None), good[2]]) == ERR_NULL  # r > 0 with only B
    assert call([good[0], _job(wts[1], x=BAD), good[2]]) == ERR_ALIGN
    assert call([good[0], good[1], _job(wts[2], u=BAD)]) == ERR_ALIGN
    assert call(good, ws_bytes=ws_need - 1) == ERR_WORKSPACE
    assert call(good, ws=None) == ERR_NULL
    assert call(good, ws=BAD) == ERR_ALIGN


def test_merge_rejects_bad_arguments():
    w = _w()
    assert q.lib.qlora_merge(ctypes.byref(w), GOOD, GOOD, 8, 16.0, None, None) == ERR_NULL
    assert q.lib.qlora_merge(ctypes.byref(w), GOOD, GOOD, 12, 16.0, GOOD, None) == ERR_SHAPE   # r % 8
    assert q.lib.qlora_merge(ctypes.byref(w), GOOD, None, 8, 16.0, GOOD, None) == ERR_NULL     # B missing
    assert q.lib.qlora_merge(ctypes.byref(w), BAD, GOOD, 8, 16.0, GOOD, None) == ERR_ALIGN
    assert q.lib.qlora_merge(ctypes.byref(_w(d_in=96)), GOOD, GOOD, 8, 16.0, GOOD, None) == ERR_SHAPE


ERR_VALUE = -9


def test_adamw_rejects_bad_arguments():
    """Host-side validation runs before any pointer is looked up, so these need no GPU."""
    def call(hp=None, step=1, n=16, grad=GOOD, master=GOOD, m=GOOD, v=GOOD, param=None):
        hp = hp if hp is not None else q.AdamWHparams(1e-3, 0.9, 0.999, 1e-8, 0.0)
        return q.lib.qlora_adamw_step(ctypes.byref(hp), step, n, grad, master, m, v, param, None)
    assert q.lib.qlora_adamw_step(None, 1, 16, GOOD, GOOD, GOOD, GOOD, None, None) == ERR_NULL
    assert call(grad=None) == ERR_NULL and call(v=None) == ERR_NULL
    assert call(n=-1) == ERR_SHAPE
    assert call(step=0) == ERR_VALUE
    assert call(hp=q.AdamWHparams(1e-3, 1.0, 0.999, 1e-8, 0.0)) == ERR_VALUE     # beta1 = 1
    assert call(hp=q.AdamWHparams(1e-3, 0.9, 0.999, 0.0, 0.0)) == ERR_VALUE      # eps = 0
    assert call(hp=q.AdamWHparams(-1e-3, 0.9, 0.999, 1e-8, 0.0)) == ERR_VALUE    # lr < 0
    assert call(hp=q.AdamWHparams(float("nan"), 0.9, 0.999, 1e-8, 0.0)) == ERR_VALUE
    assert call(m=BAD) == ERR_ALIGN and call(param=BAD) == ERR_ALIGN
    assert call(n=0) == 0                                                          # nothing to do


@pytest.mark.parametrize("shape", [(16, 64), (80, 320), (4096, 4096), (11008, 4096)])
def test_absmax_storage_bytes_matches_oracle(shape):
    assert q.qlora_storage_bytes_absmax(*shape) == oracle.storage_bytes_absmax(*shape)


def test_absmax_weight_validation():
    """qscale = NULL selects absmax-only storage: accepted as a weight, but its other checks still apply."""
    absmax = _w(qs=None)
    assert _fwd(absmax, x=None) == ERR_NULL          # the weight itself passes; the missing x is reported
    assert _fwd(_w(qs=None, sm=None)) == ERR_NULL
    assert _fwd(_w(qs=None, sm=BAD)) == ERR_ALIGN
    assert _fwd(_w(qs=None, d_in=100)) == ERR_SHAPE
    # one buffer range of float32 block scales: nblocks * 4 must stay below 2^31 bytes
    assert _fwd(_w(d_out=1 << 20, d_in=1 << 15, qs=None)) == ERR_SHAPE
    assert _fwd(_w(d_out=1 << 20, d_in=1 << 15, qs=GOOD), x=None) == ERR_NULL   # double quant: no such limit
    assert q.lib.qlora_dequantize(ctypes.byref(_w(qs=None)), 1, None, None) == ERR_NULL


def test_weight_with_2_pow_32_blocks_is_refused():
    """Block indices are 32-bit in the kernels: d_out * d_in / 64 must stay below 2^32."""
    assert _fwd(_w(d_out=1 << 20, d_in=1 << 18), x=None) == ERR_SHAPE
    assert _fwd(_w(d_out=(1 << 20) - 16, d_in=1 << 18), x=None) == ERR_NULL   # just below: the weight passes


def test_header_and_library_from_plain_c(tmp_path):
    """A C11 program (gcc, not hipcc) includes include/qlora.h, links libqlora.so and calls the host-side entry
    points: the codebook and thresholds equal the oracle's bit for bit, the sizes equal the oracle's formulas, and
    a malformed weight is refused with QLORA_ERR_SHAPE."""
    import shutil
    import subprocess

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    libdir = os.path.dirname(q.LIB_PATH)
    exe = tmp_path / "abi_check"
    subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    os.path.join(ROOT, "tests", "c_abi", "abi_check.c"), "-L", libdir, "-lqlora",
                    "-Wl,-rpath," + libdir, "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    vals = np.array([float.fromhex(v) for v in out[:31]], dtype=np.float32)
    assert np.array_equal(vals[:16].view(np.uint32), oracle.nf4_codebook().view(np.uint32))
    assert np.array_equal(vals[16:31].view(np.uint32), oracle.nf4_thresholds_f32().view(np.uint32))
    sb, sa, ws = (int(v) for v in out[31].split())
    assert sb == oracle.storage_bytes(4096, 4096) and sa == oracle.storage_bytes_absmax(4096, 4096)
    assert ws == q.qlora_workspace_bytes(4096, 4096, 16, 64)
    assert out[32].split()[0] == str(ERR_SHAPE)
