"""The Python binding refuses malformed tensors before any library call (CPU only).

The C ABI receives bare pointers and sizes: it cannot see that a tensor is
shorter than M x K, or that an output is narrower than N. Each refusal below
must raise ValueError in the binding, so a wrong-shaped tensor never reaches a
kernel that would read or write past it. All tensors here live on the CPU; the
last check of each call (the tensor is not on a GPU) is reached only when every
shape, dtype and layout check has passed.
"""
import numpy as np
import pytest
import torch

import bit_packed_weight_amd as bpw

M, K, N = 3, 256, 40


def _ternary(n=N, k=K):
    return bpw.PackedWeights(bpw.TERNARY2, bpw.F16, n, k, torch.zeros((n, k // 4), dtype=torch.uint8),
                             torch.zeros((n, k // 128), dtype=torch.float16))


def _int4_zp(n=N, k=K, perm=True):
    g = k // 128
    return bpw.PackedWeights(bpw.INT4_ZP, bpw.F16, n, k, torch.zeros((n, k // 2), dtype=torch.uint8),
                             torch.zeros((n, g), dtype=torch.float16), torch.zeros((n, (g + 1) // 2), dtype=torch.uint8),
                             torch.arange(k, dtype=torch.int32) if perm else None)


def _q(m=M, k=K):
    return torch.zeros((m, k), dtype=torch.int8)


def _refuses(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_well_formed_cpu_call_stops_at_the_device_check():
    _refuses("GPU tensor", bpw.gemv_packed, _ternary(), _q(), torch.ones(M))
    _refuses("GPU tensor", bpw.gemm_packed, _int4_zp(), torch.zeros((M, K), dtype=torch.float16))
    _refuses("GPU tensor", bpw.partials, _ternary(), _q(), bpw.PATH_GEMV, 0, M, 0, N)
    _refuses("GPU tensor", bpw.quantize_rows, torch.zeros((M, K)))
    _refuses("GPU tensor", bpw.quantize_groups, torch.zeros((M, K)))


def test_activation_width_must_be_k():
    _refuses("x has shape", bpw.gemv_packed, _ternary(), _q(k=K - 128), torch.ones(M))
    _refuses("x has shape", bpw.gemv_packed, _ternary(), _q(k=K + 16), torch.ones(M))
    _refuses("x has shape", bpw.gemm_packed, _int4_zp(), torch.zeros((M, K // 2), dtype=torch.float16))


def test_activation_dtype_and_layout():
    _refuses("not supported", bpw.gemv_packed, _int4_zp(), torch.zeros((M, K), dtype=torch.float32))
    _refuses("not supported", bpw.gemv_packed, _ternary(), torch.zeros((M, K), dtype=torch.int32))
    # fp32 rows for ternary weights are the fused one-token call: no x_scale
    _refuses("x_scale must be None", bpw.gemv_packed, _ternary(), torch.zeros((M, K), dtype=torch.float32),
             torch.ones(M))
    _refuses("contiguous", bpw.gemv_packed, _ternary(), _q(k=2 * K)[:, ::2], torch.ones(M))


def test_row_scale_shape_dtype_and_presence():
    w = _ternary()
    _refuses("need x_scale", bpw.gemv_packed, w, _q())
    _refuses("x_scale has shape", bpw.gemv_packed, w, _q(), torch.ones(M - 1))
    _refuses("x_scale has shape", bpw.gemv_packed, w, _q(), torch.ones(M + 1))
    _refuses("x_scale has dtype", bpw.gemv_packed, w, _q(), torch.ones(M, dtype=torch.float64))
    _refuses("x_scale must be None", bpw.gemm_packed, _int4_zp(), torch.zeros((M, K), dtype=torch.float16),
             torch.ones(M))


def test_group_scale_shape():
    w = _ternary()
    _refuses("x_scale has shape", bpw.gemv_packed, w, _q(), torch.ones((M, K // 128 - 1)))
    _refuses("x_scale has shape", bpw.gemv_packed, w, _q(), torch.ones((M + 1, K // 128)))


def test_output_shape_dtype_and_layout():
    w = _ternary()
    xs = torch.ones(M)
    _refuses("out has shape", bpw.gemv_packed, w, _q(), xs, out=torch.empty((M, N - 1), dtype=torch.float16))
    _refuses("out has shape", bpw.gemv_packed, w, _q(), xs, out=torch.empty((M - 1, N), dtype=torch.float16))
    _refuses("out has dtype", bpw.gemv_packed, w, _q(), xs, out=torch.empty((M, N), dtype=torch.int32))
    _refuses("out must be contiguous", bpw.gemv_packed, w, _q(), xs,
             out=torch.empty((N, M), dtype=torch.float16).t())


def test_weight_planes_against_n_and_k():
    w = _ternary()
    w.codes = torch.zeros((N, K // 4 - 1), dtype=torch.uint8)
    _refuses("codes has shape", bpw.gemv_packed, w, _q(), torch.ones(M))
    w = _ternary()
    w.scales = torch.zeros((N - 1, K // 128), dtype=torch.float16)
    _refuses("scales has shape", bpw.gemv_packed, w, _q(), torch.ones(M))
    w = _ternary()
    w.scales = torch.zeros((N, K // 128), dtype=torch.bfloat16)
    _refuses("scales has dtype", bpw.gemv_packed, w, _q(), torch.ones(M))
    w = _int4_zp()
    w.zeros = torch.zeros((N, 2), dtype=torch.uint8)
    _refuses("zeros has shape", bpw.gemm_packed, w, torch.zeros((M, K), dtype=torch.float16))
    w = _int4_zp()
    w.perm = torch.arange(K - 1, dtype=torch.int32)
    _refuses("perm has shape", bpw.gemm_packed, w, torch.zeros((M, K), dtype=torch.float16))
    w = _int4_zp()
    w.perm = torch.arange(K, dtype=torch.int64)
    _refuses("perm has dtype", bpw.gemm_packed, w, torch.zeros((M, K), dtype=torch.float16))


def test_partials_window_and_q():
    w = _ternary()
    _refuses("q has shape", bpw.partials, w, _q(k=K - 128), bpw.PATH_GEMV, 0, 1, 0, 1)
    _refuses("window", bpw.partials, w, _q(), bpw.PATH_GEMV, 0, M + 1, 0, N)
    _refuses("window", bpw.partials, w, _q(), bpw.PATH_GEMV, 0, M, 5, 5)
    _refuses("window", bpw.partials, w, _q(), bpw.PATH_GEMV, 0, M, 0, N + 1)


def test_quantizer_outputs():
    x = torch.zeros((M, K))
    _refuses("q has shape", bpw.quantize_rows, x, q=torch.empty((M, K - 1), dtype=torch.int8))
    _refuses("q has dtype", bpw.quantize_rows, x, q=torch.empty((M, K), dtype=torch.uint8))
    _refuses("x_scale has shape", bpw.quantize_rows, x, x_scale=torch.empty(M - 1))
    _refuses("x_scale has shape", bpw.quantize_groups, x, x_scale=torch.empty(M))
    _refuses("multiple of 128", bpw.quantize_groups, torch.zeros((M, 100)))
    _refuses("x has dtype", bpw.quantize_rows, torch.zeros((M, K), dtype=torch.float64))


def test_workspace_too_small_or_wrong_dtype():
    w = _int4_zp()
    x = torch.zeros((M, K), dtype=torch.float16)
    need = bpw.workspace_size(w, M, bpw.F16, bpw.PATH_GEMV)
    assert need >= 2 * M * K
    _refuses("workspace has", bpw.gemv_packed, w, x, workspace=torch.empty(need - 1, dtype=torch.uint8))
    _refuses("workspace has dtype", bpw.gemv_packed, w, x, workspace=torch.empty(need, dtype=torch.int8))
    _refuses("1-D", bpw.gemv_packed, w, x, workspace=torch.empty((2, need), dtype=torch.uint8))


def test_probe_sizes():
    src = torch.zeros(1024, dtype=torch.uint8)
    _refuses("dst holds", bpw.probe, bpw.PROBE_COPY, src, torch.zeros(1008, dtype=torch.uint8))
    _refuses("dst holds", bpw.probe, bpw.PROBE_READ, src, torch.zeros(0, dtype=torch.uint8))
    _refuses("GPU tensor", bpw.probe, bpw.PROBE_COPY, src, torch.zeros(1024, dtype=torch.uint8))
    _refuses("contiguous", bpw.probe, bpw.PROBE_COPY, torch.zeros(2048, dtype=torch.uint8)[::2],
             torch.zeros(1024, dtype=torch.uint8))
