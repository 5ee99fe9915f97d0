"""bpw_gemv_packed_scratch: the decode product with the library's fixed per-GPU
scratch in place of a caller workspace. Its output must equal bpw_gemv_packed's
bit for bit (same kernels, fixed-order sums) and meet the oracle's parity rule,
on two calls in a row whose second input is smaller, for each workload that
needs a workspace (ternary split-K slices, the 4-bit act-order gather, 4-bit
split-K slices behind the gather) and one that needs none. A call whose workspace would exceed the scratch is refused
before any launch (CPU test)."""
import ctypes

import numpy as np
import pytest
import torch

import bit_packed_weight_amd as bpw
import synth
from oracle import compare, quant, reference

DEV = "cuda"


def _host(t):
    return t.detach().float().cpu().numpy()


def _ternary_pair(m, k, n, seed):
    w = synth.ternary_int8(f"scratch_t{m}_{k}_{n}", seed, m, k, n, 0.005, 0.05, "f16")
    pw = bpw.prepare_packed(bpw.TERNARY2, w.codes, w.scales)
    q, xs = bpw.quantize_rows(torch.from_numpy(w.x).to(DEV))
    return w, pw, q, xs


@pytest.mark.gpu
def test_scratch_matches_workspace_entry_ternary_split_k():
    shapes = [(16, 14336, 4096, 61), (4, 8192, 1000, 62)]     # the second call is smaller
    for m, k, n, seed in shapes:
        print(f"[scratch] ternary split-K m={m} k={k} n={n}", flush=True)
        w, pw, q, xs = _ternary_pair(m, k, n, seed)
        need = bpw.workspace_size(pw, m, bpw.I8, bpw.PATH_GEMV)
        assert 0 < need <= bpw.SCRATCH_BYTES
        y_ref_gpu = bpw.gemv_packed(pw, q, xs)
        y = torch.full((m, n), float("nan"), dtype=torch.float16, device=DEV)
        bpw.gemv_packed_scratch(pw, q, xs, out=y)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_host(y), _host(y_ref_gpu))
        qh, xsh = quant.quantize_rows(w.x)
        _, y_ref = reference.ternary_int8_product(qh, xsh, w.codes, w.scales)
        r = compare.compare(_host(y), y_ref, "f16")
        assert r["ok"], r


@pytest.mark.gpu
def test_scratch_matches_workspace_entry_w4_act_order():
    for m, k, n, seed in [(8, 5120, 2000, 63), (1, 1024, 300, 64)]:
        print(f"[scratch] w4 act-order m={m} k={k} n={n}", flush=True)
        w = synth.int4_zp_actorder(f"scratch_w{m}_{k}_{n}", seed, m, k, n)
        pw = bpw.prepare_packed(bpw.INT4_ZP, w.codes, w.scales, w.zeros, w.g_idx)
        x = torch.from_numpy(w.x).to(DEV)
        assert 0 < bpw.workspace_size(pw, m, bpw.F16, bpw.PATH_GEMV) <= bpw.SCRATCH_BYTES
        y_ws = bpw.gemv_packed(pw, x)
        y = torch.full((m, n), float("nan"), dtype=torch.float16, device=DEV)
        bpw.gemv_packed_scratch(pw, x, out=y)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_host(y), _host(y_ws))
        wd = reference.weights_int4(w.codes, w.scales_f64(), w.zeros, w.g_idx)
        r = compare.compare(_host(y), reference.product(w.x_f32(), wd), "f16")
        assert r["ok"], r


@pytest.mark.gpu
def test_scratch_matches_workspace_entry_w4_split_k():
    # 4-bit beyond 48 groups at 2 <= M <= 16: the gathered rows, then the fp32 slices in the
    # scratch; the second call is smaller and has no act order (slices only)
    for m, k, n, seed, act in [(8, 13824, 1500, 66, True), (3, 6272, 700, 67, False)]:
        print(f"[scratch] w4 split-K m={m} k={k} n={n} act_order={act}", flush=True)
        w = synth.int4_zp_actorder(f"scratch_ws{m}_{k}_{n}", seed, m, k, n, act_order=act)
        pw = bpw.prepare_packed(bpw.INT4_ZP, w.codes, w.scales, w.zeros, w.g_idx)
        x = torch.from_numpy(w.x).to(DEV)
        assert 0 < bpw.workspace_size(pw, m, bpw.F16, bpw.PATH_GEMV) <= bpw.SCRATCH_BYTES
        y_ws = bpw.gemv_packed(pw, x)
        y = torch.full((m, n), float("nan"), dtype=torch.float16, device=DEV)
        bpw.gemv_packed_scratch(pw, x, out=y)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_host(y), _host(y_ws))
        wd = reference.weights_int4(w.codes, w.scales_f64(), w.zeros, w.g_idx)
        r = compare.compare(_host(y), reference.product(w.x_f32(), wd), "f16")
        assert r["ok"], r


@pytest.mark.gpu
def test_scratch_without_workspace_need():
    w, pw, q, xs = _ternary_pair(1, 4096, 3000, 65)
    assert bpw.workspace_size(pw, 1, bpw.I8, bpw.PATH_GEMV) == 0
    y = bpw.gemv_packed_scratch(pw, q, xs)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_host(y), _host(bpw.gemv_packed(pw, q, xs)))


def test_scratch_refuses_a_workspace_beyond_its_size():
    # ternary x int8 with M = 64 runs the prefill kernels, whose workspace is M * K bytes:
    # 64 * 2**19 = 32 MiB > 16 MiB. Refused on the host before any HIP call (the device
    # pointers below are never dereferenced).
    m, k, n = 64, 1 << 19, 256
    fake = 1 << 20
    st = bpw.BpwWeights(bpw.TERNARY2, bpw.F16, 128, 0, n, k, fake, fake, None, None)
    rc = bpw.lib().bpw_gemv_packed_scratch(ctypes.byref(st), fake, bpw.I8, fake, m, fake, bpw.F16, None)
    assert rc == bpw.ESHAPE
    assert "fixed scratch" in bpw.last_error() and str(bpw.SCRATCH_BYTES) in bpw.last_error()
    # the same arguments with a workspace entry report the larger need
    need = ctypes.c_size_t()
    assert bpw.lib().bpw_workspace_size(ctypes.byref(st), m, bpw.I8, bpw.PATH_GEMV, ctypes.byref(need)) == 0
    assert need.value > bpw.SCRATCH_BYTES
