"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Each case names its workload, shape and seed in the test id. Integer results
(quantised activations, int32 group partials) must match bit for bit; float
outputs must satisfy oracle.compare's rule (1e-3 relative plus half an output
ulp). Inputs come from synth; both sides compute from them independently.
"""
import dataclasses

import numpy as np
import pytest
import torch

import bit_packed_weight_amd as bpw
import synth
from oracle import compare, formats, quant, reference

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def to_dev(a: np.ndarray, dtype: str):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64) if t.is_floating_point() else t.cpu().numpy()


def assert_close(y, y_ref, dtype, what):
    r = compare.compare(y, y_ref, dtype)
    assert r["ok"], f"{what}: {r}"
    return r


def prepare(w: synth.Workload):
    fmt = bpw.FORMAT_NAMES[w.fmt]
    sd = bpw.F16 if w.scale_dtype == "f16" else bpw.BF16
    zeros = w.zeros if w.fmt == "int4_zp" else None
    return bpw.prepare_packed(fmt, w.codes, w.scales, zeros, w.g_idx, scale_dtype=sd, device=DEV)


# ------------------------------------------------------------------ quantiser
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("m,k", [(1, 512), (5, 4096), (3, 1000), (64, 8192), (2, 1002), (2, 20480), (1, 14336)])
def test_quantize_rows_bit_exact(dtype, m, k):
    rng = np.random.default_rng(m * 7 + k)
    x = (rng.standard_normal((m, k)) * rng.uniform(0.01, 50, size=(m, 1))).astype(np.float32)
    x[0, : min(k, 8)] = [127.0, 2.5, 3.5, -2.5, -0.5, 126.5, 0.5, 1.5][: min(k, 8)]
    if m > 2:
        x[2] = 0.0
    if dtype == "f16":
        xs = x.astype(np.float16)
        xf = xs.astype(np.float32)
    elif dtype == "bf16":
        xs = synth.f32_to_bf16_bits(x)
        xf = synth.bf16_bits_to_f32(xs)
    else:
        xs = xf = x
    q, s = bpw.quantize_rows(to_dev(xs, dtype))
    torch.cuda.synchronize()
    q_ref, s_ref = quant.quantize_rows(xf)
    np.testing.assert_array_equal(host(s).astype(np.float32), s_ref)
    np.testing.assert_array_equal(host(q), q_ref)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("m,k", [(1, 128), (1, 4096), (3, 1152), (16, 8192)])
def test_quantize_groups_bit_exact(dtype, m, k):
    rng = np.random.default_rng(m * 11 + k)
    g = k // 128
    # a different magnitude per (row, group), ties in group 0 of row 0, a zero group
    x = (rng.standard_normal((m, k)) * np.repeat(rng.uniform(0.01, 50, size=(m, g)), 128, axis=1)).astype(np.float32)
    x[0, :8] = [127.0, 2.5, 3.5, -2.5, -0.5, 126.5, 0.5, 1.5]
    if g > 1:
        x[m - 1, 128:256] = 0.0
    if dtype == "f16":
        xs = x.astype(np.float16)
        xf = xs.astype(np.float32)
    elif dtype == "bf16":
        xs = synth.f32_to_bf16_bits(x)
        xf = synth.bf16_bits_to_f32(xs)
    else:
        xs = xf = x
    q, s = bpw.quantize_groups(to_dev(xs, dtype))
    torch.cuda.synchronize()
    q_ref, s_ref = quant.quantize_groups(xf)
    assert s.shape == (m, g)
    np.testing.assert_array_equal(host(s).astype(np.float32), s_ref)
    np.testing.assert_array_equal(host(q), q_ref)


# ------------------------------------------------------------------ ternary x int8
def ternary_case(m, k, n, seed, out="f16"):
    return synth.ternary_int8(f"t{m}x{k}x{n}", seed, m, k, n, 0.005, 0.05, out)


def run_ternary(w: synth.Workload, entry: str):
    pw = prepare(w)
    x = to_dev(w.x, "f32")
    q, xs = bpw.quantize_rows(x)
    fn = bpw.gemv_packed if entry == "gemv" else bpw.gemm_packed
    y = fn(pw, q, xs, out_dtype=TORCH[w.out_dtype])
    torch.cuda.synchronize()
    q_ref, xs_ref = quant.quantize_rows(w.x)
    np.testing.assert_array_equal(host(q), q_ref)
    _, y_ref = reference.ternary_int8_product(q_ref, xs_ref, w.codes, w.scales)
    return pw, q, xs, y, y_ref


@pytest.mark.parametrize("m,k,n", [(1, 512, 256), (1, 4096, 1000), (2, 640, 333), (4, 128, 64),
                                   (7, 1024, 520), (16, 4096, 300), (32, 256, 97), (1, 8192, 130),
                                   # skinny kernel: four-tile shares, ragged tiles; long-K kernel: 2..4 phases,
                                   # ragged last phase; M = 1 past the row kernel's K; row kernel partial chunk
                                   (32, 8192, 3000), (9, 3072, 20000), (24, 6144, 9000), (16, 14336, 4096),
                                   (4, 11008, 700), (1, 20480, 500), (1, 14336, 1000), (1, 1152, 333),
                                   # M = 1, N >= 16384: four rows per wave, ragged last wave, one and four chunks
                                   (1, 4096, 16387), (1, 16384, 16390),
                                   # 2 <= M <= 16 up to K = 4096: one 16-row tile per wave, a last workgroup
                                   # with one row or half a tile, waves without rows, 56-row shares
                                   (2, 2048, 33), (16, 1024, 5000), (13, 4096, 14001)])
@pytest.mark.parametrize("out", ["f32", "f16", "bf16"])
def test_gemv_ternary_parity(m, k, n, out):
    w = ternary_case(m, k, n, 100 + m + k + n, out)
    _, _, _, y, y_ref = run_ternary(w, "gemv")
    assert_close(host(y), y_ref, out, f"gemv ternary m={m} k={k} n={n}")


# Split-K decode (2 <= M <= 32 beyond 32 groups): slices of 32 groups side by
# side, fp32 partials summed in slice order. Ragged last slices (2 and 1
# groups), M past 16, and a repeat that must be bit-identical.
@pytest.mark.parametrize("m,k,n", [(16, 14336, 4096), (5, 4352, 1000), (32, 8320, 777), (2, 16384, 64),
                                   # K a multiple of 1024, M <= 16: the staged kernel over 32-group slices
                                   # (last slice of 8 and 16 groups, one-row and ragged workgroups)
                                   (16, 5120, 300), (3, 8192, 1000), (16, 14336, 33), (7, 30720, 2000)])
def test_gemv_ternary_split_k(m, k, n):
    w = ternary_case(m, k, n, 900 + m + k + n, "f16")
    pw = prepare(w)
    need = bpw.workspace_size(pw, m, bpw.I8, bpw.PATH_GEMV)
    assert need == -(-(-(-k // (128 * 32)) * m * n * 4) // 256) * 256      # slices x M x N fp32, 256-byte rounded
    q, xs = bpw.quantize_rows(to_dev(w.x, "f32"))
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=DEV)
    y1 = bpw.gemv_packed(pw, q, xs, workspace=ws)
    y2 = bpw.gemv_packed(pw, q, xs, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2), "split-K result changed between calls"
    q_ref, xs_ref = quant.quantize_rows(w.x)
    _, y_ref = reference.ternary_int8_product(q_ref, xs_ref, w.codes, w.scales)
    assert_close(host(y1), y_ref, "f16", f"gemv ternary split-K m={m} k={k} n={n}")


@pytest.mark.parametrize("m,k,n", [(1, 4096, 1000), (1, 16384, 77), (1, 512, 256), (2, 640, 333),
                                   (16, 4096, 14336), (32, 8192, 3000), (9, 3072, 20000), (20, 4096, 700),
                                   (1, 20480, 300), (8, 14336, 1000),
                                   # M = 1, N >= 16384: four rows per wave, ragged last wave
                                   (1, 1024, 16389), (1, 12288, 20001)])
@pytest.mark.parametrize("out", ["f32", "f16"])
def test_gemv_ternary_group_scales(m, k, n, out):
    # one activation scale per (row, 128-group): y = sum_g xs[m,g] * ws[n,g] * P[m,n,g]
    w = ternary_case(m, k, n, 600 + m + k + n, out)
    pw = prepare(w)
    q, xs = bpw.quantize_groups(to_dev(w.x, "f32"))
    y = bpw.gemv_packed(pw, q, xs, out_dtype=TORCH[out])
    torch.cuda.synchronize()
    q_ref, xs_ref = quant.quantize_groups(w.x)
    np.testing.assert_array_equal(host(q), q_ref)
    _, y_ref = reference.ternary_int8_product_group_scales(q_ref, xs_ref, w.codes, w.scales)
    assert_close(host(y), y_ref, out, f"gemv ternary group scales m={m} k={k} n={n}")


def test_group_scales_through_both_entries():
    # The decode GEMV and the prefill GEMM both take per-group scales; on the
    # same inputs each meets the parity rule (their fp32 fold orders differ).
    w = ternary_case(4, 256, 64, 9)
    pw = prepare(w)
    q, xs = bpw.quantize_groups(to_dev(w.x, "f32"))
    y1 = bpw.gemv_packed(pw, q, xs)
    y2 = bpw.gemm_packed(pw, q, xs)
    torch.cuda.synchronize()
    q_ref, xs_ref = quant.quantize_groups(w.x)
    _, y_ref = reference.ternary_int8_product_group_scales(q_ref, xs_ref, w.codes, w.scales)
    assert_close(host(y1), y_ref, "f16", "group scales, decode entry")
    assert_close(host(y2), y_ref, "f16", "group scales, prefill entry")


@pytest.mark.parametrize("m,k,n", [(1, 256, 300), (130, 1024, 520), (300, 640, 257), (64, 128, 256)])
def test_gemm_ternary_parity(m, k, n):
    w = ternary_case(m, k, n, 200 + m + k + n, "f16")
    _, _, _, y, y_ref = run_ternary(w, "gemm")
    assert_close(host(y), y_ref, "f16", f"gemm ternary m={m} k={k} n={n}")


@pytest.mark.parametrize("path", [bpw.PATH_GEMV, bpw.PATH_GEMM])
@pytest.mark.parametrize("m,k,n,win", [(3, 256, 70, (0, 3, 0, 70)), (32, 512, 200, (5, 29, 33, 170)),
                                       (1, 128, 40, (0, 1, 7, 9)), (1, 4096, 77, (0, 1, 3, 70)),
                                       (1, 8192, 9, (0, 1, 0, 9)), (16, 8192, 600, (3, 14, 100, 580)),
                                       (12, 3072, 20000, (0, 12, 9000, 9777)), (3, 12288, 500, (0, 3, 17, 463)),
                                       (1, 5248, 300, (0, 1, 0, 300)), (1, 2048, 16400, (0, 1, 15990, 16400)),
                                       (16, 4096, 1000, (0, 16, 0, 1000)), (2, 1024, 33, (1, 2, 5, 30))])
def test_partials_bit_exact(path, m, k, n, win):
    # stress inputs: full int8 range and every 2-bit code including 3
    rng = np.random.default_rng(m + k + n)
    q = synth.random_int8(m + k, m, k)
    codes = rng.integers(0, 4, size=(n, k), dtype=np.uint8)
    scales = rng.uniform(0.005, 0.05, size=(n, k // 128)).astype(np.float16)
    pw = bpw.prepare_packed(bpw.TERNARY2, codes, scales, device=DEV)
    m0, m1, n0, n1 = win
    p = bpw.partials(pw, to_dev(q, "i8"), path, m0, m1, n0, n1)
    torch.cuda.synchronize()
    p_ref = reference.ternary_partials(q[m0:m1], codes[n0:n1])
    np.testing.assert_array_equal(host(p), p_ref)


def test_ternary_row_independence_and_determinism():
    w = ternary_case(8, 1024, 300, 7)
    pw = bpw.prepare_packed(bpw.TERNARY2, w.codes, w.scales, device=DEV)
    x = to_dev(w.x, "f32")
    q, xs = bpw.quantize_rows(x)
    for fn in (bpw.gemv_packed, bpw.gemm_packed):
        y1 = fn(pw, q, xs)
        y2 = fn(pw, q, xs)
        q2 = q.clone()
        q2[1:] = torch.randint(-127, 128, q2[1:].shape, device=DEV, dtype=torch.int8)
        y3 = fn(pw, q2, xs)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
        assert torch.equal(y1[0].view(torch.int16), y3[0].view(torch.int16))


def test_outputs_fully_written_over_nan_poison():
    w = ternary_case(5, 512, 333, 9)
    pw = bpw.prepare_packed(bpw.TERNARY2, w.codes, w.scales, device=DEV)
    q, xs = bpw.quantize_rows(to_dev(w.x, "f32"))
    for fn in (bpw.gemv_packed, bpw.gemm_packed):
        y = torch.full((5, 333), float("nan"), dtype=torch.float16, device=DEV)
        fn(pw, q, xs, out=y)
        torch.cuda.synchronize()
        assert torch.isfinite(y).all()


# ------------------------------------------------------------------ 4-bit x fp16/bf16
def w4_case(fmt, m, k, n, seed, act_order, x_dtype):
    if fmt == "int4_zp":
        return synth.int4_zp_actorder(f"w{m}x{k}x{n}", seed, m, k, n, act_order=act_order, x_dtype=x_dtype)
    return synth.int4_sym(f"w{m}x{k}x{n}", seed, m, k, n, x_dtype=x_dtype)


def w4_reference(w: synth.Workload, rounded: bool):
    zeros = w.zeros if w.fmt == "int4_zp" else None
    s = w.scales_f64()
    if rounded:
        wt = reference.weights_int4_rounded(w.codes, s, zeros, w.g_idx, w.x_dtype)
    else:
        wt = reference.weights_int4(w.codes, s, zeros, w.g_idx)
    return reference.product(w.x_f32(), wt)


@pytest.mark.parametrize("fmt,x_dtype,act_order", [("int4_zp", "f16", True), ("int4_zp", "f16", False),
                                                   ("int4_sym", "bf16", False), ("int4_sym", "f16", False),
                                                   ("int4_zp", "bf16", True)])
@pytest.mark.parametrize("m,k,n", [(1, 640, 333), (1, 2048, 301), (1, 8192, 66), (1, 3072, 13), (3, 128, 64), (8, 5120, 200),
                                   (16, 1024, 97), (32, 256, 130),
                                   # streaming skinny kernel: 16..48 groups, 4..6 per wave, ragged waves and tiles
                                   (2, 2048, 1000), (16, 6144, 777), (5, 4224, 3000), (12, 2560, 9000),
                                   # M = 1: a partial last 1024-column chunk, and K split over 2 or 4 waves
                                   # (9088: 5 chunks per wave, the second wave's last one partial and one
                                   # past K; 20608: 6 per wave; 32768: the longest K, 8 per wave)
                                   (1, 1152, 77), (1, 9088, 130), (1, 13824, 300), (1, 20608, 50), (1, 32768, 70),
                                   # 2 <= M <= 16 beyond 48 groups: split-K slices (49 groups: 28 + 21;
                                   # 108: 28, 28, 28, 24; 256: 8 x 32) and the fixed-order reduce
                                   (2, 6272, 70), (8, 13824, 300), (16, 8192, 500), (5, 32768, 40)])
def test_gemv_w4_parity(fmt, x_dtype, act_order, m, k, n):
    w = w4_case(fmt, m, k, n, 300 + m + k + n, act_order, x_dtype)
    pw = prepare(w)
    y = bpw.gemv_packed(pw, to_dev(w.x, x_dtype))
    torch.cuda.synchronize()
    assert_close(host(y), w4_reference(w, rounded=False), x_dtype, f"gemv {fmt} {x_dtype} m={m} k={k} n={n}")


# Act order gathers inside the decode kernels (M = 1, and the skinny kernel
# where M rows of x fit in LDS) when the permutation plane is 16-byte aligned;
# a plane that is only 4-byte aligned (what the boundary requires) takes the
# separate gather launch. At M = 1 both run the same arithmetic and must give
# the same bits; the skinny kernel splits K over more waves when it gathers
# (the fp32 sum over waves is grouped differently), so there both must meet
# the oracle's rule.
@pytest.mark.parametrize("x_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("m,k,n", [(1, 5120, 700), (8, 5120, 700), (11, 2560, 3000), (2, 6144, 100)])
def test_w4_act_order_fused_and_separate_gather_agree(x_dtype, m, k, n):
    w = w4_case("int4_zp", m, k, n, 77 + m, True, x_dtype)
    pw = prepare(w)
    x = to_dev(w.x, x_dtype)
    pbig = torch.zeros(k + 1, dtype=torch.int32, device=DEV)
    pbig[1:] = pw.perm
    pw_off = dataclasses.replace(pw, perm=pbig[1:])
    assert pw_off.perm.data_ptr() % 16 == 4
    ws = torch.empty(bpw.workspace_size(pw, m, bpw.F16 if x_dtype == "f16" else bpw.BF16, bpw.PATH_GEMV),
                     dtype=torch.uint8, device=DEV)
    y_fused = bpw.gemv_packed(pw, x, workspace=ws)
    y_sep = bpw.gemv_packed(pw_off, x, workspace=ws)
    torch.cuda.synchronize()
    ref = w4_reference(w, rounded=False)
    if m == 1:
        assert torch.equal(y_fused.view(torch.int16), y_sep.view(torch.int16))
    else:
        assert_close(host(y_sep), ref, x_dtype, f"separate act-order gather {x_dtype} m={m}")
    assert_close(host(y_fused), ref, x_dtype, f"fused act-order gather {x_dtype} m={m}")


# Bit-identical repeats, outputs of one token row independent of the other
# rows, and every output written over a NaN-poisoned buffer: the M = 1 row
# kernel (act order), the skinny M = 8 kernel, and the prefill GEMM.
@pytest.mark.parametrize("entry,m,k,n", [("gemv", 1, 5120, 700), ("gemv", 8, 5120, 700), ("gemm", 300, 1024, 520)])
def test_w4_determinism_row_independence(entry, m, k, n):
    w = w4_case("int4_zp", m, k, n, 600 + m + k + n, True, "f16")
    pw = prepare(w)
    fn = bpw.gemv_packed if entry == "gemv" else bpw.gemm_packed
    x = to_dev(w.x, "f16")
    y1 = torch.full((m, n), float("nan"), dtype=torch.float16, device=DEV)
    fn(pw, x, out=y1)
    y2 = fn(pw, x)
    x2 = x.clone()
    if m > 1:
        x2[1:] = torch.randn(x2[1:].shape, device=DEV).to(torch.float16)
    y3 = fn(pw, x2)
    torch.cuda.synchronize()
    assert torch.isfinite(y1).all()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(y1[0].view(torch.int16), y3[0].view(torch.int16))


@pytest.mark.parametrize("x_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("m,k,n", [(1, 5120, 700), (8, 5120, 700), (3, 2048, 5000)])
def test_gemv_w4_f32_out(x_dtype, m, k, n):
    w = w4_case("int4_zp", m, k, n, 500 + m + k + n, True, x_dtype)
    pw = prepare(w)
    y = bpw.gemv_packed(pw, to_dev(w.x, x_dtype), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert y.dtype == torch.float32
    assert_close(host(y), w4_reference(w, rounded=False), "f32", f"gemv int4_zp {x_dtype} f32 out m={m} k={k} n={n}")


@pytest.mark.parametrize("fmt,x_dtype,act_order", [("int4_sym", "bf16", False), ("int4_zp", "f16", True),
                                                   ("int4_sym", "f16", False)])
@pytest.mark.parametrize("m,k,n", [(1, 256, 300), (200, 512, 260), (129, 1024, 513)])
def test_gemm_w4_parity(fmt, x_dtype, act_order, m, k, n):
    w = w4_case(fmt, m, k, n, 400 + m + k + n, act_order, x_dtype)
    pw = prepare(w)
    y = bpw.gemm_packed(pw, to_dev(w.x, x_dtype))
    torch.cuda.synchronize()
    assert_close(host(y), w4_reference(w, rounded=True), x_dtype, f"gemm {fmt} {x_dtype} m={m} k={k} n={n}")


# Degenerate shapes: one output row, one 128-group, and M on both sides of the
# decode entry's hand-over to the GEMM kernels (M = 32 decode, M = 33 GEMM).
@pytest.mark.parametrize("entry,m,k,n", [("gemv", 1, 128, 1), ("gemv", 32, 128, 1), ("gemv", 33, 256, 65),
                                         ("gemv", 32, 4096, 33), ("gemm", 1, 128, 1), ("gemm", 33, 128, 257)])
def test_ternary_degenerate_shapes(entry, m, k, n):
    w = ternary_case(m, k, n, 1100 + m + k + n, "f32")
    _, q, _, y, y_ref = run_ternary(w, entry)
    assert y.shape == (m, n)
    assert_close(host(y), y_ref, "f32", f"{entry} ternary m={m} k={k} n={n}")


@pytest.mark.parametrize("fmt,x_dtype,entry,m,k,n", [("int4_zp", "f16", "gemv", 1, 1024, 1), ("int4_sym", "bf16", "gemv", 16, 2048, 1),
                                                     ("int4_zp", "f16", "gemv", 33, 128, 40), ("int4_sym", "bf16", "gemm", 1, 128, 1),
                                                     # one output row: K split over waves (M = 1), one
                                                     # split-K slice holding a single group (M = 2, 49 groups)
                                                     ("int4_zp", "f16", "gemv", 1, 9088, 1), ("int4_sym", "bf16", "gemv", 1, 32768, 3),
                                                     ("int4_zp", "f16", "gemv", 2, 6272, 1), ("int4_sym", "bf16", "gemv", 16, 16384, 17)])
def test_w4_degenerate_shapes(fmt, x_dtype, entry, m, k, n):
    w = w4_case(fmt, m, k, n, 1200 + m + k + n, fmt == "int4_zp", x_dtype)
    pw = prepare(w)
    fn = bpw.gemv_packed if entry == "gemv" else bpw.gemm_packed
    y = fn(pw, to_dev(w.x, x_dtype))
    torch.cuda.synchronize()
    assert y.shape == (m, n)
    # the GEMM kernels (entry gemm, or M > 32 through the decode entry) round W to the activation dtype
    rounded = entry == "gemm" or m > 32
    assert_close(host(y), w4_reference(w, rounded=rounded), x_dtype, f"{entry} {fmt} m={m} k={k} n={n}")


# ------------------------------------------------------------------ named workloads, full size
def test_workload_ternary_tiny_full():
    w = synth.ternary_tiny()
    pw, q, xs, y, y_ref = run_ternary(w, "gemv")
    assert_close(host(y), y_ref, "f32", "ternary_gemv_tiny")
    p = bpw.partials(pw, q, bpw.PATH_GEMV, 0, 1, 0, w.n)
    q_ref, _ = quant.quantize_rows(w.x)
    np.testing.assert_array_equal(host(p), reference.ternary_partials(q_ref, w.codes))


@pytest.mark.parametrize("m", [1, 16])
def test_workload_ternary_decode_full(m):
    w = synth.ternary_decode(m)
    pw, q, xs, y, y_ref = run_ternary(w, "gemv")
    assert_close(host(y), y_ref, "f16", f"ternary_decode m={m}")
    # int32 group partials of the whole product, bit-exact
    p = bpw.partials(pw, q, bpw.PATH_GEMV, 0, m, 0, w.n)
    q_ref, _ = quant.quantize_rows(w.x)
    np.testing.assert_array_equal(host(p), reference.ternary_partials(q_ref, w.codes))


def test_gemv_ternary_large_weight_sampled():
    # The M = 1 decode GEMV on the ternary prefill weight (K=8192, N=28672):
    # sampled outputs against the oracle, and every group partial of a few
    # column windows bit-exact.
    w = synth.leading_rows(synth.ternary_prefill(), 1)
    pw = bpw.prepare_packed(bpw.TERNARY2, w.codes, w.scales, device=DEV)
    q, xs = bpw.quantize_rows(to_dev(w.x, "f32"))
    y = bpw.gemv_packed(pw, q, xs)
    torch.cuda.synchronize()
    q_ref, xs_ref = quant.quantize_rows(w.x)
    np.testing.assert_array_equal(host(q), q_ref)
    rng = np.random.default_rng(4)
    cols = np.unique(np.concatenate([np.arange(64), np.arange(w.n - 64, w.n), rng.choice(w.n, 1024, replace=False)]))
    _, y_ref = reference.ternary_int8_product(q_ref, xs_ref, w.codes[cols], w.scales[cols])
    assert_close(host(y)[:, cols], y_ref, "f16", "ternary GEMV on the prefill weight, sampled")
    for (n0, n1) in [(0, 256), (w.n - 256, w.n), (13000, 13300)]:
        p = bpw.partials(pw, q, bpw.PATH_GEMV, 0, 1, n0, n1)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(p), reference.ternary_partials(q_ref, w.codes[n0:n1]))


@pytest.mark.parametrize("m", [1, 8])
def test_workload_w4a16_decode_full(m):
    w = synth.w4a16_decode(m)
    pw = prepare(w)
    y = bpw.gemv_packed(pw, to_dev(w.x, "f16"))
    torch.cuda.synchronize()
    assert_close(host(y), w4_reference(w, rounded=False), "f16", f"w4a16_decode m={m}")


@pytest.mark.parametrize("m", [1, 8])
@pytest.mark.parametrize("act_order", [True, False])
def test_w4a16_down_projection_full(m, act_order):
    # The down projection of the W4A16 decode layer (K=13824, N=5120): at
    # M = 1 the row kernel with K split over two waves per row pair, at M = 8
    # the skinny kernel's split-K slices and the reduce; act order gathers in
    # a separate launch at this K.
    w = synth.w4a16_down(m, act_order=act_order)
    pw = prepare(w)
    y = bpw.gemv_packed(pw, to_dev(w.x, "f16"))
    torch.cuda.synchronize()
    assert_close(host(y), w4_reference(w, rounded=False), "f16", f"w4a16 down projection m={m} act_order={act_order}")


def test_workload_w4a16_prefill_sampled():
    w = synth.w4a16_prefill()
    pw = prepare(w)
    y = bpw.gemm_packed(pw, to_dev(w.x, "bf16"))
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, w.m - 1], rng.choice(w.m, 30, replace=False)]))
    cols = np.unique(np.concatenate([np.arange(64), np.arange(w.n - 64, w.n), rng.choice(w.n, 512, replace=False)]))
    wt = reference.weights_int4_rounded(w.codes[cols], w.scales_f64()[cols], None, None, "bf16")
    y_ref = reference.product(w.x_f32()[rows], wt)
    assert_close(host(y)[np.ix_(rows, cols)], y_ref, "bf16", "w4a16_prefill sampled")


def test_workload_w4a16_prefill_full():
    """Every output of the 4-bit prefill workload (M=2048, K=4096, N=14336) against the
    fp64 oracle (bf16-rounded dequantised weights, then a dgemm)."""
    w = synth.w4a16_prefill()
    pw = prepare(w)
    y = bpw.gemm_packed(pw, to_dev(w.x, "bf16"))
    torch.cuda.synchronize()
    yh = host(y)
    del y
    wt = reference.weights_int4_rounded(w.codes, w.scales_f64(), None, None, "bf16")
    xf = w.x_f32()
    y_ref = reference.product(xf, wt)
    # sum_k |x w| per output: the scale of the fp32 accumulation error (near-zero
    # outputs cancel; the plain rule's floor is below one fp32 rounding there)
    abs_sum = reference.product(np.abs(xf), np.abs(wt))
    del wt
    r = compare.compare(yh, y_ref, "bf16", abs_sum=abs_sum, k=w.k)
    assert r["ok"], f"w4a16_prefill full: {r}"
    # without the accumulation term the rule holds for all but a handful of near-zero outputs
    plain = compare.compare(yh, y_ref, "bf16")
    assert plain["worst_ratio"] < 2.0 and plain["rel_rms"] < 2.5e-3, plain


def test_workload_ternary_prefill_sampled():
    w = synth.ternary_prefill()
    pw = bpw.prepare_packed(bpw.TERNARY2, w.codes, w.scales, device=DEV)
    x = to_dev(w.x, "f32")
    q, xs = bpw.quantize_rows(x)
    y = bpw.gemm_packed(pw, q, xs, out_dtype=torch.float16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, w.m - 1], rng.choice(w.m, 14, replace=False)]))
    cols = np.unique(np.concatenate([np.arange(32), np.arange(w.n - 32, w.n), rng.choice(w.n, 256, replace=False)]))
    q_ref, xs_ref = quant.quantize_rows(w.x[rows])
    np.testing.assert_array_equal(host(q)[rows], q_ref)
    _, y_ref = reference.ternary_int8_product(q_ref, xs_ref, w.codes[cols], w.scales[cols])
    assert_close(host(y)[np.ix_(rows, cols)], y_ref, "f16", "ternary_int8_prefill sampled")
    # int32 group partials on corner and random windows, through the GEMM core
    wins = [(0, 64, 0, 256), (w.m - 64, w.m, w.n - 256, w.n), (0, 64, w.n - 256, w.n), (w.m - 64, w.m, 0, 256)]
    for _ in range(4):                                    # four random windows beside the corners
        a, b = int(rng.integers(0, w.m - 64)), int(rng.integers(0, w.n - 256))
        wins.append((a, a + 64, b, b + 256))
    for (m0, m1, n0, n1) in wins:
        p = bpw.partials(pw, q, bpw.PATH_GEMM, m0, m1, n0, n1)
        torch.cuda.synchronize()
        q_win, _ = quant.quantize_rows(w.x[m0:m1])        # the oracle quantises its own rows
        np.testing.assert_array_equal(host(p), reference.ternary_partials(q_win, w.codes[n0:n1]),
                                      err_msg=f"window {(m0, m1, n0, n1)}")


# ------------------------------------------------------------------ 4-bit x int8 (prefill GEMM)
def w4a8_case(fmt, m, k, n, seed, act_order, scale_dtype):
    w = w4_case(fmt, m, k, n, seed, act_order, scale_dtype)
    q_ref, xs_ref = quant.quantize_rows(w.x_f32())
    return w, q_ref, xs_ref


def w4a8_reference(w, q_ref, xs_ref, rows=None, cols=None):
    rows = slice(None) if rows is None else rows
    cols = slice(None) if cols is None else cols
    zeros = w.zeros[cols] if w.fmt == "int4_zp" else None
    return reference.int4_int8_product(q_ref[rows], xs_ref[rows], w.codes[cols], w.scales_f64()[cols], zeros,
                                       w.g_idx)


@pytest.mark.parametrize("fmt,scale_dtype,act_order", [("int4_sym", "bf16", False), ("int4_zp", "f16", True),
                                                       ("int4_zp", "f16", False), ("int4_sym", "f16", True)])
@pytest.mark.parametrize("m,k,n", [(1, 256, 300), (130, 1024, 520), (300, 640, 257), (64, 128, 256),
                                   (129, 2048, 1000),
                                   # K % 1024 == 0: codes two groups ahead through LDS, scale and zero-point
                                   # rows staged per tile; ragged last weight tile, 32 and 64 groups
                                   (257, 4096, 300), (40, 8192, 513)])
def test_gemm_w4a8_parity(fmt, scale_dtype, act_order, m, k, n):
    w, q_ref, xs_ref = w4a8_case(fmt, m, k, n, 400 + m + k + n, act_order, scale_dtype)
    pw = prepare(w)
    q, xs = bpw.quantize_rows(to_dev(w.x_f32(), "f32"))
    y = bpw.gemm_packed(pw, q, xs)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(q), q_ref)
    _, y_ref = w4a8_reference(w, q_ref, xs_ref)
    assert_close(host(y), y_ref, "f16", f"gemm w4a8 {fmt} {scale_dtype} act={act_order} m={m} k={k} n={n}")


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm_w4a8_output_dtypes(out):
    w, q_ref, xs_ref = w4a8_case("int4_zp", 77, 512, 300, 431, True, "bf16")
    pw = prepare(w)
    y = bpw.gemm_packed(pw, to_dev(q_ref, "i8"), to_dev(xs_ref, "f32"), out_dtype=TORCH[out])
    torch.cuda.synchronize()
    _, y_ref = w4a8_reference(w, q_ref, xs_ref)
    assert_close(host(y), y_ref, out, f"gemm w4a8 out={out}")


@pytest.mark.parametrize("fmt,act_order", [("int4_sym", False), ("int4_zp", True), ("int4_zp", False)])
@pytest.mark.parametrize("m,k,n,win", [(3, 256, 70, (0, 3, 0, 70)), (300, 640, 520, (5, 290, 33, 510)),
                                       (130, 1024, 260, (128, 130, 255, 260)), (129, 4096, 300, (1, 129, 250, 300)),
                                       (64, 2048, 257, (0, 64, 0, 257))])
def test_partials_w4a8_bit_exact(fmt, act_order, m, k, n, win):
    # stress inputs: the full int8 range, every code and zero point
    rng = np.random.default_rng(m + k + n + 5)
    q = synth.random_int8(m + k + 1, m, k)
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    scales = rng.uniform(0.001, 0.02, size=(n, k // 128)).astype(np.float16)
    zeros = rng.integers(0, 16, size=(n, k // 128), dtype=np.uint8) if fmt == "int4_zp" else None
    g_idx = None
    if act_order:
        g_idx = np.empty(k, np.int32)
        g_idx[rng.permutation(k)] = np.arange(k, dtype=np.int32) // 128
    pw = bpw.prepare_packed(bpw.FORMAT_NAMES[fmt], codes, scales, zeros, g_idx, device=DEV)
    m0, m1, n0, n1 = win
    p = bpw.partials(pw, to_dev(q, "i8"), bpw.PATH_GEMM, m0, m1, n0, n1)
    torch.cuda.synchronize()
    z = zeros[n0:n1] if zeros is not None else None
    p_ref = reference.int4_partials(q[m0:m1], codes[n0:n1], z, g_idx)
    np.testing.assert_array_equal(host(p), p_ref)


def test_w4a8_determinism_row_independence_and_poison():
    w, q_ref, xs_ref = w4a8_case("int4_zp", 300, 1024, 520, 441, True, "f16")
    pw = prepare(w)
    q, xs = to_dev(q_ref, "i8"), to_dev(xs_ref, "f32")
    y1 = torch.full((300, 520), float("nan"), dtype=torch.float16, device=DEV)
    bpw.gemm_packed(pw, q, xs, out=y1)
    y2 = bpw.gemm_packed(pw, q, xs)
    q2 = q.clone()
    q2[1:] = torch.randint(-127, 128, q2[1:].shape, device=DEV, dtype=torch.int8)
    y3 = bpw.gemm_packed(pw, q2, xs)
    torch.cuda.synchronize()
    assert torch.isfinite(y1).all()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(y1[0].view(torch.int16), y3[0].view(torch.int16))


@pytest.mark.parametrize("fmt,m,k,n", [("int4_sym", 1, 128, 1), ("int4_zp", 33, 256, 65), ("int4_sym", 129, 128, 257),
                                       ("int4_zp", 128, 384, 256)])
def test_w4a8_degenerate_shapes(fmt, m, k, n):
    # one row / one output column / one group, and exact tile multiples
    w, q_ref, xs_ref = w4a8_case(fmt, m, k, n, 460 + m + n, fmt == "int4_zp", "f16")
    pw = prepare(w)
    y = bpw.gemm_packed(pw, to_dev(q_ref, "i8"), to_dev(xs_ref, "f32"))
    p = bpw.partials(pw, to_dev(q_ref, "i8"), bpw.PATH_GEMM, 0, m, 0, n)
    torch.cuda.synchronize()
    p_ref, y_ref = w4a8_reference(w, q_ref, xs_ref)
    np.testing.assert_array_equal(host(p), p_ref)
    assert_close(host(y), y_ref, "f16", f"w4a8 degenerate {fmt} m={m} k={k} n={n}")


def test_w4a8_refused_by_gemv_entry():
    w, q_ref, xs_ref = w4a8_case("int4_sym", 4, 256, 64, 451, False, "bf16")
    pw = prepare(w)
    with pytest.raises(bpw.BpwError) as e:
        bpw.gemv_packed(pw, to_dev(q_ref, "i8"), to_dev(xs_ref, "f32"))
    assert e.value.status == bpw.EUNSUPPORTED and "bpw_gemm_packed" in str(e.value)


def test_workload_w4a8_prefill_sampled():
    # The 4-bit prefill workload's weights (M=2048, K=4096, N=14336) against
    # its activations quantised to int8 rows.
    w = synth.w4a16_prefill()
    pw = prepare(w)
    q, xs = bpw.quantize_rows(to_dev(w.x, "bf16"))
    y = bpw.gemm_packed(pw, q, xs, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([[0, w.m - 1], rng.choice(w.m, 30, replace=False)]))
    cols = np.unique(np.concatenate([np.arange(64), np.arange(w.n - 64, w.n), rng.choice(w.n, 512, replace=False)]))
    q_ref, xs_ref = quant.quantize_rows(w.x_f32()[rows])
    np.testing.assert_array_equal(host(q)[rows], q_ref)
    _, y_ref = reference.int4_int8_product(q_ref, xs_ref, w.codes[cols], w.scales_f64()[cols])
    assert_close(host(y)[np.ix_(rows, cols)], y_ref, "bf16", "w4a8 prefill sampled")
    for (m0, m1, n0, n1) in [(0, 64, 0, 256), (w.m - 64, w.m, w.n - 256, w.n)]:
        p = bpw.partials(pw, q, bpw.PATH_GEMM, m0, m1, n0, n1)
        torch.cuda.synchronize()
        q_win, _ = quant.quantize_rows(w.x_f32()[m0:m1])
        np.testing.assert_array_equal(host(p), reference.int4_partials(q_win, w.codes[n0:n1]),
                                      err_msg=f"window {(m0, m1, n0, n1)}")


# ------------------------------------------------------------------ non-finite activations
def _with_non_finite(x):
    x = x.copy()
    x[1, 5] = np.nan
    x[3, 0] = np.inf
    x[3, 9] = -np.inf
    return x


def _as_dtype(x, dtype):
    if dtype == "f16":
        xs = x.astype(np.float16)
        return xs, xs.astype(np.float32)
    if dtype == "bf16":
        xs = synth.f32_to_bf16_bits(x)
        return xs, synth.bf16_bits_to_f32(xs)
    return x, x


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("k", [512, 10240])
def test_quantizers_non_finite_blocks(dtype, k):
    # rows 1 and 3 hold a NaN / infinities: their scale is NaN and their codes 0
    rng = np.random.default_rng(k + 3)
    x = _with_non_finite(rng.standard_normal((5, k)).astype(np.float32) * 3)
    xs, xf = _as_dtype(x, dtype)
    q, s = bpw.quantize_rows(to_dev(xs, dtype))
    qg, sg = bpw.quantize_groups(to_dev(xs, dtype))
    torch.cuda.synchronize()
    q_ref, s_ref = quant.quantize_rows(xf)
    qg_ref, sg_ref = quant.quantize_groups(xf)
    assert np.isnan(s_ref[[1, 3]]).all() and np.isnan(sg_ref[1, 0]) and np.isnan(sg_ref[3, 0])
    np.testing.assert_array_equal(host(s).astype(np.float32), s_ref)
    np.testing.assert_array_equal(host(q), q_ref)
    np.testing.assert_array_equal(host(sg).astype(np.float32), sg_ref)
    np.testing.assert_array_equal(host(qg), qg_ref)


def _check_flagged_rows(y_bad, y_clean, bad_rows):
    yb, yc = host(y_bad), host(y_clean)
    assert np.isnan(yb[bad_rows]).all()
    keep = [r for r in range(yb.shape[0]) if r not in bad_rows]
    np.testing.assert_array_equal(yb[keep], yc[keep])


@pytest.mark.parametrize("entry,fmt,m,k,n", [("gemv", "ternary", 1, 4096, 1000), ("gemv", "ternary", 5, 2048, 700),
                                             ("gemv", "ternary", 16, 14336, 300), ("gemm", "ternary", 40, 1024, 520),
                                             ("gemm", "int4_zp", 40, 1024, 520)])
def test_products_of_non_finite_rows_are_nan(entry, fmt, m, k, n):
    # A row with a NaN / infinity quantises to scale NaN, and every output of
    # that row is NaN; the other rows are bit-identical to a run without them.
    rng = np.random.default_rng(m + k + n)
    if fmt == "ternary":
        w = ternary_case(m, k, n, 600 + m)
    else:
        w = w4_case(fmt, m, k, n, 600 + m, True, "f16")
    pw = prepare(w)
    clean = rng.standard_normal((m, k)).astype(np.float32)
    bad_rows = [0] if m == 1 else [1, 3]
    dirty = clean.copy()
    for r in bad_rows:
        dirty[r, (7 * r) % k] = np.nan if r % 2 else np.inf
    fn = bpw.gemv_packed if entry == "gemv" else bpw.gemm_packed
    outs = []
    for xin in (dirty, clean):
        q, xs = bpw.quantize_rows(to_dev(xin, "f32"))
        outs.append(fn(pw, q, xs))
    torch.cuda.synchronize()
    _check_flagged_rows(outs[0], outs[1], bad_rows)
    if entry == "gemv" and fmt == "ternary":
        # per-group scales: only the flagged group is NaN, but it reaches every output of its row
        outs = []
        for xin in (dirty, clean):
            q, xs = bpw.quantize_groups(to_dev(xin, "f32"))
            outs.append(fn(pw, q, xs))
        torch.cuda.synchronize()
        _check_flagged_rows(outs[0], outs[1], bad_rows)


# ------------------------------------------------------------------ one-token complete call
# Ternary weights with fp32 / fp16 / bf16 activations at M = 1: the row quantiser
# runs inside the GEMV launch. q, the row scale and the fold are those of the
# quantiser launch followed by the int8 call, so the output bits must be equal;
# against the oracle (its quantiser, then its product) the usual rule holds.
@pytest.mark.parametrize("x_dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("k,n", [(4096, 14336), (512, 256), (1152, 333), (8192, 130), (12288, 77), (16384, 500),
                                 # N >= 16384: four rows per wave; ragged last workgroup
                                 (4096, 16387), (640, 3)])
def test_fused_quantise_gemv_matches_two_launches(x_dtype, k, n):
    w = ternary_case(1, k, n, 900 + k + n)
    pw = prepare(w)
    x_np = w.x.astype(np.float16).astype(np.float32) if x_dtype == "f16" else w.x
    if x_dtype == "bf16":
        x_np = (w.x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)   # exact bf16 values
    x32 = to_dev(x_np, "f32")
    x = x32.to(TORCH[x_dtype])
    assert torch.equal(x.float(), x32)
    y1 = torch.full((1, n), float("nan"), dtype=torch.float16, device=DEV)
    bpw.gemv_packed(pw, x, out=y1)
    q, xs = bpw.quantize_rows(x)
    y2 = bpw.gemv_packed(pw, q, xs)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    q_ref, xs_ref = quant.quantize_rows(x_np)
    _, y_ref = reference.ternary_int8_product(q_ref, xs_ref, w.codes, w.scales)
    assert_close(host(y1), y_ref, "f16", f"fused quantise + GEMV {x_dtype} k={k} n={n}")


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_fused_quantise_gemv_outputs_and_special_rows(out):
    # every output dtype; an all-zero row gives zeros; a row with a NaN or an
    # infinity gives a NaN row, as the two-launch call does
    k, n = 4096, 700
    w = ternary_case(1, k, n, 931)
    pw = prepare(w)
    x = to_dev(w.x, "f32")
    y = bpw.gemv_packed(pw, x, out_dtype=TORCH[out])
    q, xs = bpw.quantize_rows(x)
    y2 = bpw.gemv_packed(pw, q, xs, out_dtype=TORCH[out])
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    z = bpw.gemv_packed(pw, torch.zeros_like(x))
    torch.cuda.synchronize()
    assert not torch.any(z.float() != 0)
    for bad in (float("nan"), float("inf"), float("-inf")):
        xb = x.clone()
        xb[0, 1234] = bad
        yb = bpw.gemv_packed(pw, xb)
        torch.cuda.synchronize()
        assert torch.isnan(yb).all()


def test_fused_quantise_gemv_through_scratch_entry():
    w = ternary_case(1, 4096, 1000, 932)
    pw = prepare(w)
    x = to_dev(w.x, "f32")
    y1 = bpw.gemv_packed_scratch(pw, x)
    y2 = bpw.gemv_packed(pw, x)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


# ------------------------------------------------------------------ graph replay
def _graph_cases():
    cases = []
    # ternary decode: row kernel, skinny, split-K (two launches + workspace), group scales
    for m, k, n in [(1, 4096, 1000), (5, 2048, 700), (16, 14336, 512)]:
        w = ternary_case(m, k, n, 700 + m)
        cases.append(("t2 gemv m=%d k=%d" % (m, k), w, "gemv", "rows"))
    cases.append(("t2 gemv groups", ternary_case(3, 4096, 300, 710), "gemv", "groups"))
    cases.append(("t2 gemm", ternary_case(200, 1024, 520, 711), "gemm", "rows"))
    # 4-bit: act-order gather + GEMV, bf16 GEMM, W4A8 GEMM (nibble reorder + GEMM)
    cases.append(("w4 gemv act", w4_case("int4_zp", 8, 5120, 700, 712, True, "f16"), "gemv", "float"))
    cases.append(("w4 gemm", w4_case("int4_sym", 300, 1024, 520, 713, False, "bf16"), "gemm", "float"))
    cases.append(("w4a8 gemm", w4_case("int4_zp", 200, 1024, 520, 714, True, "f16"), "gemm", "rows"))
    # the one-launch complete call (fp32 row quantised in the GEMV); 4-bit long K: the M = 1
    # K split over waves, and split-K slices + reduce behind the act-order gather at M = 8
    cases.append(("t2 fused", ternary_case(1, 4096, 1000, 715), "gemv", "fp32"))
    cases.append(("w4 gemv long k", w4_case("int4_zp", 1, 13824, 500, 716, False, "f16"), "gemv", "float"))
    cases.append(("w4 gemv split", w4_case("int4_zp", 8, 13824, 700, 717, True, "f16"), "gemv", "float"))
    return cases


def test_graph_replay_matches_eager():
    # Each entry point captured into a HIP graph (the form the benchmark times),
    # replayed three times with eager calls of the library in between, matches
    # the eager result bit for bit on every replay.
    for name, w, entry, act in _graph_cases():
        pw = prepare(w)
        fn = bpw.gemv_packed if entry == "gemv" else bpw.gemm_packed
        if act == "float":
            args = (to_dev(w.x, w.x_dtype),)
            xd = bpw.dtype_code(TORCH[w.x_dtype])
        elif act == "fp32":
            args = (to_dev(w.x_f32(), "f32"),)
            xd = bpw.F32
        else:
            x = to_dev(w.x_f32(), "f32")
            args = bpw.quantize_rows(x) if act == "rows" else bpw.quantize_groups(x)
            xd = bpw.I8G if act == "groups" else bpw.I8
        path = bpw.PATH_GEMV if entry == "gemv" else bpw.PATH_GEMM
        need = bpw.workspace_size(pw, w.m, xd, path)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV) if need else None
        eager = fn(pw, *args, workspace=ws)
        torch.cuda.synchronize()
        out = torch.full_like(eager, float("nan"))
        stream = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            fn(pw, *args, out=out, workspace=ws)
        for rep in range(3):
            out.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16) if out.element_size() == 2 else out.view(torch.int32),
                               eager.view(torch.int16) if eager.element_size() == 2 else eager.view(torch.int32)), \
                f"{name}: replay {rep} differs from the eager result"
            fn(pw, *args, workspace=ws)                     # eager work of the library between replays
            torch.cuda.synchronize()


def test_two_streams_with_their_own_workspaces():
    # The library keeps no state between calls: the same entry points running
    # on two streams at once, each with its own workspace, give the
    # single-stream results bit for bit.
    cases = []
    for m, k, n, seed in [(16, 14336, 512, 801), (200, 1024, 520, 802)]:
        w = ternary_case(m, k, n, seed)
        pw = prepare(w)
        q, xs = bpw.quantize_rows(to_dev(w.x_f32(), "f32"))
        fn = bpw.gemv_packed if m <= 32 else bpw.gemm_packed
        path = bpw.PATH_GEMV if m <= 32 else bpw.PATH_GEMM
        need = bpw.workspace_size(pw, m, bpw.I8, path)
        ref = fn(pw, q, xs)
        cases.append((fn, pw, q, xs, need, ref))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[], []]
    wss = [[torch.empty(max(c[4], 1), dtype=torch.uint8, device=DEV) for c in cases] for _ in streams]
    for it in range(20):
        for si, st in enumerate(streams):
            with torch.cuda.stream(st):
                for ci, (fn, pw, q, xs, need, ref) in enumerate(cases):
                    outs[si].append((ci, fn(pw, q, xs, workspace=wss[si][ci] if need else None)))
    torch.cuda.synchronize()
    for si in range(2):
        for ci, y in outs[si]:
            assert torch.equal(y.view(torch.int16), cases[ci][5].view(torch.int16)), f"stream {si} case {ci}"
