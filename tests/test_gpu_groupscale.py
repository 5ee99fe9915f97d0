"""GPU parity of the per-(row, group) activation paths of the prefill GEMM.

* The group quantiser with exact group sums ("TensorFold PR #1176", "What
  changes": int8 codes, a = amax / 127 and the exact fp32 sum per group, groups
  following the weight's act-order permutation): codes, scales and sums bit
  for bit against oracle.quant.quantize_groups_sums.
* 4-bit weights x those activations in the page's affine form
  (s * a * (code . q) + b * sum(x) per group): the raw-code int32 dots bit for
  bit (bpw_partials, BPW_PATH_GEMM_RAW) and the outputs within oracle.compare's
  rule against oracle.reference.w4a8_affine_product.
* Ternary weights x int8 with one scale per (row, 128-group) on the prefill
  kernel ("Kernel experiments", Test 7's per-group fold): partials bit for bit,
  outputs against ternary_int8_product_group_scales.
"""
import numpy as np
import pytest
import torch

import bit_packed_weight_amd as bpw
import synth
from oracle import compare, quant, reference

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def to_dev(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if t.is_floating_point() else t.cpu().numpy()


def assert_close(y, y_ref, dtype, what):
    r = compare.compare(y, y_ref, dtype)
    assert r["ok"], f"{what}: {r}"
    return r


def prepare(w):
    fmt = bpw.FORMAT_NAMES[w.fmt]
    sd = bpw.F16 if w.scale_dtype == "f16" else bpw.BF16
    zeros = w.zeros if w.fmt == "int4_zp" else None
    return bpw.prepare_packed(fmt, w.codes, w.scales, zeros, w.g_idx, scale_dtype=sd, device=DEV)


def w4_case(fmt, m, k, n, seed, act_order, x_dtype):
    if fmt == "int4_zp":
        return synth.int4_zp_actorder(f"g{m}x{k}x{n}", seed, m, k, n, act_order=act_order, x_dtype=x_dtype)
    return synth.int4_sym(f"g{m}x{k}x{n}", seed, m, k, n, x_dtype=x_dtype)


def perm_of(w):
    return None if w.g_idx is None else reference.act_order_perm(w.g_idx, w.k)


def quantise_both(w, pw):
    """GPU quantiser on the workload's activations (its storage dtype) and the oracle's;
    codes, scales and sums must agree bit for bit."""
    q, xss = bpw.quantize_groups_sums(to_dev(w.x, w.x_dtype), pw.perm)
    torch.cuda.synchronize()
    q_ref, a_ref, s_ref = quant.quantize_groups_sums(w.x_f32(), perm_of(w))
    np.testing.assert_array_equal(host(q), q_ref)
    np.testing.assert_array_equal(host(xss)[..., 0], a_ref)
    np.testing.assert_array_equal(host(xss)[..., 1], s_ref)
    return q, xss, q_ref, a_ref, s_ref


# ------------------------------------------------------------------ quantiser with sums
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("m,k,act", [(1, 512, False), (5, 4096, True), (3, 1024, False), (64, 2048, True)])
def test_quantize_groups_sums_bit_exact(dtype, m, k, act):
    rng = np.random.default_rng(m * 13 + k + act)
    x = (rng.standard_normal((m, k)) * rng.uniform(0.01, 50, size=(m, 1))).astype(np.float32)
    x[0, :6] = [127.0, 2.5, -3.5, 0.5, -0.5, 126.5]        # exact ties once a = 1
    if m > 2:
        x[2, 128:256] = 0.0                                 # an all-zero group
    if m > 4 and dtype == "f32":
        x[4, :128] = 0.0                                    # sums on an fp32 midpoint, above and below it
        x[4, :3] = [1.0, 2.0 ** -24, 2.0 ** -60]
        x[4, 128:131] = [1.0, 2.0 ** -24, -(2.0 ** -60)]
        x[4, 256:259] = [1.0, 2.0 ** -24, 0.0]
        x[4, 384:512] = (rng.standard_normal(128) * np.exp2(rng.integers(-30, 30, 128))).astype(np.float32)
    if dtype == "f16":
        xs = x.astype(np.float16)
        xf = xs.astype(np.float32)
    elif dtype == "bf16":
        xs = synth.f32_to_bf16_bits(x)
        xf = synth.bf16_bits_to_f32(xs)
    else:
        xs = xf = x
    perm = None
    perm_dev = None
    if act:
        pi = rng.permutation(k)
        g_idx = np.empty(k, np.int32)
        g_idx[pi] = np.arange(k, dtype=np.int32) // 128
        perm = reference.act_order_perm(g_idx, k)
        perm_dev = torch.from_numpy(perm.astype(np.int32)).to(DEV)
    q, xss = bpw.quantize_groups_sums(to_dev(xs, dtype), perm_dev)
    torch.cuda.synchronize()
    q_ref, a_ref, s_ref = quant.quantize_groups_sums(xf, perm)
    np.testing.assert_array_equal(host(q), q_ref)
    np.testing.assert_array_equal(host(xss)[..., 0], a_ref)
    np.testing.assert_array_equal(host(xss)[..., 1], s_ref)


def test_quantize_groups_sums_non_finite():
    x = np.random.default_rng(5).standard_normal((4, 512)).astype(np.float32)
    x[1, 5] = np.nan
    x[3, 300] = np.inf
    q, xss = bpw.quantize_groups_sums(to_dev(x, "f32"))
    torch.cuda.synchronize()
    q_ref, a_ref, s_ref = quant.quantize_groups_sums(x)
    np.testing.assert_array_equal(host(q), q_ref)
    h = host(xss)
    np.testing.assert_array_equal(np.isnan(h[..., 0]), np.isnan(a_ref))
    np.testing.assert_array_equal(np.isnan(h[..., 1]), np.isnan(s_ref))
    ok = ~np.isnan(a_ref)
    np.testing.assert_array_equal(h[..., 0][ok], a_ref[ok])
    np.testing.assert_array_equal(h[..., 1][ok], s_ref[ok])


# ------------------------------------------------------------------ affine 4-bit x int8
@pytest.mark.parametrize("fmt,x_dtype,act_order", [("int4_sym", "bf16", False), ("int4_zp", "f16", True),
                                                   ("int4_zp", "f16", False), ("int4_sym", "f16", True)])
@pytest.mark.parametrize("m,k,n", [(1, 256, 300), (130, 1024, 520), (300, 640, 257), (64, 128, 256),
                                   (129, 2048, 1000)])
def test_gemm_affine_w4a8_parity(fmt, x_dtype, act_order, m, k, n):
    w = w4_case(fmt, m, k, n, 700 + m + k + n, act_order, x_dtype)
    pw = prepare(w)
    q, xss, q_ref, a_ref, s_ref = quantise_both(w, pw)
    y = bpw.gemm_packed(pw, q, xss, out_dtype=TORCH[x_dtype])
    d = bpw.partials(pw, q, bpw.PATH_GEMM_RAW, 0, m, 0, n)
    torch.cuda.synchronize()
    zeros = w.zeros if w.fmt == "int4_zp" else None
    d_ref, y_ref = reference.w4a8_affine_product(q_ref, a_ref, s_ref, w.codes, w.scales_f64(), zeros, w.g_idx)
    np.testing.assert_array_equal(host(d), d_ref)
    assert_close(host(y), y_ref, x_dtype, f"affine w4a8 {fmt} m={m} k={k} n={n}")


@pytest.mark.parametrize("out", ["f32", "f16", "bf16"])
def test_gemm_affine_w4a8_output_dtypes(out):
    w = w4_case("int4_zp", 70, 512, 300, 771, True, "f16")
    pw = prepare(w)
    q, xss, q_ref, a_ref, s_ref = quantise_both(w, pw)
    y = bpw.gemm_packed(pw, q, xss, out_dtype=TORCH[out])
    torch.cuda.synchronize()
    _, y_ref = reference.w4a8_affine_product(q_ref, a_ref, s_ref, w.codes, w.scales_f64(), w.zeros, w.g_idx)
    assert_close(host(y), y_ref, out, f"affine w4a8 out {out}")


def test_gemm_affine_w4a8_determinism_and_row_independence():
    """Bit-identical repeats, and a row's output bits do not depend on the rows beside it
    (the page's own check for its int8 prompt kernels)."""
    w = w4_case("int4_sym", 200, 1024, 600, 772, False, "bf16")
    pw = prepare(w)
    q, xss = bpw.quantize_groups_sums(to_dev(w.x, "bf16"))
    y1 = bpw.gemm_packed(pw, q, xss)
    y2 = bpw.gemm_packed(pw, q, xss)
    rows = [0, 57, 128, 199]
    y3 = bpw.gemm_packed(pw, q[rows].contiguous(), xss[rows].contiguous())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(y1), host(y2))
    np.testing.assert_array_equal(host(y1)[rows], host(y3))


def test_gemm_affine_w4a8_non_finite_rows():
    w = w4_case("int4_zp", 6, 512, 300, 773, False, "f16")
    x = w.x.astype(np.float32)
    x[2, 7] = np.nan
    x[4, 400] = np.inf
    pw = prepare(w)
    q, xss = bpw.quantize_groups_sums(to_dev(x, "f32"))
    y = host(bpw.gemm_packed(pw, q, xss, out_dtype=torch.float32))
    torch.cuda.synchronize()
    assert np.isnan(y[2]).all() and np.isnan(y[4]).all()
    assert np.isfinite(y[[0, 1, 3, 5]]).all()


def test_workload_affine_w4a8_prefill_sampled():
    """The 4-bit prefill workload (M=2048, K=4096, N=14336, symmetric codes, bf16
    scales) in the affine form: quantiser bit for bit on sampled rows, outputs on
    sampled rows x columns, raw-code partials on corner and random windows."""
    w = synth.w4a16_prefill()
    pw = prepare(w)
    q, xss = bpw.quantize_groups_sums(to_dev(w.x, "bf16"))
    y = bpw.gemm_packed(pw, q, xss, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([[0, w.m - 1], rng.choice(w.m, 30, replace=False)]))
    cols = np.unique(np.concatenate([np.arange(64), np.arange(w.n - 64, w.n), rng.choice(w.n, 512, replace=False)]))
    q_ref, a_ref, s_ref = quant.quantize_groups_sums(w.x_f32()[rows])
    np.testing.assert_array_equal(host(q)[rows], q_ref)
    np.testing.assert_array_equal(host(xss)[rows], np.stack([a_ref, s_ref], -1))
    _, y_ref = reference.w4a8_affine_product(q_ref, a_ref, s_ref, w.codes[cols], w.scales_f64()[cols])
    assert_close(host(y)[np.ix_(rows, cols)], y_ref, "bf16", "affine w4a8 prefill sampled")
    wins = [(0, 64, 0, 256), (w.m - 64, w.m, w.n - 256, w.n)]
    for _ in range(2):
        m0, n0 = int(rng.integers(0, w.m - 64)), int(rng.integers(0, w.n - 256))
        wins.append((m0, m0 + 64, n0, n0 + 256))
    for (m0, m1, n0, n1) in wins:
        d = bpw.partials(pw, q, bpw.PATH_GEMM_RAW, m0, m1, n0, n1)
        torch.cuda.synchronize()
        q_win, _, _ = quant.quantize_groups_sums(w.x_f32()[m0:m1])
        np.testing.assert_array_equal(host(d), reference.int4_raw_partials(q_win, w.codes[n0:n1]),
                                      err_msg=f"window {(m0, m1, n0, n1)}")


# ------------------------------------------------------------------ ternary x int8, per-group scales
@pytest.mark.parametrize("m,k,n", [(1, 256, 300), (130, 1024, 520), (300, 640, 257), (64, 128, 256),
                                   (129, 2048, 1000)])
def test_gemm_ternary_group_scales_parity(m, k, n):
    w = synth.ternary_int8(f"tg{m}x{k}x{n}", 800 + m + k + n, m, k, n, 0.005, 0.05, "f16")
    pw = prepare(w)
    q, xs = bpw.quantize_groups(to_dev(w.x, "f32"))
    y = bpw.gemm_packed(pw, q, xs)
    p = bpw.partials(pw, q, bpw.PATH_GEMM_RAW, 0, m, 0, n)
    torch.cuda.synchronize()
    q_ref, xs_ref = quant.quantize_groups(w.x)
    np.testing.assert_array_equal(host(q), q_ref)
    p_ref, y_ref = reference.ternary_int8_product_group_scales(q_ref, xs_ref, w.codes, w.scales)
    np.testing.assert_array_equal(host(p), p_ref)
    assert_close(host(y), y_ref, "f16", f"ternary group scales gemm m={m} k={k} n={n}")


def test_gemv_entry_routes_group_scales_beyond_32_rows():
    """Above 32 rows the decode entry takes the prefill kernel: same bits as the GEMM entry."""
    w = synth.ternary_int8("tg40", 811, 40, 1024, 700, 0.005, 0.05, "f16")
    pw = prepare(w)
    q, xs = bpw.quantize_groups(to_dev(w.x, "f32"))
    y1 = bpw.gemv_packed(pw, q, xs)
    y2 = bpw.gemm_packed(pw, q, xs)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(y1), host(y2))
    q_ref, xs_ref = quant.quantize_groups(w.x)
    _, y_ref = reference.ternary_int8_product_group_scales(q_ref, xs_ref, w.codes, w.scales)
    assert_close(host(y1), y_ref, "f16", "ternary group scales via gemv entry")


def test_workload_ternary_group_scales_prefill_sampled():
    """The ternary prefill workload's weights (K=8192, N=28672) against its first 512
    rows with one activation scale per (row, group): sampled outputs and windows."""
    w = synth.leading_rows(synth.ternary_prefill(), 512)
    pw = prepare(w)
    q, xs = bpw.quantize_groups(to_dev(w.x, "f32"))
    y = bpw.gemm_packed(pw, q, xs)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, w.m - 1], rng.choice(w.m, 16, replace=False)]))
    cols = np.unique(np.concatenate([np.arange(32), np.arange(w.n - 32, w.n), rng.choice(w.n, 256, replace=False)]))
    q_ref, xs_ref = quant.quantize_groups(w.x[rows])
    _, y_ref = reference.ternary_int8_product_group_scales(q_ref, xs_ref, w.codes[cols], w.scales[cols])
    assert_close(host(y)[np.ix_(rows, cols)], y_ref, "f16", "ternary group scales prefill sampled")
    for (m0, m1, n0, n1) in [(0, 32, 0, 128), (w.m - 32, w.m, w.n - 128, w.n)]:
        p = bpw.partials(pw, q, bpw.PATH_GEMM_RAW, m0, m1, n0, n1)
        torch.cuda.synchronize()
        q_win, _ = quant.quantize_groups(w.x[m0:m1])
        np.testing.assert_array_equal(host(p), reference.ternary_partials(q_win, w.codes[n0:n1]))
