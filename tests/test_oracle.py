"""Pins for the CPU oracle: each check compares it with something other than itself.

Brute force with Python integers / fractions, closed forms, the pages' printed
mappings (tests/golden), invariants and negative controls. CPU only.
"""
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats, quant, reference
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ------------------------------------------------------------------ decode
def _digits_base4(b):
    out = []
    for _ in range(4):
        b, d = divmod(b, 4)
        out.append(d)
    return out


def test_ternary_unpack_all_bytes_matches_base4_digits():
    plane = np.arange(256, dtype=np.uint8).reshape(256, 1)
    codes = formats.unpack_ternary(plane, 4)
    for b in range(256):
        assert list(codes[b]) == _digits_base4(b)


def test_ternary_values_match_add_xor_expansion_all_bytes():
    # "Kernel experiments", Test 1: spread the four codes to byte lanes, add
    # 0x7F7F7F7F, XOR 0x80808080 -> signed -1/0/1/2 per byte.
    plane = np.arange(256, dtype=np.uint8).reshape(256, 1)
    vals = formats.ternary_value(formats.unpack_ternary(plane, 4))
    for p in range(256):
        spread = (p & 3) | ((p << 6) & 0x300) | ((p << 12) & 0x30000) | ((p << 18) & 0x3000000)
        word = ((spread + 0x7F7F7F7F) & 0xFFFFFFFF) ^ 0x80808080
        signed = [struct.unpack("b", bytes([(word >> (8 * t)) & 0xFF]))[0] for t in range(4)]
        assert list(vals[p]) == signed


def test_ternary_values_match_byte_select_table_all_bytes():
    # "Kernel experiments", Test 16 CUDA decoder: byte_perm(0x020100ff) with the code as index.
    table = (0x020100FF).to_bytes(4, "little")
    plane = np.arange(256, dtype=np.uint8).reshape(256, 1)
    vals = formats.ternary_value(formats.unpack_ternary(plane, 4))
    for b in range(256):
        sel = [(b >> (2 * t)) & 3 for t in range(4)]
        expect = [struct.unpack("b", bytes([table[s]]))[0] for s in sel]
        assert list(vals[b]) == expect


def test_golden_code_values():
    rows = _golden_rows("pq2_code_values.txt")
    assert len(rows) == 4
    for code, plus127, table_hex, value in rows:
        code, plus127, value = int(code), int(plus127), int(value)
        assert code + 127 == plus127
        assert struct.unpack("b", bytes([plus127 ^ 0x80]))[0] == value
        assert struct.unpack("b", bytes([int(table_hex, 16)]))[0] == value
        assert int(formats.ternary_value(np.array([code], np.uint8))[0]) == value


def test_ternary_pack_roundtrip_and_group_position():
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 4, size=(5, 256), dtype=np.uint8)
    plane = formats.pack_ternary(codes)
    assert plane.shape == (5, 64)
    np.testing.assert_array_equal(formats.unpack_ternary(plane, 256), codes)
    # weight k = 128 g + 4 j + t sits in byte 32 g + j at bits 2t
    for n in range(5):
        for k in range(256):
            g, r = divmod(k, 128)
            j, t = divmod(r, 4)
            assert (int(plane[n, 32 * g + j]) >> (2 * t)) & 3 == codes[n, k]


def test_int4_unpack_all_bytes_matches_divmod():
    plane = np.arange(256, dtype=np.uint8).reshape(256, 1)
    codes = formats.unpack_int4(plane, 2)
    for b in range(256):
        hi, lo = divmod(b, 16)
        assert list(codes[b]) == [lo, hi]
    rng = np.random.default_rng(3)
    c = rng.integers(0, 16, size=(3, 64), dtype=np.uint8)
    np.testing.assert_array_equal(formats.unpack_int4(formats.pack_int4(c), 64), c)
    z = rng.integers(0, 16, size=(3, 5), dtype=np.uint8)
    np.testing.assert_array_equal(formats.unpack_zeros(formats.pack_zeros(z), 5), z)


def test_pq2_block_split_against_struct_encoding():
    rng = np.random.default_rng(11)
    n, g = 3, 2
    raw = bytearray()
    want_scales, want_codes = [], []
    for _ in range(n):
        row_s, row_c = [], []
        for _ in range(g):
            s = float(np.float16(rng.uniform(0.005, 0.05)))
            codes = [int(v) for v in rng.integers(0, 256, size=32)]
            raw += struct.pack("<e", s) + bytes(codes)
            row_s.append(s)
            row_c += codes
        want_scales.append(row_s)
        want_codes.append(row_c)
    arr = np.frombuffer(bytes(raw), np.uint8).reshape(n, g * 34)
    plane, scales = formats.split_pq2_blocks(arr)
    np.testing.assert_array_equal(plane, np.array(want_codes, np.uint8))
    np.testing.assert_array_equal(scales.astype(np.float64), np.array(want_scales))
    np.testing.assert_array_equal(formats.join_pq2_blocks(plane, scales), arr)


# ------------------------------------------------------------------ partials
def _brute_partials(q, plane, k):
    m, n, g = q.shape[0], plane.shape[0], k // 128
    out = np.zeros((m, n, g), dtype=np.int64)
    for mi in range(m):
        for ni in range(n):
            for kk in range(k):
                byte = int(plane[ni, kk // 4])
                code = _digits_base4(byte)[kk % 4]
                out[mi, ni, kk // 128] += int(q[mi, kk]) * (code - 1)
    return out


@pytest.mark.parametrize("m,k,n", [(1, 128, 3), (3, 256, 5), (2, 128, 1)])
def test_ternary_partials_brute_force(m, k, n):
    rng = np.random.default_rng(m * 100 + k + n)
    q = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    plane = rng.integers(0, 256, size=(n, k // 4), dtype=np.uint8)   # every code incl. 3
    p = reference.ternary_partials(q, formats.unpack_ternary(plane, k))
    np.testing.assert_array_equal(p, _brute_partials(q, plane, k))


def test_masked_plane_identity():
    # "Kernel experiments", Test 21: plane s of a byte is byte & (3 << 2s) = code * 4**s
    # (plane 3 pre-shifted by 2); plane-ordered activations (position (i%4)*32 + i//4),
    # shifted products, minus the group sum of q, equal the integer group dot.
    rng = np.random.default_rng(5)
    m, n, k = 4, 6, 512
    q = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    plane = rng.integers(0, 256, size=(n, k // 4), dtype=np.uint8)
    p = reference.ternary_partials(q, formats.unpack_ternary(plane, k))
    for g in range(k // 128):
        qg = q[:, 128 * g:128 * (g + 1)].astype(np.int64)
        qp = np.empty_like(qg)
        i = np.arange(128)
        qp[:, (i % 4) * 32 + i // 4] = qg
        packed = plane[:, 32 * g:32 * (g + 1)].astype(np.int64)
        q0, q1, q2, q3 = (qp[:, 32 * s:32 * (s + 1)] for s in range(4))
        part = (packed & 0x03) @ q0.T
        part += ((packed & 0x0C) @ q1.T) >> 2
        part += ((packed & 0x30) @ q2.T) >> 4
        part += (((packed >> 2) & 0x30) @ q3.T) >> 4
        part -= qg.sum(axis=1)[None, :]
        np.testing.assert_array_equal(part.T, p[:, :, g])


# ------------------------------------------------------------------ float products
def _fraction_product(x, codes, scales, values_fn):
    m, k = x.shape
    n = codes.shape[0]
    y = [[Fraction(0)] * n for _ in range(m)]
    for mi in range(m):
        for ni in range(n):
            acc = Fraction(0)
            for kk in range(k):
                w = Fraction(int(values_fn(codes[ni, kk]))) * Fraction(float(scales[ni, kk // 128]))
                acc += Fraction(float(x[mi, kk])) * w
            y[mi][ni] = acc
    return y


def test_ternary_float_product_exact_on_power_of_two_scales():
    rng = np.random.default_rng(2)
    m, k, n = 2, 256, 3
    codes = rng.integers(0, 4, size=(n, k), dtype=np.uint8)
    scales = np.ldexp(1.0, rng.integers(-8, -2, size=(n, k // 128))).astype(np.float16)
    x = rng.integers(-40, 41, size=(m, k)).astype(np.float32)
    y = reference.product(x, reference.weights_ternary(codes, scales))
    want = _fraction_product(x, codes, scales, lambda c: int(c) - 1)
    for mi in range(m):
        for ni in range(n):
            assert Fraction(float(y[mi, ni])) == want[mi][ni]


def test_ternary_float_product_random_within_1e12():
    rng = np.random.default_rng(9)
    m, k, n = 2, 256, 3
    codes = rng.integers(0, 3, size=(n, k), dtype=np.uint8)
    scales = rng.uniform(0.005, 0.05, size=(n, k // 128)).astype(np.float16)
    x = rng.standard_normal((m, k)).astype(np.float32)
    y = reference.product(x, reference.weights_ternary(codes, scales))
    want = _fraction_product(x, codes, scales, lambda c: int(c) - 1)
    for mi in range(m):
        for ni in range(n):
            assert abs(Fraction(float(y[mi, ni])) - want[mi][ni]) <= Fraction(1, 10**12) * abs(want[mi][ni])


def test_int8_product_single_group_closed_form():
    # K = 128: y = xs * ws * P with P the one integer group dot.
    rng = np.random.default_rng(4)
    q = rng.integers(-127, 128, size=(2, 128), dtype=np.int8)
    codes = rng.integers(0, 3, size=(3, 128), dtype=np.uint8)
    ws = rng.uniform(0.01, 0.05, size=(3, 1)).astype(np.float16)
    xs = np.array([0.25, 0.0078125], np.float32)
    p, y = reference.ternary_int8_product(q, xs, codes, ws)
    for mi in range(2):
        for ni in range(3):
            dot = sum(int(q[mi, kk]) * (int(codes[ni, kk]) - 1) for kk in range(128))
            assert p[mi, ni, 0] == dot
            assert Fraction(float(y[mi, ni])) == Fraction(float(xs[mi])) * Fraction(float(ws[ni, 0])) * dot


def test_int8_product_unit_scales_is_sum_of_partials():
    rng = np.random.default_rng(6)
    q = rng.integers(-127, 128, size=(3, 512), dtype=np.int8)
    codes = rng.integers(0, 3, size=(4, 512), dtype=np.uint8)
    p, y = reference.ternary_int8_product(q, np.ones(3, np.float32), codes, np.ones((4, 4), np.float16))
    np.testing.assert_array_equal(y, p.sum(axis=2).astype(np.float64))
    # and equals the dense integer product with values code - 1
    dense = q.astype(np.int64) @ (codes.astype(np.int64) - 1).T
    np.testing.assert_array_equal(p.sum(axis=2), dense)


def test_int8_product_group_scale_variant_reduces_to_row_scales():
    rng = np.random.default_rng(8)
    q = rng.integers(-127, 128, size=(2, 384), dtype=np.int8)
    codes = rng.integers(0, 3, size=(3, 384), dtype=np.uint8)
    ws = rng.uniform(0.01, 0.05, size=(3, 3)).astype(np.float16)
    xs = np.array([0.5, 0.125], np.float32)
    _, y1 = reference.ternary_int8_product(q, xs, codes, ws)
    _, y2 = reference.ternary_int8_product_group_scales(q, np.repeat(xs[:, None], 3, 1), codes, ws)
    np.testing.assert_array_equal(y1, y2)


def _fraction_group_scale_product(q, xs, codes, ws):
    """y[m][n] = sum over k of q[m,k] * (code[n,k] - 1) * xs[m, k // 128] * ws[n, k // 128],
    weight by weight in exact rationals ("Kernel experiments", Test 6: one activation
    scale per group of 128, folded with the weight scale of the same group)."""
    m, k = q.shape
    n = codes.shape[0]
    out = [[Fraction(0)] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for kk in range(k):
                g = kk // 128
                acc += (Fraction(int(q[i, kk])) * (int(codes[j, kk]) - 1) * Fraction(float(xs[i, g]))
                        * Fraction(float(ws[j, g])))
            out[i][j] = acc
    return out


def test_int8_product_group_scales_fraction_brute_force():
    """Distinct scales in every (row, group) and (weight row, group): a paired-up group
    index (reversed, shifted, or the row scale of group 0 for all) must fail."""
    rng = np.random.default_rng(9)
    m, k, n = 3, 384, 4
    q = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    codes = rng.integers(0, 4, size=(n, k), dtype=np.uint8)       # code 3 (+2) included
    ws = rng.uniform(0.01, 0.05, size=(n, 3)).astype(np.float16)
    xs = rng.uniform(0.001, 0.1, size=(m, 3)).astype(np.float32)
    assert len(np.unique(xs)) == xs.size and len(np.unique(ws)) == ws.size
    exact = _fraction_group_scale_product(q, xs, codes, ws)
    p, y = reference.ternary_int8_product_group_scales(q, xs, codes, ws)
    for i in range(m):
        for j in range(n):
            assert abs(Fraction(float(y[i, j])) - exact[i][j]) <= abs(exact[i][j]) * Fraction(1, 10 ** 12)
    # partials by brute force too
    np.testing.assert_array_equal(p, _brute_partials(q, formats.pack_ternary(codes), k))

    def far(yy):
        return max(abs(Fraction(float(yy[i, j])) - exact[i][j]) / abs(exact[i][j])
                   for i in range(m) for j in range(n)) > Fraction(1, 1000)
    for bad in (xs[:, ::-1], np.roll(xs, 1, axis=1), np.repeat(xs[:, :1], 3, axis=1)):
        _, yb = reference.ternary_int8_product_group_scales(q, np.ascontiguousarray(bad), codes, ws)
        assert far(yb)
    _, yb = reference.ternary_int8_product_group_scales(q, xs, codes, np.ascontiguousarray(ws[:, ::-1]))
    assert far(yb)


# ------------------------------------------------------------------ act order / zero points
def _valid_gidx(rng, k):
    pi = rng.permutation(k)
    g = np.empty(k, np.int32)
    g[pi] = np.arange(k) // 128
    return g


def test_act_order_invariant_exact_on_integer_data():
    rng = np.random.default_rng(12)
    m, k, n = 3, 512, 4
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    zeros = rng.integers(0, 16, size=(n, 4), dtype=np.uint8)
    scales = np.ldexp(1.0, rng.integers(-9, -5, size=(n, 4))).astype(np.float16)
    g_idx = _valid_gidx(rng, k)
    x = rng.integers(-8, 9, size=(m, k)).astype(np.float16)
    w = reference.weights_int4(codes, scales, zeros, g_idx)
    perm = reference.act_order_perm(g_idx, k)
    assert np.array_equal(g_idx[perm], np.arange(k) // 128)
    # sorted-order weights use group j // 128 for column j
    w_sorted = reference.weights_int4(codes[:, perm], scales, zeros, None)
    np.testing.assert_array_equal(w_sorted, w[:, perm])
    y = reference.product(x, w)
    y_perm = reference.product(x[:, perm], w_sorted)
    np.testing.assert_array_equal(y, y_perm)
    # brute force on one element
    acc = Fraction(0)
    for kk in range(k):
        gi = int(g_idx[kk])
        acc += Fraction(float(x[1, kk])) * (int(codes[2, kk]) - int(zeros[2, gi])) * Fraction(float(scales[2, gi]))
    assert Fraction(float(y[1, 2])) == acc


def test_act_order_negative_controls():
    # mate PR: a skipped gather and a k // group scale index both change the answer.
    wl = synth.int4_zp_actorder("t", 21, 2, 512, 8)
    x = wl.x.astype(np.float64)
    w = reference.weights_int4(wl.codes, wl.scales, wl.zeros, wl.g_idx)
    perm = reference.act_order_perm(wl.g_idx, wl.k)
    w_sorted = reference.weights_int4(wl.codes[:, perm], wl.scales, wl.zeros, None)
    y = reference.product(x, w)
    np.testing.assert_allclose(reference.product(x[:, perm], w_sorted), y, rtol=1e-12, atol=1e-12)
    skipped = reference.product(x, w_sorted)
    canonical = reference.product(x, reference.weights_int4(wl.codes, wl.scales, wl.zeros, None))
    scale = np.abs(y).max()
    assert np.abs(skipped - y).max() > 0.1 * scale
    assert np.abs(canonical - y).max() > 0.1 * scale


def test_act_order_refuses_malformed_gidx():
    k = 256
    g = np.repeat(np.arange(2, dtype=np.int32), 128)
    reference.act_order_perm(g, k)
    bad = g.copy()
    bad[0] = 1          # group 0: 127 members, group 1: 129
    with pytest.raises(ValueError, match="group 0 has 127 members"):
        reference.act_order_perm(bad, k)
    bad = g.copy()
    bad[5] = 2
    with pytest.raises(ValueError, match="outside"):
        reference.act_order_perm(bad, k)


def test_zero_point_convention_swap_is_detected():
    # mate PR: two packed zero-point conventions share shape and value multiset;
    # reading one as the other must give a visibly wrong product.
    rng = np.random.default_rng(13)
    n, k = 6, 512
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    zeros = rng.integers(0, 16, size=(n, 4), dtype=np.uint8)
    scales = rng.uniform(0.001, 0.02, size=(n, 4)).astype(np.float16)
    x = rng.standard_normal((2, k))
    zp = formats.pack_zeros(zeros)
    swapped = formats.unpack_int4((zp >> 4) | ((zp & 0x0F) << 4), 4)   # high nibble first
    assert sorted(swapped.ravel()) != [] and not np.array_equal(swapped, zeros)
    y = reference.product(x, reference.weights_int4(codes, scales, formats.unpack_zeros(zp, 4)))
    y_bad = reference.product(x, reference.weights_int4(codes, scales, swapped))
    assert np.linalg.norm(y_bad - y) / np.linalg.norm(y) > 0.05


def test_symmetric_int4_is_zero_point_eight():
    rng = np.random.default_rng(14)
    codes = rng.integers(0, 16, size=(3, 256), dtype=np.uint8)
    scales = rng.uniform(0.001, 0.02, size=(3, 2)).astype(np.float16)
    np.testing.assert_array_equal(reference.weights_int4(codes, scales),
                                  reference.weights_int4(codes, scales, np.full((3, 2), 8, np.uint8)))


# ------------------------------------------------------------------ rounding
def test_round_to_matches_library_conversions():
    rng = np.random.default_rng(15)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 4, 20000),
                        np.array([0.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2.0 ** -20, 3 * 2.0 ** -25])])
    np.testing.assert_array_equal(reference.round_to(v, "f16"), v.astype(np.float16).astype(np.float64))
    v32 = v.astype(np.float32)   # torch's bf16 conversion rounds from fp32: compare on fp32 inputs
    got = reference.round_to(v32.astype(np.float64), "bf16")
    want = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(got, want)
    # ties to even
    assert reference.round_to(np.array([1 + 2 ** -8]), "bf16")[0] == 1.0
    assert reference.round_to(np.array([1 + 3 * 2 ** -8]), "bf16")[0] == 1 + 2 ** -6


def test_rounded_int4_weights_are_nearest_representable():
    rng = np.random.default_rng(16)
    codes = rng.integers(0, 16, size=(4, 256), dtype=np.uint8)
    scales = synth.f32_to_bf16_bits(rng.uniform(0.001, 0.02, size=(4, 2)).astype(np.float32))
    s = synth.bf16_bits_to_f32(scales).astype(np.float64)
    w = reference.weights_int4_rounded(codes, s, None, None, "bf16")
    exact = reference.weights_int4(codes, s)
    got = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).double().numpy()  # exact fits fp32
    np.testing.assert_array_equal(w, got)


# ------------------------------------------------------------------ quantiser
def test_quantizer_scale_rule_and_bounds():
    rng = np.random.default_rng(17)
    x = (rng.standard_normal((64, 512)) * rng.uniform(0.01, 100, size=(64, 1))).astype(np.float32)
    x[3] = 0.0
    q, s = quant.quantize_rows(x)
    assert q.dtype == np.int8 and s.dtype == np.float32
    # scale = fl32(amax * fl32(1/127)): product of two fp32 values is exact in fp64
    amax = np.abs(x).max(axis=1).astype(np.float64)
    want_s = (amax * float(np.float32(1) / np.float32(127))).astype(np.float32)
    np.testing.assert_array_equal(s, want_s)
    assert np.abs(q.astype(np.int32)).max() <= 127
    nz = s > 0
    assert np.all(np.abs(q[nz].astype(np.int32)).max(axis=1) == 127)
    assert np.all(q[3] == 0) and s[3] == 0
    # |x/s - q| <= 1/2 exactly for unclamped entries, ties to even (rational check on a sample)
    for r in range(0, 64, 7):
        for c in range(0, 512, 37):
            if s[r] == 0:
                continue
            ratio = Fraction(float(x[r, c])) / Fraction(float(s[r]))
            rq = Fraction(float(np.float32(x[r, c] / s[r])))   # the fp32 quotient the rule rounds
            assert abs(rq - ratio) <= abs(ratio) * Fraction(1, 2 ** 24)
            qi = int(q[r, c])
            if abs(qi) < 127:
                assert abs(rq - qi) <= Fraction(1, 2)
                if abs(rq - qi) == Fraction(1, 2):
                    assert qi % 2 == 0


def test_quantizer_ties_to_even_when_scale_is_one():
    # amax = 127 gives scale fl32(127 * fl32(1/127)) = 1.0 exactly, so q = rint(x).
    x = np.array([[127.0, 2.5, 3.5, -2.5, -0.5, 126.5, 0.5, 1.5]], np.float32)
    q, s = quant.quantize_rows(x)
    assert s[0] == 1.0
    assert list(q[0]) == [127, 2, 4, -2, 0, 126, 0, 2]


def test_group_quantizer_matches_rows_on_each_group():
    rng = np.random.default_rng(18)
    x = rng.standard_normal((3, 384)).astype(np.float32)
    q, s = quant.quantize_groups(x)
    for g in range(3):
        qg, sg = quant.quantize_rows(x[:, 128 * g:128 * (g + 1)])
        np.testing.assert_array_equal(q[:, 128 * g:128 * (g + 1)], qg)
        np.testing.assert_array_equal(s[:, g], sg)


def test_quantizer_reconstruction_error_bound():
    rng = np.random.default_rng(19)
    x = rng.standard_normal((8, 1024)).astype(np.float32)
    q, s = quant.quantize_rows(x)
    err = np.abs(quant.dequantize_rows(q, s) - x.astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 1e-6))


# ------------------------------------------------------------------ generators
def test_workload_generators_shapes_and_ranges():
    w = synth.ternary_tiny()
    assert (w.m, w.k, w.n) == (1, 512, 256) and w.codes.max() <= 2
    assert w.scales.dtype == np.float16 and 0.01 <= w.scales.min() and w.scales.max() <= 0.05
    w3 = synth.int4_zp_actorder("t", 2, 2, 512, 16)
    perm = reference.act_order_perm(w3.g_idx, 512)
    assert perm.shape == (512,)
    w4 = synth.int4_sym("t", 3, 4, 256, 8)
    assert w4.x.dtype == np.uint16 and w4.scales.dtype == np.uint16


# ------------------------------------------------------------------ 4-bit x int8
def _brute_int4_partials(q, codes, zeros, g_idx):
    m, k = q.shape
    n = codes.shape[0]
    out = np.zeros((m, n, k // 128), dtype=np.int64)
    for mi in range(m):
        for ni in range(n):
            for kk in range(k):
                g = kk // 128 if g_idx is None else int(g_idx[kk])
                z = 8 if zeros is None else int(zeros[ni, g])
                out[mi, ni, g] += int(q[mi, kk]) * (int(codes[ni, kk]) - z)
    return out


@pytest.mark.parametrize("m,k,n,zp,act", [(1, 128, 3, False, False), (3, 256, 4, True, False),
                                          (2, 256, 2, True, True), (2, 384, 3, False, True)])
def test_int4_partials_brute_force(m, k, n, zp, act):
    rng = np.random.default_rng(7000 + 10 * m + n + k)
    q = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    zeros = rng.integers(0, 16, size=(n, k // 128), dtype=np.uint8) if zp else None
    g_idx = _valid_gidx(rng, k) if act else None
    np.testing.assert_array_equal(reference.int4_partials(q, codes, zeros, g_idx),
                                  _brute_int4_partials(q, codes, zeros, g_idx))


def test_int4_partials_extremes():
    # |P| reaches 127 * 15 * 128 with q = -127, code 0, zero 15 (and the opposite sign).
    k = 256
    q = np.full((2, k), -127, np.int8)
    q[1] = 127
    codes = np.zeros((2, k), np.uint8)
    codes[1] = 15
    zeros = np.array([[15, 15], [0, 0]], np.uint8)
    p = reference.int4_partials(q, codes, zeros)
    assert p[0, 0, 0] == 127 * 15 * 128 and p[1, 0, 0] == -127 * 15 * 128
    assert p[0, 1, 1] == -127 * 15 * 128 and p[1, 1, 1] == 127 * 15 * 128


def test_int4_int8_product_matches_affine_split_exactly():
    # The page's form: per group scale * (q . code) plus the offset -scale * zero
    # times the group's activation sum, in exact rationals; power-of-two scales
    # keep the oracle's fp64 sums exact.
    rng = np.random.default_rng(7101)
    m, k, n = 2, 384, 3
    q = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    zeros = rng.integers(0, 16, size=(n, 3), dtype=np.uint8)
    scales = np.ldexp(1.0, rng.integers(-12, -4, size=(n, 3))).astype(np.float16)
    xs = np.ldexp(1.0, rng.integers(-9, -3, size=m)).astype(np.float32)
    g_idx = _valid_gidx(rng, k)
    _, y = reference.int4_int8_product(q, xs, codes, scales, zeros, g_idx)
    for mi in range(m):
        for ni in range(n):
            acc = Fraction(0)
            for g in range(3):
                cols = [kk for kk in range(k) if g_idx[kk] == g]
                dot = sum(int(q[mi, kk]) * int(codes[ni, kk]) for kk in cols)
                qsum = sum(int(q[mi, kk]) for kk in cols)
                s = Fraction(float(scales[ni, g]))
                acc += s * dot + (-s * int(zeros[ni, g])) * qsum
            assert Fraction(float(y[mi, ni])) == Fraction(float(xs[mi])) * acc


def test_int4_int8_product_equals_dequantised_matmul():
    # Against the (separately pinned) dequantised weights: y = xs * (q @ W^T).
    wl = synth.int4_zp_actorder("t", 31, 3, 512, 7)
    rng = np.random.default_rng(7102)
    q = rng.integers(-127, 128, size=(3, 512), dtype=np.int8)
    xs = rng.uniform(0.001, 0.05, size=3).astype(np.float32)
    _, y = reference.int4_int8_product(q, xs, wl.codes, wl.scales, wl.zeros, wl.g_idx)
    w = reference.weights_int4(wl.codes, wl.scales, wl.zeros, wl.g_idx)
    want = xs.astype(np.float64)[:, None] * reference.product(q.astype(np.float64), w)
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_int4_partials_act_order_sorted_form_and_negative_control():
    # The sorted form (activations and codes permuted, group j // 128) gives the
    # same partials; reading the zero points by k // 128 in the original order does not.
    rng = np.random.default_rng(7103)
    m, k, n = 2, 512, 5
    q = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    zeros = rng.integers(0, 16, size=(n, 4), dtype=np.uint8)
    g_idx = _valid_gidx(rng, k)
    perm = reference.act_order_perm(g_idx, k)
    p = reference.int4_partials(q, codes, zeros, g_idx)
    np.testing.assert_array_equal(reference.int4_partials(q[:, perm], codes[:, perm], zeros, None), p)
    assert not np.array_equal(reference.int4_partials(q, codes, zeros, None), p)


def test_quantizer_non_finite_blocks():
    # A row (or group) holding NaN or an infinity: scale NaN, codes 0; the
    # other rows keep the ordinary rule (row 2 worked by hand: amax 3).
    x = np.array([[1.0, np.nan, 2.0, 0.5],
                  [np.inf, 0.0, 0.0, 0.0],
                  [1.0, 2.0, -3.0, 0.0],
                  [-np.inf, 1.0, 1.0, 1.0]], np.float32)
    q, s = quant.quantize_rows(x)
    assert np.isnan(s[[0, 1, 3]]).all() and not np.isnan(s[2])
    assert (q[[0, 1, 3]] == 0).all()
    assert s[2] == np.float32(np.float32(3.0) * (np.float32(1.0) / np.float32(127.0)))
    assert q[2].tolist() == [42, 85, -127, 0]
    # group granularity: only the group with the NaN is affected
    xg = np.ones((1, 256), np.float32)
    xg[0, 200] = np.nan
    qg, sg = quant.quantize_groups(xg)
    assert not np.isnan(sg[0, 0]) and np.isnan(sg[0, 1])
    assert (qg[0, :128] == 127).all() and (qg[0, 128:] == 0).all()
    # the product of a flagged row is NaN everywhere, the other rows are finite
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 3, size=(3, 4 * 128)).astype(np.uint8)
    scales = rng.uniform(0.01, 0.05, size=(3, 4)).astype(np.float16)
    xr = rng.standard_normal((3, 512)).astype(np.float32)
    xr[1, 7] = np.inf
    qr, sr = quant.quantize_rows(xr)
    _, y = reference.ternary_int8_product(qr, sr, codes, scales)
    assert np.isnan(y[1]).all() and np.isfinite(y[[0, 2]]).all()


# ------------------------------------------------- W4A8 in TensorFold's affine form
def _nearest_f32(exact: Fraction) -> np.float32:
    """Brute force: the fp32 value nearest to an exact rational (ties to an even significand)."""
    c = np.float32(float(exact))
    cands = {float(c), float(np.nextafter(c, np.float32(np.inf))), float(np.nextafter(c, np.float32(-np.inf)))}
    best = min(cands, key=lambda v: (abs(Fraction(v) - exact), int(np.float32(v).view(np.uint32)) % 2))
    return np.float32(best)


def test_exact_sum_f32_against_fraction_rounding():
    rng = np.random.default_rng(7201)
    cases = [rng.standard_normal(128).astype(np.float32) for _ in range(40)]
    cases += [(rng.standard_normal(128) * np.exp2(rng.integers(-40, 40, 128))).astype(np.float32) for _ in range(40)]
    # fp64 sum lands exactly on an fp32 midpoint; the exact sum is on it, above it, below it
    cases += [np.array([1.0, 2.0 ** -24], np.float32),
              np.array([1.0, 2.0 ** -24, 2.0 ** -60], np.float32),
              np.array([1.0, 2.0 ** -24, -(2.0 ** -60)], np.float32),
              np.array([1.0 + 2.0 ** -23, 2.0 ** -24], np.float32),
              np.array([3.0e38, 3.0e38, -3.0e38], np.float32),
              np.zeros(128, np.float32), np.array([-0.0, 0.0], np.float32)]
    for v in cases:
        exact = sum((Fraction(float(t)) for t in v), Fraction(0))
        got = quant.exact_sum_f32(v)
        want = _nearest_f32(exact)
        assert got == want, (v[:4], got, want)
    assert quant.exact_sum_f32(np.array([1.0, 2.0 ** -24, 2.0 ** -60], np.float32)) == np.float32(1.0 + 2.0 ** -23)
    assert quant.exact_sum_f32(np.array([1.0, 2.0 ** -24, -(2.0 ** -60)], np.float32)) == np.float32(1.0)
    assert quant.exact_sum_f32(np.array([1.0 + 2.0 ** -23, 2.0 ** -24], np.float32)) == np.float32(1.0 + 2.0 ** -22)


def test_quantize_groups_sums_rule():
    rng = np.random.default_rng(7202)
    x = rng.standard_normal((4, 512)).astype(np.float32)
    x[1, 128:256] = 0.0                                        # an all-zero group
    x[2, 0] = 127.0                                            # amax 127 -> a = 1 exactly
    q, a, sums = quant.quantize_groups_sums(x)
    xb = x.reshape(4, 4, 128)
    # a = fl32(amax / 127), an IEEE division (not the reciprocal multiply of the row quantiser)
    np.testing.assert_array_equal(a, (np.abs(xb).max(-1) / np.float32(127)).astype(np.float32))
    assert a[2, 0] == 1.0 and np.array_equal(q[2, :128], np.rint(x[2, :128]).astype(np.int8))
    assert a[1, 1] == 0.0 and not q[1, 128:256].any() and sums[1, 1] == 0.0
    qb = q.reshape(4, 4, 128).astype(np.float64)
    nz = a > 0
    assert np.abs(q).max() <= 127 and np.all(np.abs(qb).max(-1)[nz] == 127)
    err = np.abs(qb * a[..., None] - xb)
    assert np.all(err <= a[..., None] / 2 * (1 + 2.0 ** -20))
    for i in range(4):
        for g in range(4):
            exact = sum((Fraction(float(t)) for t in xb[i, g]), Fraction(0))
            assert sums[i, g] == _nearest_f32(exact)
    # a value where the division and the reciprocal multiply round apart: the division wins
    for amax in rng.uniform(0.5, 8.0, 2000).astype(np.float32):
        div = np.float32(amax / np.float32(127.0))
        mul = np.float32(amax * quant.INV127)
        if div != mul:
            row = np.zeros((1, 128), np.float32)
            row[0, 5] = -amax
            _, aa, _ = quant.quantize_groups_sums(row)
            assert aa[0, 0] == div
            break
    else:
        pytest.fail("no amax separates the two scale rules")


def test_quantize_groups_sums_follows_the_weight_groups():
    rng = np.random.default_rng(7203)
    x = rng.standard_normal((3, 512)).astype(np.float32)
    g_idx = _valid_gidx(rng, 512)
    perm = reference.act_order_perm(g_idx, 512)
    q1, a1, s1 = quant.quantize_groups_sums(x, perm)
    q2, a2, s2 = quant.quantize_groups_sums(np.ascontiguousarray(x[:, perm]))
    np.testing.assert_array_equal(q1[:, perm], q2)
    np.testing.assert_array_equal(a1, a2)
    np.testing.assert_array_equal(s1, s2)
    # group g of the permuted form is the columns whose g_idx is g
    for g in range(4):
        cols = np.flatnonzero(g_idx == g)
        assert a1[0, g] == np.float32(np.abs(x[0, cols]).max() / np.float32(127))


def test_quantize_groups_sums_non_finite_group():
    x = np.ones((1, 256), np.float32)
    x[0, 200] = np.inf
    q, a, s = quant.quantize_groups_sums(x)
    assert a[0, 0] == np.float32(1.0 / 127.0) and s[0, 0] == 128.0
    assert np.isnan(a[0, 1]) and np.isnan(s[0, 1]) and not q[0, 128:].any()


@pytest.mark.parametrize("m,k,n,act", [(1, 128, 3, False), (3, 256, 4, True), (2, 384, 2, True)])
def test_int4_raw_partials_brute_force(m, k, n, act):
    rng = np.random.default_rng(7204 + m * 10 + n)
    q = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    g_idx = _valid_gidx(rng, k) if act else None
    d = reference.int4_raw_partials(q, codes, g_idx)
    for mi in range(m):
        for ni in range(n):
            for g in range(k // 128):
                cols = range(g * 128, g * 128 + 128) if g_idx is None else np.flatnonzero(g_idx == g)
                assert d[mi, ni, g] == sum(int(q[mi, c]) * int(codes[ni, c]) for c in cols)
    # extremes: |D| reaches 127 * 15 * 128
    qx = np.full((1, 128), -127, np.int8)
    cx = np.full((1, 128), 15, np.uint8)
    assert reference.int4_raw_partials(qx, cx)[0, 0, 0] == -127 * 15 * 128


def _fraction_affine(q, a, sums, codes, scales, zeros, g_idx):
    m, k = q.shape
    n = codes.shape[0]
    out = np.empty((m, n), object)
    for mi in range(m):
        for ni in range(n):
            acc = Fraction(0)
            for g in range(k // 128):
                cols = range(g * 128, g * 128 + 128) if g_idx is None else np.flatnonzero(g_idx == g)
                dot = sum(int(q[mi, c]) * int(codes[ni, c]) for c in cols)
                s = Fraction(float(scales[ni, g]))
                z = 8 if zeros is None else int(zeros[ni, g])
                acc += s * Fraction(float(a[mi, g])) * dot + (-z * s) * Fraction(float(sums[mi, g]))
            out[mi, ni] = acc
    return out


@pytest.mark.parametrize("zp,act", [(False, False), (True, False), (True, True)])
def test_w4a8_affine_product_fraction_brute_force(zp, act):
    """Distinct scales, zero points, activation scales and sums everywhere; dropping the
    offset term, flipping its sign, or taking it from the quantised sum a * sum(q) in
    place of the exact sum of x must fail."""
    rng = np.random.default_rng(7210 + 2 * zp + act)
    m, k, n = 3, 384, 4
    x = rng.standard_normal((m, k)).astype(np.float32)
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    zeros = rng.integers(0, 16, size=(n, 3), dtype=np.uint8) if zp else None
    scales = rng.uniform(0.001, 0.02, size=(n, 3)).astype(np.float16)
    g_idx = _valid_gidx(rng, k) if act else None
    perm = None if g_idx is None else reference.act_order_perm(g_idx, k)
    q, a, sums = quant.quantize_groups_sums(x, perm)
    exact = _fraction_affine(q, a, sums, codes, scales, zeros, g_idx)
    d, y = reference.w4a8_affine_product(q, a, sums, codes, scales, zeros, g_idx)
    np.testing.assert_array_equal(d, reference.int4_raw_partials(q, codes, g_idx))
    for i in range(m):
        for j in range(n):
            assert abs(Fraction(float(y[i, j])) - exact[i, j]) <= abs(exact[i, j]) * Fraction(1, 10 ** 12)

    def off(yy):
        return max(abs(Fraction(float(yy[i, j])) - exact[i, j]) / abs(exact[i, j]) for i in range(m) for j in range(n))
    qsum = np.zeros_like(sums)
    grp = np.arange(k) // 128 if g_idx is None else g_idx
    for g in range(3):
        qsum[:, g] = a[:, g] * q[:, grp == g].astype(np.float32).sum(1)
    for bad in (np.zeros_like(sums), -sums, qsum):
        _, yb = reference.w4a8_affine_product(q, a, bad, codes, scales, zeros, g_idx)
        assert off(yb) > Fraction(1, 10 ** 9)


def test_w4a8_affine_product_equals_dequantised_matmul_when_x_is_exact():
    """Activations built as x = 2^e * q with a +-127 entry in every group: the quantiser
    returns q, a = 2^e and the exact sum, so the affine form must equal the (separately
    pinned) dequantised matmul x @ W^T."""
    rng = np.random.default_rng(7220)
    m, k, n = 3, 512, 5
    wl = synth.int4_zp_actorder("t", 71, m, k, n)
    perm = reference.act_order_perm(wl.g_idx, k)
    qn = rng.integers(-127, 128, size=(m, k)).astype(np.float64)
    e = rng.integers(-10, -3, size=(m, 4))
    for g in range(4):
        cols = perm[128 * g:128 * (g + 1)]
        qn[:, cols[7]] = 127.0
    scale_col = np.empty((m, k))
    scale_col[:, perm] = np.repeat(np.exp2(e), 128, axis=1)
    x = (qn * scale_col).astype(np.float32)
    q, a, sums = quant.quantize_groups_sums(x, perm)
    np.testing.assert_array_equal(q, qn.astype(np.int8))
    np.testing.assert_array_equal(a, np.exp2(e).astype(np.float32))
    _, y = reference.w4a8_affine_product(q, a, sums, wl.codes, wl.scales, wl.zeros, wl.g_idx)
    want = reference.product(x, reference.weights_int4(wl.codes, wl.scales, wl.zeros, wl.g_idx))
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
