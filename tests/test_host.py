"""Host-side checks of the C ABI (no GPU): exports, sizes, prepare, validation.

Every validation error is detected on the host before any HIP call, so these
tests force each status from the CPU with placeholder (never dereferenced)
pointers.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import bit_packed_weight_amd as bpw
from oracle import formats, reference
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_header_symbol():
    text = open(os.path.join(ROOT, "include", "bpw.h")).read()
    declared = set(re.findall(r"\b(bpw_[a-z0-9_]+)\s*\(", text))
    assert {"bpw_prepare_packed", "bpw_gemv_packed", "bpw_gemm_packed", "bpw_partials"} <= declared
    lib = bpw.lib()
    for name in sorted(declared):
        assert hasattr(lib, name), name
    assert set(bpw.EXPORTS) == declared
    assert bpw.version() >= 100


def _golden(name):
    rows = []
    for line in open(os.path.join(ROOT, "tests", "golden", name)):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(line.split())
    return rows


def test_packed_sizes_match_logical_byte_formula():
    # "Kernel experiments", Test 19: bytes per call = n*k//4 + n*(k//128)*2, which
    # Test 25 writes as n*(k//128)*34.
    for name, n, k in _golden("pq2_shapes.txt"):
        n, k = int(n), int(k)
        s = bpw.packed_sizes(bpw.TERNARY2, n, k)
        assert s.codes + s.scales == n * k // 4 + n * (k // 128) * 2 == n * (k // 128) * 34
        assert s.zeros == 0 and s.perm == 0
    s = bpw.packed_sizes(bpw.INT4_ZP, 13824, 5120, bpw.F16, True)
    assert (s.codes, s.scales, s.zeros, s.perm) == (13824 * 2560, 13824 * 40 * 2, 13824 * 20, 5120 * 4)
    s = bpw.packed_sizes(bpw.INT4_ZP, 3, 384, bpw.F16)     # odd group count: ceil(G/2) zero bytes
    assert s.zeros == 3 * 2


@pytest.mark.parametrize("src", ["codes", "planes", "pq2"])
def test_prepare_ternary_bit_exact_against_oracle(src):
    w = synth.ternary_int8("t", 31, 1, 512, 37, 0.005, 0.05, "f16")
    codes = w.codes.copy()
    codes[0, :4] = 3                                # every code value, incl. 3
    plane = formats.pack_ternary(codes)
    if src == "codes":
        out = bpw.prepare_packed_host(bpw.TERNARY2, codes, w.scales)
    elif src == "planes":
        out = bpw.prepare_packed_host(bpw.TERNARY2, plane, w.scales, src_format=bpw.SRC_PLANES)
    else:
        raw = formats.join_pq2_blocks(plane, w.scales)
        out = bpw.prepare_packed_host(bpw.TERNARY2, raw, None, src_format=bpw.SRC_PQ2_BLOCKS)
    np.testing.assert_array_equal(out["codes"], plane)
    np.testing.assert_array_equal(out["scales"], w.scales.view(np.uint16))
    np.testing.assert_array_equal(formats.unpack_ternary(out["codes"], 512), codes)


@pytest.mark.parametrize("fmt", ["int4_zp", "int4_sym"])
@pytest.mark.parametrize("act_order", [False, True])
@pytest.mark.parametrize("src", ["codes", "planes"])
def test_prepare_int4_bit_exact_against_oracle(fmt, act_order, src):
    k = 640                                        # 5 groups: odd zero-point count
    w = synth.int4_zp_actorder("t", 41, 2, k, 9, act_order=act_order)
    zeros = w.zeros if fmt == "int4_zp" else None
    code = bpw.INT4_ZP if fmt == "int4_zp" else bpw.INT4_SYM
    if src == "codes":
        out = bpw.prepare_packed_host(code, w.codes, w.scales, zeros, w.g_idx)
    else:
        zp = None if zeros is None else formats.pack_zeros(zeros)
        out = bpw.prepare_packed_host(code, formats.pack_int4(w.codes), w.scales, zp, w.g_idx,
                                      src_format=bpw.SRC_PLANES)
    if act_order:
        perm = reference.act_order_perm(w.g_idx, k)
        np.testing.assert_array_equal(out["perm"], perm)
        sorted_codes = w.codes[:, perm]
    else:
        assert out["perm"] is None
        sorted_codes = w.codes
    np.testing.assert_array_equal(out["codes"], formats.pack_int4(sorted_codes))
    np.testing.assert_array_equal(out["scales"], w.scales.view(np.uint16))
    if zeros is not None:
        np.testing.assert_array_equal(out["zeros"], formats.pack_zeros(zeros))
    # the prepared planes reproduce the original product: x[:, perm] @ W_sorted^T == x @ W^T
    x = w.x.astype(np.float64)
    w_orig = reference.weights_int4(w.codes, w.scales, zeros, w.g_idx)
    w_prep = reference.weights_int4(formats.unpack_int4(out["codes"], k), w.scales,
                                    None if zeros is None else formats.unpack_zeros(out["zeros"], 5))
    xp = x[:, out["perm"]] if act_order else x
    np.testing.assert_allclose(reference.product(xp, w_prep), reference.product(x, w_orig), rtol=1e-12, atol=1e-12)


def _expect(status, fn, *args, match=None):
    with pytest.raises(bpw.BpwError) as e:
        fn(*args)
    assert e.value.status == status, str(e.value)
    if match:
        assert re.search(match, str(e.value)), str(e.value)


def test_prepare_refuses_bad_inputs_and_writes_nothing():
    w = synth.int4_zp_actorder("t", 5, 1, 256, 4)
    bad = w.g_idx.copy()
    bad[np.flatnonzero(bad == 0)[0]] = 1
    _expect(bpw.EGIDX, bpw.prepare_packed_host, bpw.INT4_ZP, w.codes, w.scales, w.zeros, bad,
            match="group 0 has 127 members")
    bad = w.g_idx.copy()
    bad[3] = 7
    _expect(bpw.EGIDX, bpw.prepare_packed_host, bpw.INT4_ZP, w.codes, w.scales, w.zeros, bad, match="outside")
    _expect(bpw.ESHAPE, bpw.prepare_packed_host, bpw.TERNARY2, np.zeros((2, 200), np.uint8),
            np.zeros((2, 1), np.float16))
    _expect(bpw.EUNSUPPORTED, bpw.prepare_packed_host, bpw.INT4_SYM, np.zeros((2, 34), np.uint8), None,
            None, None, bpw.SRC_PQ2_BLOCKS)
    _expect(bpw.EINVAL, bpw.prepare_packed_host, bpw.INT4_ZP, w.codes, w.scales, None)   # zeros missing
    # out-of-range code: the destination planes keep their previous contents
    codes = w.codes.copy()
    codes[1, 100] = 16
    lib = bpw.lib()
    dst = np.full(4 * 128, 0xAB, np.uint8)
    dsc = np.full(4 * 2 * 2, 0xAB, np.uint8)
    dz = np.full(4, 0xAB, np.uint8)
    st = lib.bpw_prepare_packed(bpw.INT4_ZP, bpw.SRC_CODES_U8, bpw.F16, 4, 256, 128,
                                codes.ctypes.data_as(ctypes.c_void_p), w.scales.ctypes.data_as(ctypes.c_void_p),
                                w.zeros.ctypes.data_as(ctypes.c_void_p), None,
                                dst.ctypes.data_as(ctypes.c_void_p), dsc.ctypes.data_as(ctypes.c_void_p),
                                dz.ctypes.data_as(ctypes.c_void_p), None)
    assert st == bpw.EINVAL and "exceeds 15" in bpw.last_error()
    assert np.all(dst == 0xAB) and np.all(dsc == 0xAB) and np.all(dz == 0xAB)


# --------------------------------------------------------------- product validation
def _weights(fmt=bpw.TERNARY2, n=64, k=256, scale_dtype=bpw.F16, zeros=False, perm=False, codes=4096):
    return bpw.BpwWeights(fmt, scale_dtype, 128, 0, n, k, codes, 8192, 12288 if zeros else None,
                          16384 if perm else None)


def _gemv(w, x=65536, x_dtype=bpw.I8, xs=1024, m=1, y=131072, y_dtype=bpw.F16, ws=None, ws_bytes=0):
    return bpw.lib().bpw_gemv_packed(ctypes.byref(w), x, x_dtype, xs, m, y, y_dtype, ws, ws_bytes, None)


def test_product_validation_statuses():
    assert _gemv(_weights(k=200)) == bpw.ESHAPE
    assert "multiple of 128" in bpw.last_error()
    assert _gemv(_weights(), m=0) == bpw.ESHAPE
    assert _gemv(_weights(), x=None) == bpw.EINVAL
    assert _gemv(_weights(), xs=None) == bpw.EINVAL                      # int8 needs row scales
    assert _gemv(_weights(), x_dtype=bpw.F16, xs=None, m=2) == bpw.EUNSUPPORTED    # fused quantiser: M = 1 only
    assert _gemv(_weights(), y_dtype=bpw.I32) == bpw.EUNSUPPORTED
    assert _gemv(_weights(codes=4100)) == bpw.EALIGN
    assert _gemv(_weights(), x=65540) == bpw.EALIGN
    w = _weights()
    w.group = 64
    assert _gemv(w) == bpw.EUNSUPPORTED
    w = _weights()
    w.reserved = 1
    assert _gemv(w) == bpw.EINVAL
    assert _gemv(_weights(scale_dtype=bpw.BF16)) == bpw.EUNSUPPORTED     # ternary: fp16 scales
    assert _gemv(_weights(perm=True)) == bpw.EUNSUPPORTED                # ternary act order
    # 4-bit
    assert _gemv(_weights(bpw.INT4_ZP), x_dtype=bpw.F16, xs=None) == bpw.EINVAL          # zero plane missing
    assert _gemv(_weights(bpw.INT4_SYM, zeros=True), x_dtype=bpw.F16, xs=None) == bpw.EINVAL
    assert _gemv(_weights(bpw.INT4_SYM), x_dtype=bpw.BF16, xs=None) == bpw.EUNSUPPORTED    # scale/act dtype
    assert _gemv(_weights(bpw.INT4_SYM), x_dtype=bpw.F16, xs=1024) == bpw.EINVAL
    assert _gemv(_weights(bpw.INT4_SYM), x_dtype=bpw.I8) == bpw.EUNSUPPORTED
    assert "bpw_gemm_packed only" in bpw.last_error()                  # 4-bit x int8: GEMM entry
    # act order needs a workspace
    wp = _weights(bpw.INT4_SYM, perm=True)
    assert _gemv(wp, x_dtype=bpw.F16, xs=None, m=4) == bpw.EINVAL
    assert "workspace" in bpw.last_error()
    assert _gemv(wp, x_dtype=bpw.F16, xs=None, m=4, ws=1 << 20, ws_bytes=16) == bpw.ESHAPE
    assert _gemv(wp, x_dtype=bpw.F16, xs=None, m=4, ws=(1 << 20) + 16, ws_bytes=1 << 20) == bpw.EALIGN


def test_fused_quantise_validation():
    # ternary weights with fp32 / fp16 / bf16 activations: the one-token complete
    # call (M = 1, K <= 16384, no x_scale, no workspace, decode entry only)
    lib = bpw.lib()
    need = ctypes.c_size_t(7)
    w = _weights(k=4096, n=300)
    for xd in (bpw.F32, bpw.F16, bpw.BF16):
        assert lib.bpw_workspace_size(ctypes.byref(w), 1, xd, bpw.PATH_GEMV, ctypes.byref(need)) == 0
        assert need.value == 0
        assert _gemv(w, x_dtype=xd) == bpw.EINVAL                             # x_scale given
        assert "quantises the activations itself" in bpw.last_error()
        assert _gemv(w, x_dtype=xd, xs=None, m=2) == bpw.EUNSUPPORTED
        assert "bpw_quantize_rows first" in bpw.last_error()
        assert _gemv(_weights(k=16512, n=300), x_dtype=xd, xs=None) == bpw.EUNSUPPORTED
        assert _gemv(w, x_dtype=xd, xs=None, x=65544) == bpw.EALIGN
        st = lib.bpw_gemm_packed(ctypes.byref(w), 65536, xd, None, 1, 131072, bpw.F16, None, 0, None)
        assert st == bpw.EUNSUPPORTED and "bpw_gemv_packed only" in bpw.last_error()
    assert _gemv(w, x_dtype=bpw.I32, xs=None) == bpw.EUNSUPPORTED


def test_group_scale_validation():
    lib = bpw.lib()
    w = _weights(k=4096, n=300)
    # the prefill entry takes per-group scales too, on its plane-ordered copy of q (M * K bytes)
    st = lib.bpw_gemm_packed(ctypes.byref(w), 65536, bpw.I8G, 1024, 4, 131072, bpw.F16, None, 0, None)
    assert st == bpw.EINVAL and "16384-byte device workspace" in bpw.last_error()
    need = ctypes.c_size_t(7)
    assert lib.bpw_workspace_size(ctypes.byref(w), 4, bpw.I8G, bpw.PATH_GEMM, ctypes.byref(need)) == 0
    assert need.value == 4 * 4096
    # beyond 32 rows the decode entry routes to the same prefill kernel
    assert _gemv(_weights(k=256), x_dtype=bpw.I8G, m=33) == bpw.EINVAL
    assert "workspace" in bpw.last_error()
    assert _gemv(_weights(k=256), x_dtype=bpw.I8G, xs=None) == bpw.EINVAL
    assert _gemv(_weights(k=256), x_dtype=bpw.I8G, xs=1026) == bpw.EALIGN
    assert _gemv(_weights(bpw.INT4_SYM), x_dtype=bpw.I8G) == bpw.EUNSUPPORTED
    need = ctypes.c_size_t(7)
    assert lib.bpw_workspace_size(ctypes.byref(_weights(k=8192, n=100)), 32, bpw.I8G, bpw.PATH_GEMV,
                                  ctypes.byref(need)) == 0
    assert need.value == 0
    quant = lib.bpw_quantize_groups
    assert quant(65536, bpw.F32, 2, 200, 131072, 1024, None) == bpw.ESHAPE      # K % 128
    assert quant(65536, bpw.I8, 2, 256, 131072, 1024, None) == bpw.EUNSUPPORTED
    assert quant(65536, bpw.F32, 2, 256, 131080, 1024, None) == bpw.EALIGN      # q 16-byte aligned
    assert quant(None, bpw.F32, 2, 256, 131072, 1024, None) == bpw.EINVAL


def test_affine_w4a8_validation():
    lib = bpw.lib()
    w4 = _weights(bpw.INT4_SYM, k=512, n=300)
    # the affine form (BPW_I8GS) is 4-bit x int8 on the prefill entry only
    assert _gemv(w4, x_dtype=bpw.I8GS) == bpw.EUNSUPPORTED and "bpw_gemm_packed" in bpw.last_error()
    assert _gemv(_weights(k=512), x_dtype=bpw.I8GS) == bpw.EUNSUPPORTED               # ternary: not this form
    st = lib.bpw_gemm_packed(ctypes.byref(w4), 65536, bpw.I8GS, 1024, 4, 131072, bpw.F16, None, 0, None)
    assert st == bpw.EINVAL and "2048-byte device workspace" in bpw.last_error()
    st = lib.bpw_gemm_packed(ctypes.byref(w4), 65536, bpw.I8GS, 1028, 4, 131072, bpw.F16, None, 0, None)
    assert st == bpw.EALIGN                                                             # (a, sum) pairs: 8 bytes
    st = lib.bpw_gemm_packed(ctypes.byref(w4), 65536, bpw.I8GS, None, 4, 131072, bpw.F16, None, 0, None)
    assert st == bpw.EINVAL
    need = ctypes.c_size_t()
    assert lib.bpw_workspace_size(ctypes.byref(w4), 4, bpw.I8GS, bpw.PATH_GEMM, ctypes.byref(need)) == 0
    assert need.value == 2048
    quant = lib.bpw_quantize_groups_sums
    assert quant(65536, bpw.F32, 2, 200, None, 131072, 1024, None) == bpw.ESHAPE          # K % 128
    assert quant(65536, bpw.I8, 2, 256, None, 131072, 1024, None) == bpw.EUNSUPPORTED
    assert quant(65536, bpw.F32, 2, 256, None, 131080, 1024, None) == bpw.EALIGN          # q 16-byte aligned
    assert quant(65536, bpw.F32, 2, 256, None, 131072, 1028, None) == bpw.EALIGN          # pairs 8-byte aligned
    assert quant(65536, bpw.F32, 2, 256, 4098, 131072, 1024, None) == bpw.EALIGN          # perm 4-byte aligned
    assert quant(None, bpw.F32, 2, 256, None, 131072, 1024, None) == bpw.EINVAL
    # raw-code partials: a known path, 4-bit or ternary, with the GEMM workspace
    st = lib.bpw_partials(ctypes.byref(w4), 65536, 4, bpw.PATH_GEMM_RAW, 0, 4, 0, 300, 131072, None, 0, None)
    assert st == bpw.EINVAL and "workspace" in bpw.last_error()
    st = lib.bpw_partials(ctypes.byref(w4), 65536, 4, 3, 0, 4, 0, 300, 131072, None, 0, None)
    assert st == bpw.EINVAL and "unknown path" in bpw.last_error()


def test_workspace_sizes():
    need = ctypes.c_size_t()
    lib = bpw.lib()
    w = _weights(k=4096, n=14336)
    assert lib.bpw_workspace_size(ctypes.byref(w), 1, bpw.I8, bpw.PATH_GEMV, ctypes.byref(need)) == 0
    assert need.value == 0
    assert lib.bpw_workspace_size(ctypes.byref(w), 2048, bpw.I8, bpw.PATH_GEMM, ctypes.byref(need)) == 0
    assert need.value == 2048 * 4096
    # ternary decode beyond 32 groups, 2 <= M <= 32: fp32 split-K slices of 32 groups
    wl = _weights(k=14336, n=4096)
    assert lib.bpw_workspace_size(ctypes.byref(wl), 16, bpw.I8, bpw.PATH_GEMV, ctypes.byref(need)) == 0
    assert need.value == 4 * 16 * 4096 * 4
    assert lib.bpw_workspace_size(ctypes.byref(wl), 1, bpw.I8, bpw.PATH_GEMV, ctypes.byref(need)) == 0
    assert need.value == 0                                             # M = 1: the row kernel
    assert lib.bpw_workspace_size(ctypes.byref(wl), 16, bpw.I8G, bpw.PATH_GEMV, ctypes.byref(need)) == 0
    assert need.value == 0                                             # group scales: long-K kernel
    wp = _weights(bpw.INT4_ZP, k=5120, zeros=True, perm=True)
    assert lib.bpw_workspace_size(ctypes.byref(wp), 8, bpw.F16, bpw.PATH_GEMV, ctypes.byref(need)) == 0
    assert need.value == 8 * 5120 * 2
    # 4-bit decode beyond 48 groups, 2 <= M <= 16: the gathered rows (act order), then
    # fp32 slices; 108 groups make 7 slices of 4 four-group waves (6 x 16, 12)
    wd = _weights(bpw.INT4_ZP, k=13824, n=5120, zeros=True, perm=True)
    assert lib.bpw_workspace_size(ctypes.byref(wd), 8, bpw.F16, bpw.PATH_GEMV, ctypes.byref(need)) == 0
    assert need.value == 8 * 13824 * 2 + 7 * 8 * 5120 * 4
    wd = _weights(bpw.INT4_SYM, k=6272, n=100)                       # 49 groups: 4 slices of 13 -> 16, 16, 16, 1
    assert lib.bpw_workspace_size(ctypes.byref(wd), 3, bpw.BF16, bpw.PATH_GEMV, ctypes.byref(need)) == 0
    assert need.value == 4 * 3 * 100 * 4 + 256 - (4 * 3 * 100 * 4) % 256
    assert lib.bpw_workspace_size(ctypes.byref(wd), 1, bpw.BF16, bpw.PATH_GEMV, ctypes.byref(need)) == 0
    assert need.value == 0                                             # M = 1: the row kernel
    assert lib.bpw_workspace_size(ctypes.byref(wd), 2, bpw.BF16, bpw.PATH_GEMM, ctypes.byref(need)) == 0
    assert need.value == 0


def test_partials_and_probe_validation():
    lib = bpw.lib()
    w = _weights(n=64, k=256)
    assert lib.bpw_partials(ctypes.byref(w), 65536, 4, bpw.PATH_GEMV, 0, 5, 0, 8, 4096, None, 0, None) == bpw.ESHAPE
    assert lib.bpw_partials(ctypes.byref(w), 65536, 4, bpw.PATH_GEMV, 0, 4, 8, 8, 4096, None, 0, None) == bpw.ESHAPE
    assert lib.bpw_partials(ctypes.byref(w), 65536, 40, bpw.PATH_GEMV, 0, 4, 0, 8, 4096, None, 0, None) == bpw.ESHAPE
    assert lib.bpw_partials(ctypes.byref(w), 65536, 4, 7, 0, 4, 0, 8, 4096, None, 0, None) == bpw.EINVAL
    assert lib.bpw_partials(ctypes.byref(w), 65536, 4, bpw.PATH_GEMM, 0, 4, 0, 8, 4096, None, 0, None) == bpw.EINVAL
    w4 = _weights(bpw.INT4_SYM)
    assert lib.bpw_partials(ctypes.byref(w4), 65536, 4, bpw.PATH_GEMV, 0, 4, 0, 8, 4096, None, 0, None) == bpw.EUNSUPPORTED
    assert lib.bpw_probe(9, 4096, 8192, 1024, None) == bpw.EINVAL
    assert lib.bpw_probe(bpw.PROBE_READ, 4096, 8192, 1000, None) == bpw.ESHAPE
    assert lib.bpw_quantize_rows(4096, bpw.I8, 1, 16, 8192, 12288, None) == bpw.EUNSUPPORTED
    assert lib.bpw_quantize_rows(None, bpw.F32, 1, 16, 8192, 12288, None) == bpw.EINVAL


def test_w4a8_validation_and_workspace():
    lib = bpw.lib()

    def gemm(w, xs=1024, ws=None, ws_bytes=0, m=4, x_dtype=bpw.I8):
        return lib.bpw_gemm_packed(ctypes.byref(w), 65536, x_dtype, xs, m, 131072, bpw.F16, ws, ws_bytes, None)

    for w in (_weights(bpw.INT4_SYM), _weights(bpw.INT4_SYM, scale_dtype=bpw.BF16),
              _weights(bpw.INT4_ZP, zeros=True, perm=True)):
        assert gemm(w, xs=None) == bpw.EINVAL                       # int8 needs row scales
        assert gemm(w, xs=1026) == bpw.EALIGN
        assert gemm(w) == bpw.EINVAL and "workspace" in bpw.last_error()   # nibble-ordered copy of q
        assert gemm(w, ws=1 << 20, ws_bytes=4 * 256 - 1) == bpw.ESHAPE
        assert gemm(w, x_dtype=bpw.I8G) == bpw.EUNSUPPORTED
        need = ctypes.c_size_t()
        assert lib.bpw_workspace_size(ctypes.byref(w), 2048, bpw.I8, bpw.PATH_GEMM, ctypes.byref(need)) == 0
        assert need.value == 2048 * 256
    # partials of 4-bit weights: GEMM core only, with the same workspace
    w4 = _weights(bpw.INT4_ZP, zeros=True)
    assert lib.bpw_partials(ctypes.byref(w4), 65536, 4, bpw.PATH_GEMM, 0, 4, 0, 8, 4096, None, 0, None) == bpw.EINVAL
    assert "workspace" in bpw.last_error()


def test_traffic_profile_matches_gemv_sources():
    # bench.py reports the decode GEMV's measured HBM traffic only while the
    # committed counter summary was taken on the current GEMV sources; a change
    # to them must come with new counter passes.
    import bench
    traffic = bench.measured_traffic()
    assert traffic is not None, "GEMV sources changed since the traffic counters were taken"
    # every weight byte once, plus the activation row, the output and line granularity
    assert 15597568 <= traffic <= 1.01 * 15597568


def test_last_error_is_per_thread():
    # Each thread sees the message of its own last failure, however the calls
    # of several threads interleave.
    import threading
    lib = bpw.lib()
    errors = []

    def worker(kind):
        for _ in range(300):
            if kind == 0:
                st = _gemv(_weights(k=200))
                want = "multiple of 128"
            else:
                st = _gemv(_weights(), x=None)
                want = "x / y is NULL"
            msg = bpw.last_error()
            if want not in msg:
                errors.append((kind, st, msg))
    threads = [threading.Thread(target=worker, args=(i % 2,)) for i in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]
