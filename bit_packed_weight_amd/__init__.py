"""Python binding of libbpw.so, the bit-packed weight library for MI355X (gfx950).

The names mirror the C ABI in ``include/bpw.h``; this module only marshals
arguments (torch tensors -> device pointers, the current HIP stream, output and
workspace allocation through PyTorch). Every step of the computation runs in
the HIP kernels of the library. There is no CPU fallback: if the library is not
built, every call raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbpw.so")

# status codes
OK, EINVAL, ESHAPE, EALIGN, EGIDX, EUNSUPPORTED, EHIP = range(7)
# weight formats
TERNARY2, INT4_SYM, INT4_ZP = 1, 2, 3
# element types (I8G: int8 activations with one scale per (row, 128-group);
# I8GS: int8 with (scale, exact sum) per (row, weight group))
F32, F16, BF16, I8, I32, I8G, I8GS = 0, 1, 2, 3, 4, 5, 6
# prepare sources
SRC_PQ2_BLOCKS, SRC_PLANES, SRC_CODES_U8 = 1, 2, 3
# partial-sum cores / workspace entries (PATH_GEMM_RAW: partials only, the core of
# the per-(row, group) GEMM: ternary code - 1, 4-bit raw codes)
PATH_GEMV, PATH_GEMM, PATH_GEMM_RAW = 0, 1, 2
# probes
PROBE_READ, PROBE_COPY = 0, 1
# fixed device scratch of bpw_gemv_packed_scratch (bytes, per GPU)
SCRATCH_BYTES = 16 << 20

FORMAT_NAMES = {"ternary": TERNARY2, "int4_sym": INT4_SYM, "int4_zp": INT4_ZP}
_STATUS_NAMES = {EINVAL: "EINVAL", ESHAPE: "ESHAPE", EALIGN: "EALIGN", EGIDX: "EGIDX",
                 EUNSUPPORTED: "EUNSUPPORTED", EHIP: "EHIP"}


class BpwError(RuntimeError):
    """A nonzero status from the library; ``status`` holds the code."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class BpwWeights(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("scale_dtype", ctypes.c_int32),
                ("group", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zeros", ctypes.c_void_p), ("perm", ctypes.c_void_p)]


class BpwSizes(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_size_t), ("scales", ctypes.c_size_t),
                ("zeros", ctypes.c_size_t), ("perm", ctypes.c_size_t)]


EXPORTS = {
    "bpw_version": (ctypes.c_int, []),
    "bpw_last_error": (ctypes.c_char_p, []),
    "bpw_packed_sizes": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int, ctypes.c_int, ctypes.POINTER(BpwSizes)]),
    "bpw_prepare_packed": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "bpw_quantize_rows": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "bpw_quantize_groups": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "bpw_quantize_groups_sums": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "bpw_workspace_size": (ctypes.c_int, [ctypes.POINTER(BpwWeights), ctypes.c_int64, ctypes.c_int,
                                          ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]),
    "bpw_gemv_packed": (ctypes.c_int, [ctypes.POINTER(BpwWeights), ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "bpw_gemm_packed": (ctypes.c_int, [ctypes.POINTER(BpwWeights), ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "bpw_partials": (ctypes.c_int, [ctypes.POINTER(BpwWeights), ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                    ctypes.c_void_p]),
    "bpw_gemv_packed_scratch": (ctypes.c_int, [ctypes.POINTER(BpwWeights), ctypes.c_void_p, ctypes.c_int,
                                               ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                               ctypes.c_void_p]),
    "bpw_probe": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                 ctypes.c_void_p]),
    "bpw_probe_blocks": (ctypes.c_int64, [ctypes.c_size_t]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libbpw.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m bit_packed_weight_amd._build` "
                               "(or __graft_entry__.build()); there is no fallback path")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def last_error() -> str:
    return lib().bpw_last_error().decode()


def _check(status: int) -> None:
    if status != OK:
        raise BpwError(status, last_error())


def version() -> int:
    return lib().bpw_version()


# ---------------------------------------------------------------- torch glue
def _torch():
    import torch  # noqa: PLC0415 (torch is only needed for device calls)
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    table = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16, torch.int8: I8,
             torch.int32: I32}
    if t not in table:
        raise ValueError(f"unsupported dtype {t}")
    return table[t]


def torch_dtype(code: int):
    torch = _torch()
    return {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16, I8: torch.int8,
            I32: torch.int32}[code]


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device=None) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _check_tensor(name: str, t, shape: tuple, dtypes: tuple, device=None) -> None:
    """Refuse, before any library call, a tensor whose shape, dtype, layout or
    device the kernels would not read within bounds: the C ABI receives bare
    pointers and cannot check sizes itself."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _check_gpu(name: str, t) -> None:
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (it is on {t.device})")


@dataclasses.dataclass
class PackedWeights:
    """Prepared planes on the device plus their metadata (see ``bpw_weights``)."""

    fmt: int
    scale_dtype: int
    n: int
    k: int
    codes: object
    scales: object
    zeros: object = None
    perm: object = None

    def struct(self) -> BpwWeights:
        return BpwWeights(self.fmt, self.scale_dtype, 128, 0, self.n, self.k, _ptr(self.codes),
                          _ptr(self.scales), _ptr(self.zeros), _ptr(self.perm))

    def validate(self, device) -> None:
        """Check every plane against n, k and the format (shapes, dtypes, device)."""
        torch = _torch()
        if self.k < 128 or self.k % 128:
            raise ValueError(f"K={self.k} must be a positive multiple of 128")
        g = self.k // 128
        cb = self.k // 4 if self.fmt == TERNARY2 else self.k // 2
        sd = {F16: torch.float16, BF16: torch.bfloat16}.get(self.scale_dtype)
        if sd is None:
            raise ValueError(f"scale dtype code {self.scale_dtype} is neither F16 nor BF16")
        _check_tensor("codes", self.codes, (self.n, cb), (torch.uint8,), device)
        _check_tensor("scales", self.scales, (self.n, g), (sd,), device)
        if self.zeros is not None:
            _check_tensor("zeros", self.zeros, (self.n, (g + 1) // 2), (torch.uint8,), device)
        if self.perm is not None:
            _check_tensor("perm", self.perm, (self.k,), (torch.int32,), device)

    @property
    def logical_bytes(self) -> int:
        """Weight bytes one product reads: codes + scales (+ zero points)."""
        total = self.codes.numel() + self.scales.numel() * self.scales.element_size()
        if self.zeros is not None:
            total += self.zeros.numel()
        return total


def packed_sizes(fmt: int, n: int, k: int, scale_dtype: int = F16, has_perm: bool = False) -> BpwSizes:
    out = BpwSizes()
    _check(lib().bpw_packed_sizes(fmt, scale_dtype, n, k, 128, int(has_perm), ctypes.byref(out)))
    return out


def _np_ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def prepare_packed_host(fmt: int, codes: np.ndarray, scales: Optional[np.ndarray] = None,
                        zeros: Optional[np.ndarray] = None, g_idx: Optional[np.ndarray] = None,
                        src_format: int = SRC_CODES_U8, scale_dtype: int = F16,
                        n: Optional[int] = None, k: Optional[int] = None) -> dict:
    """Run ``bpw_prepare_packed`` into host numpy planes (no GPU involved)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    if n is None or k is None:
        n = codes.shape[0]
        if src_format == SRC_CODES_U8:
            k = codes.shape[1]
        elif src_format == SRC_PQ2_BLOCKS:
            k = codes.shape[1] // 34 * 128
        else:
            k = codes.shape[1] * (4 if fmt == TERNARY2 else 2)
    sizes = packed_sizes(fmt, n, k, scale_dtype, g_idx is not None)
    g = k // 128
    out_codes = np.empty(sizes.codes, np.uint8)
    out_scales = np.empty(sizes.scales, np.uint8)
    out_zeros = np.empty(sizes.zeros, np.uint8) if sizes.zeros else None
    out_perm = np.empty(k, np.int32) if g_idx is not None else None
    if scales is not None:
        scales = np.ascontiguousarray(scales)
        if scales.dtype.itemsize != 2:
            raise ValueError("scales must be 16-bit (fp16 values or bf16 bit patterns)")
    if zeros is not None:
        zeros = np.ascontiguousarray(zeros, dtype=np.uint8)
    if g_idx is not None:
        g_idx = np.ascontiguousarray(g_idx, dtype=np.int32)
    _check(lib().bpw_prepare_packed(fmt, src_format, scale_dtype, n, k, 128, _np_ptr(codes),
                                    _np_ptr(scales), _np_ptr(zeros), _np_ptr(g_idx),
                                    _np_ptr(out_codes), _np_ptr(out_scales), _np_ptr(out_zeros),
                                    _np_ptr(out_perm)))
    cb = k // 4 if fmt == TERNARY2 else k // 2
    return {"fmt": fmt, "scale_dtype": scale_dtype, "n": n, "k": k,
            "codes": out_codes.reshape(n, cb), "scales": out_scales.view(np.uint16).reshape(n, g),
            "zeros": None if out_zeros is None else out_zeros.reshape(n, (g + 1) // 2),
            "perm": out_perm}


def upload(planes: dict, device="cuda") -> PackedWeights:
    """Copy host planes (from ``prepare_packed_host``) into device tensors."""
    torch = _torch()
    sd = torch.float16 if planes["scale_dtype"] == F16 else torch.bfloat16

    def dev(a, dt=None):
        if a is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(a)).to(device)
        return t.view(dt) if dt is not None else t

    return PackedWeights(planes["fmt"], planes["scale_dtype"], planes["n"], planes["k"],
                         dev(planes["codes"]), dev(planes["scales"].view(np.int16), sd),
                         dev(planes["zeros"]), dev(planes["perm"]))


def prepare_packed(fmt: int, codes: np.ndarray, scales=None, zeros=None, g_idx=None,
                   src_format: int = SRC_CODES_U8, scale_dtype: int = F16, device="cuda") -> PackedWeights:
    """``bpw_prepare_packed`` on the host, then upload the planes to ``device``."""
    return upload(prepare_packed_host(fmt, codes, scales, zeros, g_idx, src_format, scale_dtype), device)


def quantize_rows(x, q=None, x_scale=None):
    """int8 row quantiser on the GPU: returns (q [M,K] int8, x_scale [M] fp32)."""
    torch = _torch()
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [M, K] tensor")
    m, k = x.shape
    _check_tensor("x", x, (m, k), (torch.float32, torch.float16, torch.bfloat16))
    q = torch.empty((m, k), dtype=torch.int8, device=x.device) if q is None else q
    x_scale = torch.empty(m, dtype=torch.float32, device=x.device) if x_scale is None else x_scale
    _check_tensor("q", q, (m, k), (torch.int8,), x.device)
    _check_tensor("x_scale", x_scale, (m,), (torch.float32,), x.device)
    _check_gpu("x", x)
    _check(lib().bpw_quantize_rows(_ptr(x), dtype_code(x.dtype), m, k, _ptr(q), _ptr(x_scale),
                                   _stream(x.device)))
    return q, x_scale


def quantize_groups(x, q=None, x_scale=None):
    """int8 group quantiser on the GPU: returns (q [M,K] int8, x_scale [M,K/128] fp32)."""
    torch = _torch()
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [M, K] tensor")
    m, k = x.shape
    if k % 128:
        raise ValueError(f"K={k} must be a multiple of 128 for per-group scales")
    _check_tensor("x", x, (m, k), (torch.float32, torch.float16, torch.bfloat16))
    q = torch.empty((m, k), dtype=torch.int8, device=x.device) if q is None else q
    if x_scale is None:
        x_scale = torch.empty((m, k // 128), dtype=torch.float32, device=x.device)
    _check_tensor("q", q, (m, k), (torch.int8,), x.device)
    _check_tensor("x_scale", x_scale, (m, k // 128), (torch.float32,), x.device)
    _check_gpu("x", x)
    _check(lib().bpw_quantize_groups(_ptr(x), dtype_code(x.dtype), m, k, _ptr(q), _ptr(x_scale),
                                     _stream(x.device)))
    return q, x_scale


def quantize_groups_sums(x, perm=None, q=None, x_scale_sum=None):
    """Group quantiser with exact group sums (bpw_quantize_groups_sums): returns
    (q [M,K] int8, x_scale_sum [M,K/128,2] fp32 of (a, sum) pairs). ``perm`` is the
    prepared weight's act-order permutation (int32 [K] on the device) or None."""
    torch = _torch()
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [M, K] tensor")
    m, k = x.shape
    if k % 128:
        raise ValueError(f"K={k} must be a multiple of 128 for per-group scales")
    _check_tensor("x", x, (m, k), (torch.float32, torch.float16, torch.bfloat16))
    if perm is not None:
        _check_tensor("perm", perm, (k,), (torch.int32,), x.device)
    q = torch.empty((m, k), dtype=torch.int8, device=x.device) if q is None else q
    if x_scale_sum is None:
        x_scale_sum = torch.empty((m, k // 128, 2), dtype=torch.float32, device=x.device)
    _check_tensor("q", q, (m, k), (torch.int8,), x.device)
    _check_tensor("x_scale_sum", x_scale_sum, (m, k // 128, 2), (torch.float32,), x.device)
    _check_gpu("x", x)
    _check(lib().bpw_quantize_groups_sums(_ptr(x), dtype_code(x.dtype), m, k, _ptr(perm), _ptr(q),
                                          _ptr(x_scale_sum), _stream(x.device)))
    return q, x_scale_sum


def workspace_size(w: PackedWeights, m: int, x_dtype: int, entry: int) -> int:
    out = ctypes.c_size_t()
    st = w.struct()
    _check(lib().bpw_workspace_size(ctypes.byref(st), m, x_dtype, entry, ctypes.byref(out)))
    return out.value


def _workspace(w, m, x_dtype, entry, device, workspace):
    torch = _torch()
    need = workspace_size(w, m, x_dtype, entry)
    if need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if workspace.dim() != 1:
        raise ValueError("workspace must be a 1-D uint8 tensor")
    _check_tensor("workspace", workspace, (workspace.numel(),), (torch.uint8,), device)
    if workspace.numel() < need:
        raise ValueError(f"workspace has {workspace.numel()} bytes, this call needs {need}")
    return workspace, workspace.numel()


def _product(entry: int, w: PackedWeights, x, x_scale=None, out_dtype=None, out=None, workspace=None,
             scratch=False):
    torch = _torch()
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [M, K] tensor")
    m = x.shape[0]
    xd = dtype_code(x.dtype)
    if xd not in (F16, BF16, I8) and not (xd == F32 and w.fmt == TERNARY2):
        raise ValueError(f"activations of dtype {x.dtype} are not supported (fp16, bf16 or int8; fp32 for "
                         "ternary weights)")
    if xd == I8 and x_scale is not None and x_scale.dim() == 2:
        xd = I8G                                   # one scale per (row, 128-group)
    elif xd == I8 and x_scale is not None and x_scale.dim() == 3:
        xd = I8GS                                  # (scale, exact sum) per (row, weight group)
    _check_tensor("x", x, (m, w.k), (x.dtype,))
    w.validate(x.device)
    if xd == I8:
        if x_scale is None:
            raise ValueError("int8 activations need x_scale [M]")
        _check_tensor("x_scale", x_scale, (m,), (torch.float32,), x.device)
    elif xd == I8G:
        _check_tensor("x_scale", x_scale, (m, w.k // 128), (torch.float32,), x.device)
    elif xd == I8GS:
        _check_tensor("x_scale", x_scale, (m, w.k // 128, 2), (torch.float32,), x.device)
    elif x_scale is not None:
        raise ValueError("x_scale must be None for fp32/fp16/bf16 activations")
    if out is None:
        ternary_out = xd in (I8, I8G, I8GS) or w.fmt == TERNARY2
        out_dtype = out_dtype if out_dtype is not None else (torch.float16 if ternary_out else x.dtype)
        out = torch.empty((m, w.n), dtype=out_dtype, device=x.device)
    _check_tensor("out", out, (m, w.n), (torch.float32, torch.float16, torch.bfloat16), x.device)
    if scratch:
        # the library's own fixed scratch: nothing is allocated here or in the library
        _check_gpu("x", x)
        st = w.struct()
        _check(lib().bpw_gemv_packed_scratch(ctypes.byref(st), _ptr(x), xd, _ptr(x_scale), m, _ptr(out),
                                             dtype_code(out.dtype), _stream(x.device)))
        return out
    ws, ws_bytes = _workspace(w, m, xd, entry, x.device, workspace)
    _check_gpu("x", x)
    st = w.struct()
    fn = lib().bpw_gemv_packed if entry == PATH_GEMV else lib().bpw_gemm_packed
    _check(fn(ctypes.byref(st), _ptr(x), xd, _ptr(x_scale), m, _ptr(out), dtype_code(out.dtype),
              _ptr(ws), ws_bytes, _stream(x.device)))
    return out


def gemv_packed(w: PackedWeights, x, x_scale=None, out_dtype=None, out=None, workspace=None):
    """y = x @ W^T, decode-shaped (bpw_gemv_packed)."""
    return _product(PATH_GEMV, w, x, x_scale, out_dtype, out, workspace)


def gemv_packed_scratch(w: PackedWeights, x, x_scale=None, out_dtype=None, out=None):
    """y = x @ W^T through bpw_gemv_packed_scratch: the decode product with its workspace in
    the library's fixed per-GPU scratch (no workspace argument, nothing allocated when
    ``out`` is given). Calls that overlap on one GPU race."""
    return _product(PATH_GEMV, w, x, x_scale, out_dtype, out, None, scratch=True)


def gemm_packed(w: PackedWeights, x, x_scale=None, out_dtype=None, out=None, workspace=None):
    """y = x @ W^T, prefill-shaped (bpw_gemm_packed)."""
    return _product(PATH_GEMM, w, x, x_scale, out_dtype, out, workspace)


def partials(w: PackedWeights, q, path: int, m0: int, m1: int, n0: int, n1: int, workspace=None):
    """Exact int32 group partials of a window (bpw_partials)."""
    torch = _torch()
    if q.dim() != 2:
        raise ValueError("q must be an [M, K] int8 tensor")
    m = q.shape[0]
    _check_tensor("q", q, (m, w.k), (torch.int8,))
    w.validate(q.device)
    if not (0 <= m0 < m1 <= m and 0 <= n0 < n1 <= w.n):
        raise ValueError(f"window [{m0},{m1}) x [{n0},{n1}) outside M={m}, N={w.n}")
    _check_gpu("q", q)
    g = w.k // 128
    out = torch.empty((m1 - m0, n1 - n0, g), dtype=torch.int32, device=q.device)
    ws, ws_bytes = (None, 0)
    if path in (PATH_GEMM, PATH_GEMM_RAW):
        ws, ws_bytes = _workspace(w, m, I8, PATH_GEMM, q.device, workspace)
    st = w.struct()
    _check(lib().bpw_partials(ctypes.byref(st), _ptr(q), m, path, m0, m1, n0, n1, _ptr(out),
                              _ptr(ws), ws_bytes, _stream(q.device)))
    return out


def probe(kind: int, src, dst) -> None:
    """HBM probe (bpw_probe): streaming read or copy of ``src.nbytes`` bytes."""
    nbytes = src.numel() * src.element_size()
    if not src.is_contiguous() or not dst.is_contiguous():
        raise ValueError("src and dst must be contiguous")
    if dst.device != src.device:
        raise ValueError("src and dst must be on one device")
    need = nbytes if kind == PROBE_COPY else probe_blocks(nbytes) * 4
    if dst.numel() * dst.element_size() < need:
        raise ValueError(f"dst holds {dst.numel() * dst.element_size()} bytes, the probe writes {need}")
    _check_gpu("src", src)
    _check(lib().bpw_probe(kind, _ptr(src), _ptr(dst), nbytes, _stream(src.device)))


def probe_blocks(nbytes: int) -> int:
    return lib().bpw_probe_blocks(nbytes)
