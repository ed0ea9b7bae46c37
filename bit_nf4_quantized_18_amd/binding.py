"""Thin ctypes binding over libqlora_nf4.so (the C ABI in include/qlora_nf4.h).

Argument marshalling only: every step of the layer runs in the HIP kernels.
Tensors are torch tensors on the current HIP device; work is enqueued on
torch's current stream. There is no fallback: if the library is missing the
functions raise.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqlora_nf4.so")

QLORA_BF16, QLORA_F32, QLORA_F16 = 0, 1, 2
MAX_RANK = 128
BLOCK, DQ_GROUP = 64, 256

STATUS = {0: "QLORA_OK", -1: "QLORA_ERR_NULL", -2: "QLORA_ERR_SHAPE", -3: "QLORA_ERR_ALIGN",
          -4: "QLORA_ERR_UNSUPPORTED", -5: "QLORA_ERR_WORKSPACE", -6: "QLORA_ERR_HIP"}

# Every symbol include/qlora_nf4.h declares.
EXPORTS = ("qlora_nf4_quantize", "qlora_nf4_dequantize", "qlora_linear_fwd", "qlora_linear_bwd",
           "qlora_linear_workspace_bytes", "qlora_linear_fwd_grouped", "qlora_linear_bwd_grouped",
           "qlora_linear_grouped_workspace_bytes", "qlora_status_string", "qlora_nf4_levels",
           "qlora_quantize_codebook", "qlora_codebook_levels", "qlora_merge", "qlora_unmerge",
           "qlora_requantize", "qlora_linear_dropout_workspace_bytes", "qlora_linear_fwd_dropout",
           "qlora_linear_bwd_dropout", "qlora_dropout_mask", "qlora_linear_fwd_f16", "qlora_linear_bwd_f16",
           "qlora_linear_fwd_grouped_f16", "qlora_linear_bwd_grouped_f16", "qlora_linear_fwd_dropout_f16",
           "qlora_linear_bwd_dropout_f16", "qlora_linear_fwd_noalloc")
NOALLOC_SCRATCH_BYTES = 16 << 20  # QLORA_NOALLOC_SCRATCH_BYTES

CODEBOOK_NF4 = 0   # normal-quantile levels
CODEBOOK_INT4 = 1  # 16 evenly spaced levels on [-1, 1]


class QloraError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_string(status)})")


class NF4WeightC(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("k", ctypes.c_int64), ("codes", ctypes.c_void_p),
                ("scale_codes", ctypes.c_void_p), ("group_scale", ctypes.c_void_p), ("absmax", ctypes.c_void_p),
                ("double_quant", ctypes.c_int32), ("codebook", ctypes.c_int32)]


_LIB = None


def load():
    """Load the library (once). Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m bit_nf4_quantized_18_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    wp = ctypes.POINTER(NF4WeightC)
    lib.qlora_nf4_quantize.argtypes = [vp, i64, i32, vp, vp, vp, vp, vp]
    lib.qlora_nf4_quantize.restype = i32
    lib.qlora_nf4_dequantize.argtypes = [wp, i32, vp, vp]
    lib.qlora_nf4_dequantize.restype = i32
    lib.qlora_linear_fwd.argtypes = [wp, vp, i64, vp, vp, i32, f32, vp, vp, vp, sz, vp]
    lib.qlora_linear_fwd.restype = i32
    lib.qlora_linear_bwd.argtypes = [wp, vp, vp, i64, vp, vp, i32, f32, vp, vp, vp, vp, vp, sz, vp]
    lib.qlora_linear_bwd.restype = i32
    lib.qlora_linear_fwd_f16.argtypes = lib.qlora_linear_fwd.argtypes
    lib.qlora_linear_fwd_f16.restype = i32
    lib.qlora_linear_bwd_f16.argtypes = lib.qlora_linear_bwd.argtypes
    lib.qlora_linear_bwd_f16.restype = i32
    lib.qlora_linear_fwd_noalloc.argtypes = [wp, vp, i64, vp, vp, i32, f32, vp, vp, vp]
    lib.qlora_linear_fwd_noalloc.restype = i32
    lib.qlora_linear_workspace_bytes.argtypes = [i64, i64, i64, i32]
    lib.qlora_linear_workspace_bytes.restype = sz
    p64 = ctypes.POINTER(ctypes.c_int64)
    lib.qlora_linear_fwd_grouped.argtypes = [wp, i32, p64, vp, i64, vp, vp, i32, f32, vp, vp, vp, sz, vp]
    lib.qlora_linear_fwd_grouped.restype = i32
    lib.qlora_linear_bwd_grouped.argtypes = [wp, i32, p64, vp, vp, i64, vp, vp, i32, f32, vp, vp, vp, vp, vp, sz, vp]
    lib.qlora_linear_bwd_grouped.restype = i32
    lib.qlora_linear_grouped_workspace_bytes.argtypes = [i64, i64, i64, i32, i32]
    lib.qlora_linear_grouped_workspace_bytes.restype = sz
    lib.qlora_status_string.argtypes = [i32]
    lib.qlora_status_string.restype = ctypes.c_char_p
    lib.qlora_nf4_levels.argtypes = [ctypes.POINTER(ctypes.c_float)]
    lib.qlora_nf4_levels.restype = i32
    lib.qlora_quantize_codebook.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp, vp]
    lib.qlora_quantize_codebook.restype = i32
    lib.qlora_codebook_levels.argtypes = [i32, ctypes.POINTER(ctypes.c_float)]
    lib.qlora_codebook_levels.restype = i32
    lib.qlora_merge.argtypes = [wp, vp, vp, i32, f32, i32, vp, vp]
    lib.qlora_merge.restype = i32
    lib.qlora_unmerge.argtypes = [vp, i32, i64, i64, vp, vp, i32, f32, vp, vp]
    lib.qlora_unmerge.restype = i32
    lib.qlora_requantize.argtypes = [wp, vp, vp, i32, f32, i32, i32, vp, vp, vp, vp, vp, vp]
    lib.qlora_requantize.restype = i32
    lib.qlora_linear_dropout_workspace_bytes.argtypes = [i64, i64, i64, i32]
    lib.qlora_linear_dropout_workspace_bytes.restype = sz
    lib.qlora_linear_fwd_dropout.argtypes = [wp, vp, i64, vp, vp, i32, f32, vp, f32, vp, vp, vp, sz, vp]
    lib.qlora_linear_fwd_dropout.restype = i32
    lib.qlora_linear_bwd_dropout.argtypes = [wp, vp, vp, i64, vp, vp, i32, f32, vp, f32, vp, vp, vp, vp, vp, sz, vp]
    lib.qlora_linear_bwd_dropout.restype = i32
    lib.qlora_dropout_mask.argtypes = [ctypes.c_uint64, ctypes.c_uint64, i64, f32, vp, vp]
    lib.qlora_dropout_mask.restype = i32
    # the fp16 compute calls share their bf16 counterparts' signatures
    for name in ("grouped", "dropout"):
        for d in ("fwd", "bwd"):
            f16 = getattr(lib, f"qlora_linear_{d}_{name}_f16")
            f16.argtypes = getattr(lib, f"qlora_linear_{d}_{name}").argtypes
            f16.restype = i32
    _LIB = lib
    return lib


def status_string(status: int) -> str:
    return load().qlora_status_string(status).decode()


def levels(codebook: int = CODEBOOK_NF4):
    """The 16 float32 levels the kernels use for `codebook` (host call)."""
    buf = (ctypes.c_float * 16)()
    if codebook == CODEBOOK_NF4:
        n = load().qlora_nf4_levels(buf)
    else:
        n = load().qlora_codebook_levels(int(codebook), buf)
    if n != 16:
        raise QloraError(n, "qlora_codebook_levels")
    return list(buf)


def workspace_bytes(m: int, n: int, k: int, r: int) -> int:
    return int(load().qlora_linear_workspace_bytes(m, n, k, r))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status: int, where: str):
    if status != 0:
        raise QloraError(status, where)


def _need(t, name, shape, dtypes, device, optional=False):
    """Raise unless ``t`` is a contiguous tensor of one of ``dtypes`` on
    ``device`` with exactly ``shape`` (None allowed only when ``optional``).
    The library takes raw pointers and sizes, so a tensor that does not match
    what the call assumes is refused here rather than read out of bounds."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the weight on {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_packed(q):
    """The packed weight's buffers: uint8 codes / scale codes, float32 group
    scales / absmax, contiguous, on one device, at least as long as n x k needs."""
    import torch

    dev = q.codes.device
    numel = q.n * q.k
    nb = -(-numel // BLOCK)
    ng = -(-nb // DQ_GROUP)
    for name, t, dt, need in (("codes", q.codes, torch.uint8, (numel + 1) // 2),
                              ("scale_codes", q.scale_codes, torch.uint8, nb if q.double_quant else 0),
                              ("group_scale", q.group_scale, torch.float32, ng if q.double_quant else 0),
                              ("absmax", q.absmax, torch.float32, 0 if q.double_quant else nb)):
        if t is None:
            if need:
                raise ValueError(f"packed weight: {name} is required")
            continue
        if t.device != dev or t.dtype != dt or not t.is_contiguous() or t.numel() < need:
            raise ValueError(f"packed weight: {name} must be a contiguous {dt} tensor on {dev} "
                             f"with at least {need} elements")
    return dev


def _half_types(t, name):
    import torch

    if t.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"{name} must be bfloat16 or float16, got {t.dtype}")
    return (t.dtype,)


def _need_ws(ws, device):
    import torch

    if ws is not None and (ws.device != device or ws.dtype != torch.uint8 or not ws.is_contiguous()):
        raise ValueError("ws must be a contiguous uint8 tensor on the weight's device")


def _need_adapter(a, b, r, k, n, types, device, rb=None):
    if (a is None) != (b is None):
        raise ValueError("a and b are given together or not at all")
    if a is None:
        return
    _need(a, "a", (r, k), types, device)
    _need(b, "b", (n, r if rb is None else rb), types, device)


@dataclasses.dataclass
class PackedNF4:
    """A packed NF4 weight on the device (n x k row-major)."""
    n: int
    k: int
    codes: "object"                 # uint8 [ceil(n*k/2)]
    double_quant: bool
    scale_codes: "object" = None    # uint8 [nblocks]        (double quant)
    group_scale: "object" = None    # float32 [ngroups]      (double quant)
    absmax: "object" = None         # float32 [nblocks]      (exact a_b; required without double quant)
    codebook: int = CODEBOOK_NF4    # level table the codes index

    def c_struct(self) -> NF4WeightC:
        return NF4WeightC(self.n, self.k, self.codes.data_ptr(),
                          None if self.scale_codes is None else self.scale_codes.data_ptr(),
                          None if self.group_scale is None else self.group_scale.data_ptr(),
                          None if self.absmax is None else self.absmax.data_ptr(), int(self.double_quant),
                          int(self.codebook))


def _empty(n, dtype, device):
    import torch

    # 16 extra bytes so even empty-ish buffers get a real, aligned allocation
    return torch.empty(max(n, 1), dtype=dtype, device=device)


def quantize(w, double_quant: bool = True, keep_absmax: bool = False, codebook: int = CODEBOOK_NF4) -> PackedNF4:
    """Quantize a float32 CUDA tensor (any shape; flattened row-major).
    A 2-D tensor gives n, k = its shape; other shapes give n = 1.
    codebook: CODEBOOK_NF4 (qlora_nf4_quantize) or CODEBOOK_INT4."""
    import torch

    if w.dtype != torch.float32 or not w.is_cuda:
        raise TypeError("quantize expects a float32 tensor on the GPU")
    w = w.contiguous()
    numel = w.numel()
    n, k = (w.shape[0], w.shape[1]) if w.dim() == 2 else (1, numel)
    nb = -(-numel // BLOCK)
    ng = -(-nb // DQ_GROUP)
    dev = w.device
    codes = _empty((numel + 1) // 2, torch.uint8, dev)
    sc = _empty(nb, torch.uint8, dev) if double_quant else None
    gs = _empty(ng, torch.float32, dev) if double_quant else None
    am = _empty(nb, torch.float32, dev) if (keep_absmax or not double_quant) else None
    if codebook == CODEBOOK_NF4:
        st = load().qlora_nf4_quantize(_ptr(w), numel, int(double_quant), _ptr(codes), _ptr(sc), _ptr(gs),
                                       _ptr(am), _stream())
        _check(st, "qlora_nf4_quantize")
    else:
        st = load().qlora_quantize_codebook(_ptr(w), numel, int(double_quant), int(codebook), _ptr(codes),
                                            _ptr(sc), _ptr(gs), _ptr(am), _stream())
        _check(st, "qlora_quantize_codebook")
    return PackedNF4(n, k, codes[: (numel + 1) // 2], double_quant, None if sc is None else sc[:nb],
                     None if gs is None else gs[:ng], None if am is None else am[:nb], int(codebook))


def dequantize(q: PackedNF4, dtype=None):
    import torch

    dtype = torch.bfloat16 if dtype is None else dtype
    code = {torch.bfloat16: QLORA_BF16, torch.float32: QLORA_F32, torch.float16: QLORA_F16}[dtype]
    dev = _need_packed(q)
    out = torch.empty((q.n, q.k), dtype=dtype, device=dev)
    ws = q.c_struct()
    _check(load().qlora_nf4_dequantize(ctypes.byref(ws), code, _ptr(out), _stream()), "qlora_nf4_dequantize")
    return out


def _adapter(a, b, n, k, device):
    """(r, a pointer, b pointer) of a bf16 adapter a (r, k), b (n, r), or none."""
    import torch

    r = 0 if a is None else a.shape[0]
    _need_adapter(a, b, r, k, n, (torch.bfloat16,), device)
    return r, _ptr(a), _ptr(b)


def merge(q: PackedNF4, a, b, alpha: float, dtype=None, out=None):
    """W16 + fl32(alpha/r) B A with the float32 order of qlora_merge.
    a: bf16 (r, k), b: bf16 (n, r), or both None. Returns (n, k) of dtype."""
    import torch

    dtype = torch.bfloat16 if dtype is None else dtype
    code = {torch.bfloat16: QLORA_BF16, torch.float32: QLORA_F32}[dtype]
    dev = _need_packed(q)
    out = torch.empty((q.n, q.k), dtype=dtype, device=dev) if out is None else out
    _need(out, "out", (q.n, q.k), (dtype,), dev)
    r, ap, bp = _adapter(a, b, q.n, q.k, dev)
    ws = q.c_struct()
    _check(load().qlora_merge(ctypes.byref(ws), ap, bp, r, float(alpha), code, _ptr(out), _stream()), "qlora_merge")
    return out


def unmerge(merged, a, b, alpha: float, out=None):
    """merged - fl32(alpha/r) B A (qlora_unmerge); merged: bf16 or float32
    (n, k). ``out`` may be ``merged`` (in place)."""
    import torch

    code = {torch.bfloat16: QLORA_BF16, torch.float32: QLORA_F32}[merged.dtype]
    if merged.dim() != 2:
        raise ValueError("merged must be 2-D (n, k)")
    dev = merged.device
    _need(merged, "merged", tuple(merged.shape), (merged.dtype,), dev)
    out = torch.empty_like(merged) if out is None else out
    _need(out, "out", tuple(merged.shape), (merged.dtype,), dev)
    r, ap, bp = _adapter(a, b, merged.shape[0], merged.shape[1], dev)
    _check(load().qlora_unmerge(_ptr(merged), code, merged.shape[0], merged.shape[1], ap, bp, r, float(alpha),
                                _ptr(out), _stream()), "qlora_unmerge")
    return out


def requantize(q: PackedNF4, a, b, alpha: float, double_quant: bool = True, codebook: int = CODEBOOK_NF4,
               keep_absmax: bool = False):
    """The merged weight quantized again (qlora_requantize). Returns
    (PackedNF4 of the merged weight, merged float32 (n, k))."""
    import torch

    dev = _need_packed(q)
    numel = q.n * q.k
    nb = -(-numel // BLOCK)
    ng = -(-nb // DQ_GROUP)
    merged = torch.empty((q.n, q.k), dtype=torch.float32, device=dev)
    codes = _empty((numel + 1) // 2, torch.uint8, dev)
    sc = _empty(nb, torch.uint8, dev) if double_quant else None
    gs = _empty(ng, torch.float32, dev) if double_quant else None
    am = _empty(nb, torch.float32, dev) if (keep_absmax or not double_quant) else None
    r, ap, bp = _adapter(a, b, q.n, q.k, dev)
    ws = q.c_struct()
    _check(load().qlora_requantize(ctypes.byref(ws), ap, bp, r, float(alpha), int(double_quant), int(codebook),
                                   _ptr(merged), _ptr(codes), _ptr(sc), _ptr(gs), _ptr(am), _stream()),
           "qlora_requantize")
    packed = PackedNF4(q.n, q.k, codes[: (numel + 1) // 2], double_quant, None if sc is None else sc[:nb],
                       None if gs is None else gs[:ng], None if am is None else am[:nb], int(codebook))
    return packed, merged


def _workspace(m, n, k, r, device):
    import torch

    nbytes = workspace_bytes(m, n, k, r)
    return (torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes else None), nbytes


def linear_fwd(q: PackedNF4, x, a=None, b=None, alpha: float = 0.0, want_h: bool = True, out=None, h_out=None,
               ws=None):
    """Y = X W16^T + (alpha/r) (X A^T) B^T. x: bf16 (m, k), or fp16 for the
    fp16 compute entry point (A, B and Y then fp16 too). Returns (y, h).
    ``out``, ``h_out`` and ``ws`` (uint8 workspace) may be preallocated."""
    import torch

    dev = _need_packed(q)
    m = x.shape[0]
    r = 0 if a is None else a.shape[0]
    t16 = _half_types(x, "x")
    f16 = x.dtype == torch.float16  # fp16 compute: the _f16 entry point
    _need(x, "x", (m, q.k), t16, dev)
    _need_adapter(a, b, r, q.k, q.n, t16, dev)
    y = out if out is not None else torch.empty((m, q.n), dtype=x.dtype, device=dev)
    h = h_out if h_out is not None else (
        torch.empty((m, r), dtype=torch.float32, device=dev) if (want_h and r > 0) else None)
    _need(y, "out", (m, q.n), t16, dev)
    _need(h, "h_out", (m, r), (torch.float32,), dev, optional=True)
    _need_ws(ws, dev)
    if ws is None:
        ws, nbytes = _workspace(m, q.n, q.k, r, dev)
    else:
        nbytes = ws.numel()
    wc = q.c_struct()
    fn = load().qlora_linear_fwd_f16 if f16 else load().qlora_linear_fwd
    st = fn(ctypes.byref(wc), _ptr(x), m, _ptr(a), _ptr(b), r, float(alpha), _ptr(y), _ptr(h), _ptr(ws), nbytes,
            _stream())
    _check(st, "qlora_linear_fwd_f16" if f16 else "qlora_linear_fwd")
    return y, h


def linear_fwd_noalloc(q: PackedNF4, x, a=None, b=None, alpha: float = 0.0, out=None, h_out=None):
    """qlora_linear_fwd_noalloc: the bf16 forward on the library's own scratch
    array (no workspace). ``out`` (bf16 (m, n)) and ``h_out`` (float32
    (m, r)) may be preallocated; h is returned only when ``h_out`` is given."""
    import torch

    dev = _need_packed(q)
    m = x.shape[0]
    r = 0 if a is None else a.shape[0]
    _need(x, "x", (m, q.k), (torch.bfloat16,), dev)
    _need_adapter(a, b, r, q.k, q.n, (torch.bfloat16,), dev)
    y = out if out is not None else torch.empty((m, q.n), dtype=x.dtype, device=dev)
    _need(y, "out", (m, q.n), (torch.bfloat16,), dev)
    _need(h_out, "h_out", (m, r), (torch.float32,), dev, optional=True)
    wc = q.c_struct()
    st = load().qlora_linear_fwd_noalloc(ctypes.byref(wc), _ptr(x), m, _ptr(a), _ptr(b), r, float(alpha), _ptr(y),
                                         _ptr(h_out), _stream())
    _check(st, "qlora_linear_fwd_noalloc")
    return y, h_out


def linear_bwd(q: PackedNF4, x, dy, a=None, b=None, alpha: float = 0.0, h=None, need_dx: bool = True,
               dx=None, da=None, db=None, ws=None):
    """Returns (dx (m,k) of dy's 16-bit type or None, dA float32 (r,k), dB
    float32 (n,r)). fp16 inputs take the fp16 entry point. Outputs and the
    workspace may be preallocated."""
    import torch

    dev = _need_packed(q)
    m = dy.shape[0]
    r = 0 if a is None else a.shape[0]
    t16 = _half_types(dy, "dy")
    f16 = dy.dtype == torch.float16
    _need(dy, "dy", (m, q.n), t16, dev)
    _need(x, "x", (m, q.k), t16, dev, optional=r == 0)
    _need_adapter(a, b, r, q.k, q.n, t16, dev)
    _need(h, "h", (m, r), (torch.float32,), dev, optional=True)
    if dx is None and need_dx:
        dx = torch.empty((m, q.k), dtype=dy.dtype, device=dev)
    if r and da is None:
        da = torch.empty((r, q.k), dtype=torch.float32, device=dev)
    if r and db is None:
        db = torch.empty((q.n, r), dtype=torch.float32, device=dev)
    _need(dx, "dx", (m, q.k), t16, dev, optional=True)
    _need(da, "da", (r, q.k), (torch.float32,), dev, optional=r == 0)
    _need(db, "db", (q.n, r), (torch.float32,), dev, optional=r == 0)
    _need_ws(ws, dev)
    if ws is None:
        ws, nbytes = _workspace(m, q.n, q.k, r, dev)
    else:
        nbytes = ws.numel()
    wc = q.c_struct()
    fn = load().qlora_linear_bwd_f16 if f16 else load().qlora_linear_bwd
    st = fn(ctypes.byref(wc), _ptr(x), _ptr(dy), m, _ptr(a), _ptr(b), r, float(alpha), _ptr(h), _ptr(dx), _ptr(da),
            _ptr(db), _ptr(ws), nbytes, _stream())
    _check(st, "qlora_linear_bwd_f16" if f16 else "qlora_linear_bwd")
    return dx, da, db


def dropout_workspace_bytes(m: int, n: int, k: int, r: int) -> int:
    return int(load().qlora_linear_dropout_workspace_bytes(m, n, k, r))


def _drop_ws(ws, m, n, k, r, dev):
    import torch

    if ws is not None:
        return ws, ws.numel()
    nbytes = dropout_workspace_bytes(m, n, k, r)
    return (torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None), nbytes


def dropout_mask(seed: int, offset: int, shape, p: float, out=None):
    """Keep mask (uint8, 1 = kept) drawn on the GPU by qlora_dropout_mask:
    elements offset .. offset + numel - 1 of the stream of `seed`."""
    import torch

    out = torch.empty(shape, dtype=torch.uint8, device="cuda") if out is None else out
    _check(load().qlora_dropout_mask(int(seed), int(offset), out.numel(), float(p), _ptr(out), _stream()),
           "qlora_dropout_mask")
    return out


def linear_fwd_dropout(q: PackedNF4, x, a, b, alpha: float, keep, p: float, want_h: bool = True, out=None,
                       h_out=None, ws=None):
    """qlora_linear_fwd_dropout. keep: uint8 (m, k) on the GPU, non-zero =
    kept; p: drop probability. Returns (y, h) with h from the dropped input."""
    import torch

    dev = _need_packed(q)
    m, r = x.shape[0], a.shape[0]
    t16 = _half_types(x, "x")
    _need(x, "x", (m, q.k), t16, dev)
    _need_adapter(a, b, r, q.k, q.n, t16, dev)
    _need(keep, "keep", (m, q.k), (torch.uint8,), dev)
    y = out if out is not None else torch.empty((m, q.n), dtype=x.dtype, device=dev)
    h = h_out if h_out is not None else (torch.empty((m, r), dtype=torch.float32, device=dev) if want_h else None)
    _need(y, "out", (m, q.n), t16, dev)
    _need(h, "h_out", (m, r), (torch.float32,), dev, optional=True)
    _need_ws(ws, dev)
    ws, nbytes = _drop_ws(ws, m, q.n, q.k, r, dev)
    wc = q.c_struct()
    fn = load().qlora_linear_fwd_dropout_f16 if x.dtype == torch.float16 else load().qlora_linear_fwd_dropout
    st = fn(ctypes.byref(wc), _ptr(x), m, _ptr(a), _ptr(b), r, float(alpha),
            _ptr(keep), float(p), _ptr(y), _ptr(h), _ptr(ws), nbytes, _stream())
    _check(st, "qlora_linear_fwd_dropout")
    return y, h


def linear_bwd_dropout(q: PackedNF4, x, dy, a, b, alpha: float, keep, p: float, h=None, need_dx: bool = True,
                       dx=None, da=None, db=None, ws=None):
    """qlora_linear_bwd_dropout with the forward's mask. Returns (dx, dA, dB)."""
    import torch

    dev = _need_packed(q)
    m, r = dy.shape[0], a.shape[0]
    t16 = _half_types(dy, "dy")
    _need(dy, "dy", (m, q.n), t16, dev)
    _need(x, "x", (m, q.k), t16, dev)
    _need_adapter(a, b, r, q.k, q.n, t16, dev)
    _need(keep, "keep", (m, q.k), (torch.uint8,), dev)
    _need(h, "h", (m, r), (torch.float32,), dev, optional=True)
    if dx is None and need_dx:
        dx = torch.empty((m, q.k), dtype=dy.dtype, device=dev)
    da = torch.empty((r, q.k), dtype=torch.float32, device=dev) if da is None else da
    db = torch.empty((q.n, r), dtype=torch.float32, device=dev) if db is None else db
    _need(dx, "dx", (m, q.k), t16, dev, optional=True)
    _need(da, "da", (r, q.k), (torch.float32,), dev)
    _need(db, "db", (q.n, r), (torch.float32,), dev)
    _need_ws(ws, dev)
    ws, nbytes = _drop_ws(ws, m, q.n, q.k, r, dev)
    wc = q.c_struct()
    fn = load().qlora_linear_bwd_dropout_f16 if dy.dtype == torch.float16 else load().qlora_linear_bwd_dropout
    st = fn(ctypes.byref(wc), _ptr(x), _ptr(dy), m, _ptr(a), _ptr(b), r, float(alpha),
            _ptr(keep), float(p), _ptr(h), _ptr(dx), _ptr(da), _ptr(db), _ptr(ws),
            nbytes, _stream())
    _check(st, "qlora_linear_bwd_dropout")
    return dx, da, db


def grouped_workspace_bytes(m: int, n: int, k: int, g: int, r: int) -> int:
    return int(load().qlora_linear_grouped_workspace_bytes(m, n, k, g, r))


def _parts(parts):
    arr = (ctypes.c_int64 * len(parts))(*[int(p) for p in parts])
    return arr


def linear_fwd_grouped(q: PackedNF4, parts, x, a, b, alpha: float, want_h: bool = True, out=None, h_out=None,
                       ws=None):
    """Grouped forward over a stacked weight (row counts ``parts``): y (m, n)
    with part l's columns = X W_l^T + (alpha/r) (X A_l^T) B_l^T; a is the
    stacked (g r, k) A, b the stacked (n, r) B. Returns (y, h (m, g r))."""
    import torch

    dev = _need_packed(q)
    m, g, r = x.shape[0], len(parts), b.shape[1]
    t16 = _half_types(x, "x")
    _need(x, "x", (m, q.k), t16, dev)
    _need_adapter(a, b, g * r, q.k, q.n, t16, dev, rb=r)
    y = out if out is not None else torch.empty((m, q.n), dtype=x.dtype, device=dev)
    h = h_out if h_out is not None else (torch.empty((m, g * r), dtype=torch.float32, device=dev) if want_h else None)
    _need(y, "out", (m, q.n), t16, dev)
    _need(h, "h_out", (m, g * r), (torch.float32,), dev, optional=True)
    _need_ws(ws, dev)
    if ws is None:
        nbytes = grouped_workspace_bytes(m, q.n, q.k, g, r)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    nbytes = ws.numel()
    wc = q.c_struct()
    pa = _parts(parts)
    fn = load().qlora_linear_fwd_grouped_f16 if x.dtype == torch.float16 else load().qlora_linear_fwd_grouped
    st = fn(ctypes.byref(wc), g, pa, _ptr(x), m, _ptr(a), _ptr(b), r, float(alpha),
            _ptr(y), _ptr(h), _ptr(ws), nbytes, _stream())
    _check(st, "qlora_linear_fwd_grouped")
    return y, h


def linear_bwd_grouped(q: PackedNF4, parts, x, dy, a, b, alpha: float, h=None, need_dx: bool = True, dx=None,
                       da=None, db=None, ws=None):
    """Grouped backward: (dx (m, k) = sum over parts, dA stacked (g r, k),
    dB stacked (n, r))."""
    import torch

    dev = _need_packed(q)
    m, g, r = dy.shape[0], len(parts), b.shape[1]
    t16 = _half_types(dy, "dy")
    _need(dy, "dy", (m, q.n), t16, dev)
    _need(x, "x", (m, q.k), t16, dev)
    _need_adapter(a, b, g * r, q.k, q.n, t16, dev, rb=r)
    _need(h, "h", (m, g * r), (torch.float32,), dev, optional=True)
    if dx is None and need_dx:
        dx = torch.empty((m, q.k), dtype=dy.dtype, device=dev)
    if da is None:
        da = torch.empty((g * r, q.k), dtype=torch.float32, device=dev)
    if db is None:
        db = torch.empty((q.n, r), dtype=torch.float32, device=dev)
    _need(dx, "dx", (m, q.k), t16, dev, optional=True)
    _need(da, "da", (g * r, q.k), (torch.float32,), dev)
    _need(db, "db", (q.n, r), (torch.float32,), dev)
    _need_ws(ws, dev)
    if ws is None:
        nbytes = grouped_workspace_bytes(m, q.n, q.k, g, r)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    nbytes = ws.numel()
    wc = q.c_struct()
    pa = _parts(parts)
    fn = load().qlora_linear_bwd_grouped_f16 if dy.dtype == torch.float16 else load().qlora_linear_bwd_grouped
    st = fn(ctypes.byref(wc), g, pa, _ptr(x), _ptr(dy), m, _ptr(a), _ptr(b), r,
            float(alpha), _ptr(h), _ptr(dx), _ptr(da), _ptr(db), _ptr(ws), nbytes,
            _stream())
    _check(st, "qlora_linear_bwd_grouped")
    return dx, da, db


# ---------------------------------------------------------------- storage
# A packed weight on disk: one .npz of plain arrays (no pickled objects), the
# buffers byte for byte as the kernels read them plus n, k, the scale-code kind
# and the codebook id.
def save_packed(path, q: PackedNF4):
    """Write ``q``'s buffers (copied to the host) and sizes to ``path`` (.npz)."""
    import numpy as np

    _need_packed(q)
    arrays = {"n": np.int64(q.n), "k": np.int64(q.k), "double_quant": np.int32(int(q.double_quant)),
              "codebook": np.int32(int(q.codebook)), "codes": q.codes.cpu().numpy()}
    for name in ("scale_codes", "group_scale", "absmax"):
        t = getattr(q, name)
        if t is not None:
            arrays[name] = t.cpu().numpy()
    np.savez(path, **arrays)


def load_packed(path, device="cuda") -> PackedNF4:
    """Read a packed weight written by ``save_packed`` onto ``device``; the
    buffer lengths are checked against n and k."""
    import numpy as np
    import torch

    with np.load(path, allow_pickle=False) as f:
        n, k = int(f["n"]), int(f["k"])
        dq, cb = int(f["double_quant"]), int(f["codebook"])
        get = (lambda name, dt: torch.from_numpy(np.ascontiguousarray(f[name], dtype=dt)).to(device)
               if name in f.files else None)
        q = PackedNF4(n, k, get("codes", np.uint8), dq, get("scale_codes", np.uint8),
                      get("group_scale", np.float32), get("absmax", np.float32), cb)
    _need_packed(q)
    return q
