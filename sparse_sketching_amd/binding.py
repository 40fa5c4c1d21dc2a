"""Python binding of libsksketch (the C ABI declared in include/sk.h).

Argument marshalling only: every step of the sketch runs in the library's
HIP kernels.  torch supplies device memory (tensors) and the stream
(torch.cuda.current_stream() unless one is given).  The low-level functions
carry the C names and take tensors or raw device addresses; the helpers
below them allocate outputs with torch and call those functions.

The library is loaded from this package directory on first use; when it is
missing or was built for another device the call fails loudly.  There is no
CPU fallback.
"""
import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsksketch.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "sk.h")

SK_OK, SK_ERR_NULL, SK_ERR_SHAPE, SK_ERR_ALIGN, SK_ERR_UNSUPPORTED, SK_ERR_HIP, SK_ERR_ARG = range(7)
SK_ACCUMULATE = 1
SK_VARIANT_FLAT = 2
SK_VARIANT_LDS = 4
SK_VARIANT_REG = 8
SK_COMBINE_F32 = 16
SK_PRECISION_F32 = 0
SK_PRECISION_F16ACC = 1
SK_PRECISION_LOWP = 2
SK_FORMAT_F16 = 0
SK_FORMAT_BF16 = 1
SK_CONVERT_RN = 0
SK_CONVERT_SR = 1
SK_WIRING_SHIFT = 0
SK_WIRING_AFFINE = 1
SK_BLOCKPERM_KERNEL_COMPONENT = 0
SK_BLOCKPERM_KERNEL_SLICE = 1
SK_BLOCKPERM_KERNEL_REGISTER = 2

_c = ctypes
_SIGNATURES = {
    "sk_meta_generate": (_c.c_int, [_c.c_uint64, _c.c_int64, _c.c_int64, _c.c_int32, _c.c_int32,
                                     _c.c_void_p, _c.c_void_p, _c.c_void_p]),
    "sk_apply_f32": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_int32, _c.c_int64, _c.c_void_p,
                                _c.c_void_p, _c.c_int32, _c.c_void_p, _c.c_int32, _c.c_int64,
                                _c.c_uint32, _c.c_void_p]),
    "sk_apply_f16acc": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_int32, _c.c_int64, _c.c_void_p,
                                   _c.c_void_p, _c.c_int32, _c.c_void_p, _c.c_int32, _c.c_int64,
                                   _c.c_uint32, _c.c_void_p]),
    "sk_apply_f32_ws": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_int32, _c.c_int64, _c.c_void_p,
                                   _c.c_void_p, _c.c_int32, _c.c_void_p, _c.c_int32, _c.c_int64,
                                   _c.c_uint32, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "sk_apply_f16acc_ws": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_int32, _c.c_int64,
                                      _c.c_void_p, _c.c_void_p, _c.c_int32, _c.c_void_p,
                                      _c.c_int32, _c.c_int64, _c.c_uint32, _c.c_void_p,
                                      _c.c_size_t, _c.c_void_p]),
    "sk_apply_workspace_size": (_c.c_int, [_c.c_int32, _c.c_int64, _c.c_int32, _c.c_int32,
                                           _c.c_int32, _c.c_uint32, _c.POINTER(_c.c_size_t)]),
    "sk_apply_blockperm": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_int32, _c.c_int64, _c.c_int32,
                                      _c.c_int32, _c.c_int32, _c.c_int32, _c.c_uint64, _c.c_void_p,
                                      _c.c_int64, _c.c_uint32, _c.c_void_p]),
    "sk_lstsq_qr_f32": (_c.c_int, [_c.c_void_p, _c.c_int32, _c.c_int32, _c.c_int64, _c.c_void_p,
                                   _c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "sk_lstsq_workspace_size": (_c.c_int, [_c.c_int32, _c.c_int32, _c.POINTER(_c.c_size_t)]),
    "sk_lds_plan_describe": (_c.c_int, [_c.c_int32, _c.c_int64, _c.c_int32, _c.c_int64, _c.c_int32,
                                        _c.c_int32, _c.c_int32, _c.c_int32, _c.c_int32,
                                        _c.POINTER(_c.c_int64)]),
    "sk_sketch_f32": (_c.c_int, [_c.c_uint64, _c.c_int64, _c.c_void_p, _c.c_int64, _c.c_int32,
                                 _c.c_int64, _c.c_int32, _c.c_int32, _c.c_void_p, _c.c_int64,
                                 _c.c_uint32, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "sk_sketch_f16acc": (_c.c_int, [_c.c_uint64, _c.c_int64, _c.c_void_p, _c.c_int64, _c.c_int32,
                                    _c.c_int64, _c.c_int32, _c.c_int32, _c.c_void_p, _c.c_int64,
                                    _c.c_uint32, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "sk_sketch_f16acc_noalloc": (_c.c_int, [_c.c_uint64, _c.c_int64, _c.c_void_p, _c.c_int64,
                                            _c.c_int32, _c.c_int64, _c.c_int32, _c.c_int32,
                                            _c.c_void_p, _c.c_int64, _c.c_uint32, _c.c_void_p]),
    "sk_sketch_workspace_size": (_c.c_int, [_c.c_int32, _c.c_int64, _c.c_int32, _c.c_int32,
                                            _c.c_int32, _c.POINTER(_c.c_size_t)]),
    "sk_fused_plan_describe": (_c.c_int, [_c.c_int32, _c.c_int64, _c.c_int32, _c.c_int64,
                                          _c.c_int32, _c.c_int32, _c.c_int32, _c.c_int32,
                                          _c.c_int32, _c.POINTER(_c.c_int64)]),
    "sk_sketch_plan_describe": (_c.c_int, [_c.c_int32, _c.c_int64, _c.c_int32, _c.c_int64,
                                          _c.c_int32, _c.c_int32, _c.c_int32, _c.c_int32,
                                          _c.c_int32, _c.POINTER(_c.c_int64)]),
    "sk_apply_lowp": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_int32, _c.c_int64, _c.c_void_p,
                                 _c.c_void_p, _c.c_int32, _c.c_void_p, _c.c_int32, _c.c_int64,
                                 _c.c_int32, _c.c_int32, _c.c_uint64, _c.c_int64, _c.c_uint32,
                                 _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "sk_apply_blockperm_ex": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_int32, _c.c_int64,
                                         _c.c_int32, _c.c_int32, _c.c_int32, _c.c_int32,
                                         _c.c_int32, _c.c_uint64, _c.c_void_p, _c.c_int64,
                                         _c.c_uint32, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "sk_blockperm_workspace_size": (_c.c_int, [_c.c_int64, _c.c_int32, _c.c_int32, _c.c_int32,
                                               _c.c_int32, _c.c_int32, _c.c_int32,
                                               _c.POINTER(_c.c_size_t)]),
    "sk_blockperm_plan_describe": (_c.c_int, [_c.c_int64, _c.c_int32, _c.c_int32, _c.c_int32,
                                              _c.c_int32, _c.c_int32, _c.c_int32, _c.c_uint64,
                                              _c.c_int32, _c.c_int32, _c.POINTER(_c.c_int64)]),
    "sk_status_string": (_c.c_char_p, [_c.c_int]),
}

_lib = None


class SketchError(RuntimeError):
    """A non-zero sk_status returned by the library."""

    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")


def load(path=LIB_PATH):
    """Load libsksketch.so and bind every entry point (idempotent)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m sparse_sketching_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def header_symbols(header=HEADER):
    """Names of the functions declared in include/sk.h."""
    with open(header) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sk_\w+)\s*\(", text)))


def status_string(status):
    try:
        return load().sk_status_string(int(status)).decode()
    except RuntimeError:
        return "library not loaded"


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _nbytes(buf, nbytes):
    """Byte size of a workspace given as a tensor (its storage) or an address."""
    if buf is None:
        return 0
    if nbytes:
        return nbytes
    if isinstance(buf, int):
        raise ValueError("a raw workspace address needs workspace_bytes")
    return buf.numel() * buf.element_size()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, status):
    if status != SK_OK:
        raise SketchError(fn, status)


def _launch_stream(stream):
    """The torch stream object of a launch (None: the current stream)."""
    import torch
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream)
    return stream


def _keep(stream, *tensors):
    """Mark tensors the helpers allocated as in use on the launch stream, so
    the caching allocator does not hand their memory to another stream while
    the enqueued kernels may still read or write it."""
    s = _launch_stream(stream)
    for t in tensors:
        if t is not None:
            t.record_stream(s)


# ---- the C entry points, same names and argument order -------------------

def sk_meta_generate(seed, row_offset, m, d, zeta, row_idx, val, stream=None):
    _check("sk_meta_generate", load().sk_meta_generate(
        seed, row_offset, m, d, zeta, _ptr(row_idx), _ptr(val), _stream(stream)))


def sk_apply_f32(A, m, n, lda, row_idx, val, zeta, B, d, ldb, flags=0, stream=None):
    _check("sk_apply_f32", load().sk_apply_f32(
        _ptr(A), m, n, lda, _ptr(row_idx), _ptr(val), zeta, _ptr(B), d, ldb, flags,
        _stream(stream)))


def sk_apply_f16acc(A, m, n, lda, row_idx, val, zeta, B, d, ldb, flags=0, stream=None):
    _check("sk_apply_f16acc", load().sk_apply_f16acc(
        _ptr(A), m, n, lda, _ptr(row_idx), _ptr(val), zeta, _ptr(B), d, ldb, flags,
        _stream(stream)))


def sk_apply_f32_ws(A, m, n, lda, row_idx, val, zeta, B, d, ldb, flags=0, workspace=None,
                    workspace_bytes=0, stream=None):
    _check("sk_apply_f32_ws", load().sk_apply_f32_ws(
        _ptr(A), m, n, lda, _ptr(row_idx), _ptr(val), zeta, _ptr(B), d, ldb, flags,
        _ptr(workspace), _nbytes(workspace, workspace_bytes), _stream(stream)))


def sk_apply_f16acc_ws(A, m, n, lda, row_idx, val, zeta, B, d, ldb, flags=0, workspace=None,
                       workspace_bytes=0, stream=None):
    _check("sk_apply_f16acc_ws", load().sk_apply_f16acc_ws(
        _ptr(A), m, n, lda, _ptr(row_idx), _ptr(val), zeta, _ptr(B), d, ldb, flags,
        _ptr(workspace), _nbytes(workspace, workspace_bytes), _stream(stream)))


def sk_apply_workspace_size(precision, m, n, d, zeta, flags=0):
    """Bytes of workspace the apply call uses (0: none)."""
    out = ctypes.c_size_t(0)
    _check("sk_apply_workspace_size", load().sk_apply_workspace_size(
        precision, m, n, d, zeta, flags, ctypes.byref(out)))
    return out.value


def sk_apply_blockperm(A, m, n, lda, d, M, kappa, s, seed, Y, ldy, flags=0, stream=None):
    _check("sk_apply_blockperm", load().sk_apply_blockperm(
        _ptr(A), m, n, lda, d, M, kappa, s, seed, _ptr(Y), ldy, flags, _stream(stream)))


def sk_lstsq_qr_f32(SA, d, n, ld, Sb, x, workspace, workspace_bytes=0, stream=None):
    _check("sk_lstsq_qr_f32", load().sk_lstsq_qr_f32(
        _ptr(SA), d, n, ld, _ptr(Sb), _ptr(x), _ptr(workspace),
        _nbytes(workspace, workspace_bytes), _stream(stream)))


def sk_lstsq_workspace_size(d, n):
    out = ctypes.c_size_t(0)
    _check("sk_lstsq_workspace_size", load().sk_lstsq_workspace_size(d, n, ctypes.byref(out)))
    return out.value


def lstsq_qr(SA, Sb, stream=None):
    """x = argmin ||SA x - Sb||_2 (FP32 Householder QR in the library's
    kernel) for a float32 device matrix SA (d x n, n <= d <= 2048) and
    vector Sb; returns x as a float32 device tensor."""
    import torch
    _need_device(SA, torch.float32, "SA")
    _need_device(Sb, torch.float32, "Sb")
    d, n = SA.shape
    if Sb.shape != (d,) or not Sb.is_contiguous():
        raise ValueError("Sb must be a contiguous vector of SA's row count")
    x = torch.empty(n, dtype=torch.float32, device=SA.device)
    ws = torch.empty(sk_lstsq_workspace_size(d, n), dtype=torch.uint8, device=SA.device)
    sk_lstsq_qr_f32(SA, d, n, SA.stride(0), Sb, x, ws, 0, stream)
    _keep(stream, x, ws)
    return x


PLAN_FIELDS = ("lds", "words", "slice", "groups", "zg", "threads", "rows_per_chunk", "chunks",
               "slices", "grid", "lds_bytes", "ws_bytes")


def sk_lds_plan_describe(precision, m, n, lda, d, zeta, wide_ok, num_cu, max_lds):
    """The LDS launch plan as a dict (host computation, no device needed)."""
    out = (ctypes.c_int64 * len(PLAN_FIELDS))()
    _check("sk_lds_plan_describe", load().sk_lds_plan_describe(
        precision, m, n, lda, d, zeta, int(bool(wide_ok)), num_cu, max_lds, out))
    return dict(zip(PLAN_FIELDS, list(out)))


def sk_apply_blockperm_ex(A, m, n, lda, d, M, kappa, s, wiring, seed, Y, ldy, flags=0,
                          workspace=None, workspace_bytes=0, stream=None):
    _check("sk_apply_blockperm_ex", load().sk_apply_blockperm_ex(
        _ptr(A), m, n, lda, d, M, kappa, s, wiring, seed, _ptr(Y), ldy, flags, _ptr(workspace),
        _nbytes(workspace, workspace_bytes), _stream(stream)))


def sk_blockperm_workspace_size(m, n, d, M, kappa, s, wiring):
    out = ctypes.c_size_t(0)
    _check("sk_blockperm_workspace_size", load().sk_blockperm_workspace_size(
        m, n, d, M, kappa, s, wiring, ctypes.byref(out)))
    return out.value


BLOCKPERM_PLAN_FIELDS = ("kernel", "Q", "rows_per_slice", "ws_bytes", "a", "b", "ainv",
                         "rows_per_wave", "groups", "slices")


def sk_blockperm_plan_describe(m, n, d, M, kappa, s, wiring, seed, num_cu, max_lds):
    out = (ctypes.c_int64 * len(BLOCKPERM_PLAN_FIELDS))()
    _check("sk_blockperm_plan_describe", load().sk_blockperm_plan_describe(
        m, n, d, M, kappa, s, wiring, seed, num_cu, max_lds, out))
    return dict(zip(BLOCKPERM_PLAN_FIELDS, list(out)))


def sk_apply_lowp(A, m, n, lda, row_idx, val, zeta, B, d, ldb, format, convert, sr_seed=0,
                  row_offset=0, flags=0, workspace=None, workspace_bytes=0, stream=None):
    _check("sk_apply_lowp", load().sk_apply_lowp(
        _ptr(A), m, n, lda, _ptr(row_idx), _ptr(val), zeta, _ptr(B), d, ldb, format, convert,
        sr_seed, row_offset, flags, _ptr(workspace), _nbytes(workspace, workspace_bytes),
        _stream(stream)))


def sk_sketch_f32(seed, row_offset, A, m, n, lda, d, zeta, B, ldb, flags=0, workspace=None,
                  workspace_bytes=0, stream=None):
    _check("sk_sketch_f32", load().sk_sketch_f32(
        seed, row_offset, _ptr(A), m, n, lda, d, zeta, _ptr(B), ldb, flags, _ptr(workspace),
        _nbytes(workspace, workspace_bytes), _stream(stream)))


def sk_sketch_f16acc(seed, row_offset, A, m, n, lda, d, zeta, B, ldb, flags=0, workspace=None,
                     workspace_bytes=0, stream=None):
    _check("sk_sketch_f16acc", load().sk_sketch_f16acc(
        seed, row_offset, _ptr(A), m, n, lda, d, zeta, _ptr(B), ldb, flags, _ptr(workspace),
        _nbytes(workspace, workspace_bytes), _stream(stream)))


def sk_sketch_f16acc_noalloc(seed, row_offset, A, m, n, lda, d, zeta, B, ldb, flags=0,
                             stream=None):
    _check("sk_sketch_f16acc_noalloc", load().sk_sketch_f16acc_noalloc(
        seed, row_offset, _ptr(A), m, n, lda, d, zeta, _ptr(B), ldb, flags, _stream(stream)))


def sk_sketch_workspace_size(precision, m, n, d, zeta):
    """Bytes of workspace an sk_sketch_* call needs (0 for m = 0)."""
    out = ctypes.c_size_t(0)
    _check("sk_sketch_workspace_size", load().sk_sketch_workspace_size(
        precision, m, n, d, zeta, ctypes.byref(out)))
    return out.value


FUSED_PLAN_FIELDS = ("fused", "rows_per_wave", "groups", "slices", "rows_per_chunk", "chunks",
                     "grid", "ws_bytes", "words", "stage_rows", "per_cu")


SKETCH_PLAN_FIELDS = ("kernel", "words", "lanes_per_row", "threads", "row_words", "stage_rows",
                      "cap", "load_words", "rows_per_chunk", "chunks", "grid", "ws_bytes",
                      "lds_bytes", "per_cu", "mask_stride", "list_stride", "barriers",
                      "load_slots")


def sk_sketch_plan_describe(precision, m, n, lda, a_align, d, zeta, num_cu, max_lds):
    """The complete sketch's launch plan as a dict (host computation)."""
    out = (ctypes.c_int64 * len(SKETCH_PLAN_FIELDS))()
    _check("sk_sketch_plan_describe", load().sk_sketch_plan_describe(
        precision, m, n, lda, int(a_align), d, zeta, num_cu, max_lds, out))
    return dict(zip(SKETCH_PLAN_FIELDS, list(out)))


def sk_fused_plan_describe(precision, m, n, lda, a_align, d, zeta, num_cu, max_lds):
    """The fused kernel's launch plan as a dict (host computation); a_align
    is the alignment of A's base address in bytes."""
    out = (ctypes.c_int64 * len(FUSED_PLAN_FIELDS))()
    _check("sk_fused_plan_describe", load().sk_fused_plan_describe(
        precision, m, n, lda, int(a_align), d, zeta, num_cu, max_lds, out))
    return dict(zip(FUSED_PLAN_FIELDS, list(out)))


# ---- tensor helpers ------------------------------------------------------

def _need_device(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() == 2 and t.stride(1) != 1:
        raise ValueError(f"{name} must be row-major with unit column stride")


def meta(seed, m, d, zeta, row_offset=0, device=None, stream=None):
    """(row_idx int32[m*zeta], val float32[m*zeta]) on the device."""
    import torch
    device = device or torch.device("cuda", torch.cuda.current_device())
    row_idx = torch.empty(m * zeta, dtype=torch.int32, device=device)
    val = torch.empty(m * zeta, dtype=torch.float32, device=device)
    sk_meta_generate(seed, row_offset, m, d, zeta, row_idx, val, stream)
    _keep(stream, row_idx, val)
    return row_idx, val


def workspace(A, d, zeta, precision="f16acc", flags=0):
    """A device byte tensor large enough for apply()'s store-and-reduce flush
    (None when the chosen variant needs none)."""
    import torch
    prec = SK_PRECISION_F16ACC if precision == "f16acc" else SK_PRECISION_F32
    nbytes = sk_apply_workspace_size(prec, A.shape[0], A.shape[1], d, zeta, flags)
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=A.device)


def apply(A, row_idx, val, zeta, d, precision="f16acc", out=None, flags=0, ws=True, stream=None):
    """B = S A from metadata; precision "f32" (float32 B) or "f16acc" (float16 B).

    ws=True allocates the workspace the chosen variant needs (the LDS
    variant's store-and-reduce flush, or the register variant's partials)
    and calls sk_apply_*_ws; ws=None calls sk_apply_f32 / sk_apply_f16acc,
    which take no workspace (the LDS variant flushes with global atomics);
    a byte tensor is used as the workspace."""
    import torch
    _need_device(A, torch.float32, "A")
    m, n = A.shape
    dt = torch.float16 if precision == "f16acc" else torch.float32
    if out is None:
        out = torch.empty((d, n), dtype=dt, device=A.device)
    _need_device(out, dt, "out")
    if m:
        _need_device(row_idx, torch.int32, "row_idx")
        _need_device(val, torch.float32, "val")
        if row_idx.numel() < m * zeta or val.numel() < m * zeta:
            raise ValueError("metadata shorter than m*zeta")
    fresh = None
    if ws is True:
        ws = fresh = workspace(A, d, zeta, precision, flags)
    lda = A.stride(0) if m else n
    ri, v = (row_idx, val) if m else (None, None)
    if ws is None:
        fn = sk_apply_f16acc if precision == "f16acc" else sk_apply_f32
        fn(A, m, n, lda, ri, v, zeta, out, d, out.stride(0), flags, stream)
    else:
        fn = sk_apply_f16acc_ws if precision == "f16acc" else sk_apply_f32_ws
        fn(A, m, n, lda, ri, v, zeta, out, d, out.stride(0), flags, ws, 0, stream)
    _keep(stream, out, fresh)
    return out


def sketch(A, d, zeta, seed, precision="f16acc", flags=0, ws=True, stream=None):
    """Complete sketch: metadata generation, output initialization and application."""
    row_idx, val = meta(seed, A.shape[0], d, zeta, device=A.device, stream=stream)
    return apply(A, row_idx, val, zeta, d, precision, flags=flags, ws=ws, stream=stream)


def apply_lowp(A, row_idx, val, zeta, d, fmt="f16", conv="rn", sr_seed=0, row_offset=0, out=None,
               flags=0, stream=None):
    """Reduced-precision sketch from metadata: fmt "f16" (float16 B) with
    conv "rn" or "sr", or fmt "bf16" (bfloat16 B) with conv "rn".  flags
    with SK_VARIANT_REG: the two-level design (a workspace is allocated);
    else the flat atomic design."""
    import torch
    _need_device(A, torch.float32, "A")
    m, n = A.shape
    dt = torch.float16 if fmt == "f16" else torch.bfloat16
    if out is None:
        out = torch.empty((d, n), dtype=dt, device=A.device)
    _need_device(out, dt, "out")
    if m:
        _need_device(row_idx, torch.int32, "row_idx")
        _need_device(val, torch.float32, "val")
        if row_idx.numel() < m * zeta or val.numel() < m * zeta:
            raise ValueError("metadata shorter than m*zeta")
    f = SK_FORMAT_F16 if fmt == "f16" else SK_FORMAT_BF16
    c = SK_CONVERT_RN if conv == "rn" else SK_CONVERT_SR
    ws = None
    if flags & SK_VARIANT_REG:
        nb = sk_apply_workspace_size(SK_PRECISION_LOWP, m, n, d, zeta, flags)
        if nb:
            ws = torch.empty(nb, dtype=torch.uint8, device=A.device)
    sk_apply_lowp(A, m, n, A.stride(0) if m else n, row_idx if m else None, val if m else None,
                  zeta, out, d, out.stride(0), f, c, sr_seed, row_offset, flags, ws, 0, stream)
    _keep(stream, out, ws)
    return out


def sketch_workspace(A, d, zeta, precision="f16acc"):
    """A device byte tensor large enough for sketch_fused() (None for m = 0)."""
    import torch
    prec = SK_PRECISION_F16ACC if precision == "f16acc" else SK_PRECISION_F32
    nbytes = sk_sketch_workspace_size(prec, A.shape[0], A.shape[1], d, zeta)
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=A.device)


def sketch_fused(A, d, zeta, seed, precision="f16acc", row_offset=0, out=None, flags=0, ws=None,
                 stream=None):
    """Complete sketch in one call, metadata drawn on the fly (same S as
    meta(seed, ..., row_offset) + apply).  ws: a byte tensor of at least
    sk_sketch_workspace_size bytes, or None to allocate one."""
    import torch
    _need_device(A, torch.float32, "A")
    m, n = A.shape
    dt = torch.float16 if precision == "f16acc" else torch.float32
    if out is None:
        out = torch.empty((d, n), dtype=dt, device=A.device)
    _need_device(out, dt, "out")
    fresh = None
    if ws is None and m:
        ws = fresh = sketch_workspace(A, d, zeta, precision)
    fn = sk_sketch_f16acc if precision == "f16acc" else sk_sketch_f32
    fn(seed, row_offset, A, m, n, A.stride(0) if m else n, d, zeta, out, out.stride(0), flags,
       ws, 0, stream)
    _keep(stream, out, fresh)
    return out


def blockperm(A, d, M, kappa, seed, s=1, out=None, flags=0, wiring="shift", ws=None,
              stream=None):
    """Y = S A for S ~ BlockPerm-SJLT (float32).  wiring "shift" or "affine";
    ws: a byte tensor for the general kernel's partials (allocated when
    needed and not given)."""
    import torch
    _need_device(A, torch.float32, "A")
    m, n = A.shape
    if out is None:
        out = torch.empty((d, n), dtype=torch.float32, device=A.device)
    _need_device(out, torch.float32, "out")
    w = SK_WIRING_SHIFT if wiring == "shift" else SK_WIRING_AFFINE
    fresh = None
    if ws is None:
        nbytes = sk_blockperm_workspace_size(m, n, d, M, kappa, s, w)
        if nbytes:
            ws = fresh = torch.empty(nbytes, dtype=torch.uint8, device=A.device)
    sk_apply_blockperm_ex(A, m, n, A.stride(0), d, M, kappa, s, w, seed, out, out.stride(0),
                          flags, ws, 0, stream)
    _keep(stream, out, fresh)
    return out
