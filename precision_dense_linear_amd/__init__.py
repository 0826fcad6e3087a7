"""MI355X (gfx950) scaled FP8 GEMM: thin Python binding over libfp8gemm.so.

Every function here only marshals arguments: it takes torch tensors on a
ROCm device, allocates missing outputs with torch (device memory is the only
thing torch provides), and calls the C ABI of include/fp8gemm.h with raw
device pointers and torch's current HIP stream.  All arithmetic runs in the
library's HIP kernels; if the library is missing the import fails.

Entry points (same names as the C ABI):
    fp8_quantize(x)                          -> (q, scale, amax)
    fp8_quantize_e5m2(x)                     -> (q, scale, amax)
    fp8_quantize_blocked(x)                  -> (q, tile_scales)
    fp8_quantize_blocked64(x)                -> (q, tile_scales)
    fp8_quantize_blocked_e8m0(x, k_major)    -> (q, tile_exps uint8)
    fp8_quantize_grouped(x, offsets)         -> (q, scales, amax)
    fp8_quantize_grouped_e5m2(x, offsets)    -> (q, scales, amax)
    fp8_gemm(A, B, scale_a, scale_b, out_dtype)   (fp8_gemm_ws with workspace=)
    fp8_gemm_noalloc(A, B, scale_a, scale_b, out_dtype)
    gemm_workspace(device)                   -> zeroed split-K workspace (torch.uint8)
    fp8_gemm_blockscaled(A, B, s_a, s_b, out_dtype, block=32 | 64)
    fp8_gemm_blockscaled_e8m0(A, B, e_a, e_b, out_dtype)
    fp8_quantize_2of4(w)                     -> (vals, idx, scale, amax)
    fp8_gemm_sparse24(A, vals, idx, scale_a, scale_b, out_dtype)
    fp8_grouped_gemm(A, B, offsets, scale_a, scale_b, out_dtype)
    fp8_attention(Q, K, V, scale_q, scale_k, scale_v, softmax_scale, causal, out_dtype)
FP8 codes are passed as torch.uint8 (E4M3 unless a_fmt / b_fmt say "e5m2"),
torch.float8_e4m3fn or torch.float8_e5m2 tensors; out_dtype is
torch.float32, torch.bfloat16 or torch.float16.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8gemm.so")

FP8_OK, FP8_ERR_INVALID_ARG, FP8_ERR_UNSUPPORTED_SHAPE, FP8_ERR_HIP = 0, 1, 2, 3
FP8_OUT_F32, FP8_OUT_BF16, FP8_OUT_F16 = 0, 1, 2
FP8_ACC_FAST = 0x100  # native FP8 matrix-core accumulation (see include/fp8gemm.h)
FP8_A_E5M2, FP8_B_E5M2 = 0x200, 0x400  # operand formats (default E4M3)
FP8_BLOCK64 = 0x800  # 64x64 scale tiles for the block-scaled GEMM
FP8_GEMM_WS_TILE_BYTES = 8196  # split-K workspace bytes per split tile (32 x 64 FP32 partials + counter)
FP8_GEMM_WORKSPACE_BYTES = 512 * FP8_GEMM_WS_TILE_BYTES

SYMBOLS = ("fp8_quantize", "fp8_quantize_e5m2", "fp8_quantize_blocked", "fp8_quantize_blocked64",
           "fp8_quantize_blocked_e8m0", "fp8_gemm_blockscaled_e8m0", "fp8_quantize_2of4",
           "fp8_gemm_sparse24", "fp8_quantize_grouped",
           "fp8_quantize_grouped_e5m2", "fp8_gemm", "fp8_gemm_ws", "fp8_gemm_noalloc", "fp8_gemm_blockscaled",
           "fp8_grouped_gemm", "fp8_attention", "fp8_status_string", "fp8_last_error")


class FP8Error(RuntimeError):
    def __init__(self, func: str, status: int, message: str):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (func, status_name(status), message))


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libfp8gemm.so is not built (%s); run __graft_entry__.build() or "
                          "python -m precision_dense_linear_amd._build" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    st = ctypes.c_int
    L.fp8_quantize.argtypes = [P, i64, P, P, P, P]
    L.fp8_quantize_e5m2.argtypes = [P, i64, P, P, P, P]
    L.fp8_quantize_blocked.argtypes = [P, i64, i64, P, P, P]
    L.fp8_quantize_blocked64.argtypes = [P, i64, i64, P, P, P]
    L.fp8_quantize_blocked_e8m0.argtypes = [P, i64, i64, i32, P, P, P]
    L.fp8_gemm_blockscaled_e8m0.argtypes = [P, P, P, P, P, i64, i64, i64, i32, P]
    L.fp8_quantize_2of4.argtypes = [P, i64, i64, P, P, P, P, P]
    L.fp8_gemm_sparse24.argtypes = [P, P, P, P, P, P, i64, i64, i64, i32, P]
    L.fp8_quantize_grouped.argtypes = [P, i64, i64, P, i32, P, P, P, P]
    L.fp8_quantize_grouped_e5m2.argtypes = [P, i64, i64, P, i32, P, P, P, P]
    L.fp8_gemm.argtypes = [P, P, P, P, P, i64, i64, i64, i32, P]
    L.fp8_gemm_ws.argtypes = [P, P, P, P, P, i64, i64, i64, i32, P, i64, P]
    L.fp8_gemm_noalloc.argtypes = [P, P, P, P, P, i64, i64, i64, i32, P]
    L.fp8_gemm_blockscaled.argtypes = [P, P, P, P, P, i64, i64, i64, i32, P]
    L.fp8_grouped_gemm.argtypes = [P, P, P, i32, P, P, P, i64, i64, i64, i32, P]
    L.fp8_attention.argtypes = [P, P, P, P, P, P, P, i64, i64, i64, i64, ctypes.c_float, i32, i32, P]
    for f in ("fp8_quantize", "fp8_quantize_e5m2", "fp8_quantize_blocked", "fp8_quantize_blocked64",
              "fp8_quantize_blocked_e8m0", "fp8_gemm_blockscaled_e8m0", "fp8_quantize_2of4",
           "fp8_gemm_sparse24", "fp8_quantize_grouped",
              "fp8_quantize_grouped_e5m2", "fp8_gemm", "fp8_gemm_ws", "fp8_gemm_noalloc", "fp8_gemm_blockscaled",
              "fp8_grouped_gemm", "fp8_attention"):
        getattr(L, f).restype = st
    L.fp8_status_string.restype = ctypes.c_char_p
    L.fp8_status_string.argtypes = [i32]
    L.fp8_last_error.restype = ctypes.c_char_p
    L.fp8_last_error.argtypes = []
    return L


lib = _load()


def status_name(status: int) -> str:
    return lib.fp8_status_string(status).decode()


def _check(func: str, status: int):
    if status != FP8_OK:
        raise FP8Error(func, status, lib.fp8_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _codes(t: torch.Tensor) -> torch.Tensor:
    if t.dtype in (torch.float8_e4m3fn, torch.float8_e5m2):
        return t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise TypeError("FP8 operands must be torch.uint8, torch.float8_e4m3fn or torch.float8_e5m2, got %s" % t.dtype)
    return t


def _fmt_flag(t: torch.Tensor, fmt, flag: int) -> int:
    """The operand-format flag of one operand: from an FP8 dtype, else from
    fmt ("e4m3" / "e5m2", default E4M3)."""
    from_dtype = {torch.float8_e4m3fn: "e4m3", torch.float8_e5m2: "e5m2"}.get(t.dtype)
    if fmt is None:
        fmt = from_dtype or "e4m3"
    _require(fmt in ("e4m3", "e5m2"), "format must be 'e4m3' or 'e5m2', got %r" % (fmt,))
    _require(from_dtype in (None, fmt), "a %s tensor passed with format %r" % (t.dtype, fmt))
    return flag if fmt == "e5m2" else 0


_SAME_DEVICE = contextlib.nullcontext()


def _on(dev: torch.device):
    """The device guard for a call on dev: none when dev is already current
    (entering torch.cuda.device costs a few microseconds per call)."""
    return _SAME_DEVICE if dev.index == torch.cuda.current_device() else torch.cuda.device(dev)


def _stream(dev: torch.device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _out_code(out_dtype) -> int:
    if out_dtype in (torch.float32, "f32", "fp32", FP8_OUT_F32):
        return FP8_OUT_F32
    if out_dtype in (torch.bfloat16, "bf16", FP8_OUT_BF16):
        return FP8_OUT_BF16
    if out_dtype in (torch.float16, "f16", "fp16", FP8_OUT_F16):
        return FP8_OUT_F16
    raise ValueError("out_dtype must be torch.float32, torch.bfloat16 or torch.float16")


def _require(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


_CODES = (torch.uint8, torch.float8_e4m3fn, torch.float8_e5m2)
_F32 = (torch.float32,)
_OUT_DTYPE = {FP8_OUT_F32: torch.float32, FP8_OUT_BF16: torch.bfloat16, FP8_OUT_F16: torch.float16}


def _arg(t, name: str, dev, dtypes, numel=None, at_least=False):
    """Checks a tensor before its pointer goes to the library (which can check
    sizes but not pointers): a contiguous tensor on the operands' GPU, of one
    of dtypes, with numel elements (at least numel with at_least)."""
    _require(isinstance(t, torch.Tensor), "%s must be a torch tensor" % name)
    _require(t.is_cuda, "%s must be a GPU tensor" % name)
    _require(t.device == dev, "%s is on %s, the operands on %s" % (name, t.device, dev))
    _require(t.dtype in dtypes, "%s must be %s, got %s" % (name, " or ".join(map(str, dtypes)), t.dtype))
    _require(t.is_contiguous(), "%s must be contiguous" % name)
    if numel is not None:
        n = t.numel()
        _require(n >= numel if at_least else n == numel, "%s has %d elements where %s%d are needed" % (
            name, n, "at least " if at_least else "", numel))
    return t


def _out_arg(C, name: str, dev, code: int, numel: int):
    return _arg(C, name, dev, (_OUT_DTYPE[code],), numel)


def _quantize(func: str, x: torch.Tensor, q, scale, amax, stream):
    _require(x.is_cuda and x.dtype == torch.float32 and x.is_contiguous(), "x must be a contiguous float32 GPU tensor")
    dev = x.device
    q = torch.empty(x.shape, dtype=torch.uint8, device=dev) if q is None else _arg(q, "q", dev, _CODES, x.numel())
    scale = torch.empty(1, dtype=torch.float32, device=dev) if scale is None else _arg(scale, "scale", dev, _F32, 1, True)
    amax = torch.empty(1, dtype=torch.float32, device=dev) if amax is None else _arg(amax, "amax", dev, _F32, 1, True)
    with _on(dev):
        _check(func, getattr(lib, func)(_ptr(x), x.numel(), _ptr(q), _ptr(scale), _ptr(amax), _stream(dev, stream)))
    return q, scale, amax


def fp8_quantize(x: torch.Tensor, q=None, scale=None, amax=None, stream=None):
    """Per-tensor E4M3 quantization; returns (q uint8, scale float32[1], amax float32[1])."""
    return _quantize("fp8_quantize", x, q, scale, amax, stream)


def fp8_quantize_e5m2(x: torch.Tensor, q=None, scale=None, amax=None, stream=None):
    """Per-tensor E5M2 quantization (scale = amax / 57344); returns (q uint8, scale, amax)."""
    return _quantize("fp8_quantize_e5m2", x, q, scale, amax, stream)


def _quantize_blocked(func: str, T: int, x, q, tile_scales, stream):
    _require(x.is_cuda and x.dtype == torch.float32 and x.is_contiguous() and x.dim() == 2,
             "x must be a contiguous 2-D float32 GPU tensor")
    rows, cols = x.shape
    dev = x.device
    q = torch.empty(x.shape, dtype=torch.uint8, device=dev) if q is None else _arg(q, "q", dev, _CODES, x.numel())
    if tile_scales is None:
        tile_scales = torch.empty((rows // T, cols // T), dtype=torch.float32, device=dev)
    else:
        _arg(tile_scales, "tile_scales", dev, _F32, (rows // T) * (cols // T), True)
    with _on(dev):
        _check(func, getattr(lib, func)(_ptr(x), rows, cols, _ptr(q), _ptr(tile_scales), _stream(dev, stream)))
    return q, tile_scales


def fp8_quantize_blocked(x: torch.Tensor, q=None, tile_scales=None, stream=None):
    """32x32-tile E4M3 quantization of a 2-D tensor; returns (q, tile_scales[rows/32, cols/32])."""
    return _quantize_blocked("fp8_quantize_blocked", 32, x, q, tile_scales, stream)


def fp8_quantize_blocked64(x: torch.Tensor, q=None, tile_scales=None, stream=None):
    """64x64-tile E4M3 quantization of a 2-D tensor; returns (q, tile_scales[rows/64, cols/64])."""
    return _quantize_blocked("fp8_quantize_blocked64", 64, x, q, tile_scales, stream)


def fp8_quantize_blocked_e8m0(x: torch.Tensor, k_major=False, q=None, tile_exps=None, stream=None):
    """32x32-tile E4M3 quantization with power-of-two scales; returns (q, tile_exps uint8), tile_exps
    holding e + 127 for the tile scale 2^e, shaped [rows/32, pitch(cols/32)], or [cols/32, pitch(rows/32)]
    with k_major (the layout fp8_gemm_blockscaled_e8m0 takes for A); pitch(n) rounds n up to a multiple
    of 4, the padding bytes hold 127."""
    _require(x.is_cuda and x.dtype == torch.float32 and x.is_contiguous() and x.dim() == 2,
             "x must be a contiguous 2-D float32 GPU tensor")
    rows, cols = x.shape
    dev = x.device
    q = torch.empty(x.shape, dtype=torch.uint8, device=dev) if q is None else _arg(q, "q", dev, _CODES, x.numel())
    pitch = lambda n: (n + 3) // 4 * 4
    shape = (cols // 32, pitch(rows // 32)) if k_major else (rows // 32, pitch(cols // 32))
    if tile_exps is None:
        tile_exps = torch.empty(shape, dtype=torch.uint8, device=dev)
    else:
        _arg(tile_exps, "tile_exps", dev, (torch.uint8,), shape[0] * shape[1], True)
    with _on(dev):
        _check("fp8_quantize_blocked_e8m0", lib.fp8_quantize_blocked_e8m0(_ptr(x), rows, cols, int(bool(k_major)),
                                                                          _ptr(q), _ptr(tile_exps),
                                                                          _stream(dev, stream)))
    return q, tile_exps


def _quantize_grouped(func: str, x, offsets, q, scales, amax, stream):
    _require(x.is_cuda and x.dtype == torch.float32 and x.is_contiguous() and x.dim() == 2,
             "x must be a contiguous 2-D float32 GPU tensor")
    rows, cols = x.shape
    dev = x.device
    _arg(offsets, "offsets", dev, (torch.int32,))
    G = offsets.numel() - 1
    q = torch.zeros(x.shape, dtype=torch.uint8, device=dev) if q is None else _arg(q, "q", dev, _CODES, x.numel())
    scales = torch.empty(G, dtype=torch.float32, device=dev) if scales is None else _arg(scales, "scales", dev, _F32,
                                                                                          G, True)
    amax = torch.empty(G, dtype=torch.float32, device=dev) if amax is None else _arg(amax, "amax", dev, _F32, G, True)
    with _on(dev):
        _check(func, getattr(lib, func)(_ptr(x), rows, cols, _ptr(offsets), G, _ptr(q), _ptr(scales), _ptr(amax),
                                        _stream(dev, stream)))
    return q, scales, amax


def fp8_quantize_grouped(x: torch.Tensor, offsets: torch.Tensor, q=None, scales=None, amax=None, stream=None):
    """Row-group E4M3 quantization (group g = rows offsets[g]..offsets[g+1]); returns (q, scales, amax)."""
    return _quantize_grouped("fp8_quantize_grouped", x, offsets, q, scales, amax, stream)


def fp8_quantize_grouped_e5m2(x: torch.Tensor, offsets: torch.Tensor, q=None, scales=None, amax=None, stream=None):
    """Row-group E5M2 quantization (scales = amax / 57344); returns (q, scales, amax)."""
    return _quantize_grouped("fp8_quantize_grouped_e5m2", x, offsets, q, scales, amax, stream)


def _out_tensor(C, shape, code, dev, name="C"):
    if C is not None:
        n = 1
        for d in shape:
            n *= d
        return _out_arg(C, name, dev, code, n)
    return torch.empty(shape, dtype=_OUT_DTYPE[code], device=dev)


def _operands(A, B, a_dims=2, b_dims=2):
    """The two FP8 operands as contiguous GPU code tensors on one device."""
    _require(isinstance(A, torch.Tensor) and A.is_cuda, "A must be a GPU tensor")
    dev = A.device
    _arg(A, "A", dev, _CODES)
    _arg(B, "B", dev, _CODES)
    _require(A.dim() == a_dims and B.dim() == b_dims, "A must have %d dimensions and B %d" % (a_dims, b_dims))
    return dev


def _scales(dev, n, **named):
    for name, t in named.items():
        _arg(t, name, dev, _F32, n, True)


def gemm_workspace(device=None, nbytes: int = FP8_GEMM_WORKSPACE_BYTES) -> torch.Tensor:
    """A zero-filled split-K workspace for fp8_gemm(..., workspace=...)."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    return torch.zeros(nbytes, dtype=torch.uint8, device=dev)


def fp8_gemm(A, B, scale_a, scale_b, out_dtype=torch.bfloat16, C=None, stream=None, fast=False, a_fmt=None,
             b_fmt=None, workspace=None):
    """C = scale_a*scale_b * A @ B with FP8 A (M x K) and B (K x N), FP32 accumulation.

    fast=True selects the native FP8 matrix-core accumulation (FP8_ACC_FAST);
    a_fmt / b_fmt ("e4m3" or "e5m2") give the operand formats of uint8 codes.
    workspace (a zeroed uint8 GPU tensor, e.g. gemm_workspace()) calls
    fp8_gemm_ws, which may split K across workgroups for outputs too small to
    fill the GPU; calls sharing a workspace must be ordered (one stream)."""
    flags = _fmt_flag(A, a_fmt, FP8_A_E5M2) | _fmt_flag(B, b_fmt, FP8_B_E5M2) | (FP8_ACC_FAST if fast else 0)
    dev = _operands(A, B)
    A, B = _codes(A), _codes(B)
    M, K = A.shape
    N = B.shape[1]
    _require(B.shape[0] == K, "A is %s but B is %s" % (tuple(A.shape), tuple(B.shape)))
    _scales(dev, 1, scale_a=scale_a, scale_b=scale_b)
    code = _out_code(out_dtype)
    C = _out_tensor(C, (M, N), code, A.device)
    with _on(A.device):
        if workspace is None:
            _check("fp8_gemm", lib.fp8_gemm(_ptr(A), _ptr(B), _ptr(scale_a), _ptr(scale_b), _ptr(C), M, N, K,
                                            code | flags, _stream(A.device, stream)))
        else:
            _arg(workspace, "workspace", dev, (getattr(workspace, "dtype", None),))
            _check("fp8_gemm_ws", lib.fp8_gemm_ws(_ptr(A), _ptr(B), _ptr(scale_a), _ptr(scale_b), _ptr(C), M, N,
                                                  K, code | flags, _ptr(workspace),
                                                  workspace.numel() * workspace.element_size(),
                                                  _stream(A.device, stream)))
    return C


def fp8_gemm_noalloc(A, B, scale_a, scale_b, out_dtype=torch.bfloat16, C=None, stream=None, fast=False, a_fmt=None,
                     b_fmt=None):
    """fp8_gemm with K split across workgroups where that fills the GPU, the
    partial sums in the library's own static device array (no allocation by
    the library; C is allocated here only when not given).  Calls on one GPU
    must not overlap in time."""
    flags = _fmt_flag(A, a_fmt, FP8_A_E5M2) | _fmt_flag(B, b_fmt, FP8_B_E5M2) | (FP8_ACC_FAST if fast else 0)
    dev = _operands(A, B)
    A, B = _codes(A), _codes(B)
    M, K = A.shape
    N = B.shape[1]
    _require(B.shape[0] == K, "A is %s but B is %s" % (tuple(A.shape), tuple(B.shape)))
    _scales(dev, 1, scale_a=scale_a, scale_b=scale_b)
    code = _out_code(out_dtype)
    C = _out_tensor(C, (M, N), code, A.device)
    with _on(A.device):
        _check("fp8_gemm_noalloc", lib.fp8_gemm_noalloc(_ptr(A), _ptr(B), _ptr(scale_a), _ptr(scale_b), _ptr(C), M, N,
                                                        K, code | flags, _stream(A.device, stream)))
    return C


def fp8_gemm_blockscaled(A, B, s_a, s_b, out_dtype=torch.bfloat16, C=None, stream=None, block=32):
    """C = sum over block-deep K blocks of s_a*s_b * (A_kb @ B_kb), block x block tile scales
    (block 32 or 64; E4M3 operands)."""
    _require(block in (32, 64), "block must be 32 or 64")
    _require(_fmt_flag(A, None, 1) == 0 and _fmt_flag(B, None, 1) == 0, "the block-scaled GEMM takes E4M3 operands")
    dev = _operands(A, B)
    A, B = _codes(A), _codes(B)
    M, K = A.shape
    N = B.shape[1]
    _require(B.shape[0] == K, "A is %s but B is %s" % (tuple(A.shape), tuple(B.shape)))
    _arg(s_a, "s_a", dev, _F32, (M // block) * (K // block), True)
    _arg(s_b, "s_b", dev, _F32, (K // block) * (N // block), True)
    code = _out_code(out_dtype)
    C = _out_tensor(C, (M, N), code, A.device)
    with _on(A.device):
        _check("fp8_gemm_blockscaled", lib.fp8_gemm_blockscaled(_ptr(A), _ptr(B), _ptr(s_a), _ptr(s_b), _ptr(C),
                                                                M, N, K, code | (FP8_BLOCK64 if block == 64 else 0),
                                                                _stream(A.device, stream)))
    return C


def fp8_gemm_blockscaled_e8m0(A, B, e_a, e_b, out_dtype=torch.bfloat16, C=None, stream=None):
    """C = sum over 32-deep K blocks of 2^(e_a-127) * 2^(e_b-127) * (A_kb @ B_kb) on the FP8 matrix cores
    (32x32 tile exponents, e_a [K/32, pitch(M/32)] and e_b [K/32, pitch(N/32)]; E4M3 operands)."""
    _require(_fmt_flag(A, None, 1) == 0 and _fmt_flag(B, None, 1) == 0, "E4M3 operands only")
    dev = _operands(A, B)
    A, B = _codes(A), _codes(B)
    M, K = A.shape
    N = B.shape[1]
    _require(B.shape[0] == K, "A is %s but B is %s" % (tuple(A.shape), tuple(B.shape)))
    pitch = lambda n: (n + 3) // 4 * 4
    _arg(e_a, "e_a", dev, (torch.uint8,), (K // 32) * pitch(M // 32), True)
    _arg(e_b, "e_b", dev, (torch.uint8,), (K // 32) * pitch(N // 32), True)
    code = _out_code(out_dtype)
    C = _out_tensor(C, (M, N), code, A.device)
    with _on(A.device):
        _check("fp8_gemm_blockscaled_e8m0", lib.fp8_gemm_blockscaled_e8m0(_ptr(A), _ptr(B), _ptr(e_a), _ptr(e_b),
                                                                          _ptr(C), M, N, K, code,
                                                                          _stream(A.device, stream)))
    return C


def fp8_quantize_2of4(w: torch.Tensor, vals=None, idx=None, scale=None, amax=None, stream=None):
    """2:4-prune a K x N float32 weight matrix along K, quantize it per tensor (E4M3) and compress it;
    returns (vals uint8[K/2, N], idx int32[K/32, N] position words, scale float32[1], amax float32[1])."""
    _require(w.is_cuda and w.dtype == torch.float32 and w.is_contiguous() and w.dim() == 2,
             "w must be a contiguous 2-D float32 GPU tensor")
    K, N = w.shape
    dev = w.device
    vals = (torch.empty((K // 2, N), dtype=torch.uint8, device=dev) if vals is None
            else _arg(vals, "vals", dev, _CODES, (K // 2) * N))
    idx = (torch.empty((K // 32, N), dtype=torch.int32, device=dev) if idx is None
           else _arg(idx, "idx", dev, (torch.int32,), (K // 32) * N))
    scale = torch.empty(1, dtype=torch.float32, device=dev) if scale is None else _arg(scale, "scale", dev, _F32, 1, True)
    amax = torch.empty(1, dtype=torch.float32, device=dev) if amax is None else _arg(amax, "amax", dev, _F32, 1, True)
    with _on(dev):
        _check("fp8_quantize_2of4", lib.fp8_quantize_2of4(_ptr(w), K, N, _ptr(vals), _ptr(idx), _ptr(scale),
                                                          _ptr(amax), _stream(dev, stream)))
    return vals, idx, scale, amax


def fp8_gemm_sparse24(A, vals, idx, scale_a, scale_b, out_dtype=torch.bfloat16, C=None, stream=None):
    """C = scale_a*scale_b * A @ B with E4M3 A (M x K) and a 2:4-sparse B given compressed
    (vals [K/2, N], idx [K/32, N]) on the sparse FP8 matrix cores."""
    _require(_fmt_flag(A, None, 1) == 0, "E4M3 operands only")
    dev = _operands(A, vals)
    _arg(idx, "idx", dev, (torch.int32,))
    A = _codes(A)
    vals = vals.view(torch.uint8) if vals.dtype == torch.float8_e4m3fn else vals
    M, K = A.shape
    N = vals.shape[1]
    _require(vals.shape[0] * 2 == K and tuple(idx.shape) == (K // 32, N), "A is %s but vals %s, idx %s" % (
        tuple(A.shape), tuple(vals.shape), tuple(idx.shape)))
    _scales(dev, 1, scale_a=scale_a, scale_b=scale_b)
    code = _out_code(out_dtype)
    C = _out_tensor(C, (M, N), code, A.device)
    with _on(A.device):
        _check("fp8_gemm_sparse24", lib.fp8_gemm_sparse24(_ptr(A), _ptr(vals), _ptr(idx), _ptr(scale_a),
                                                          _ptr(scale_b), _ptr(C), M, N, K, code,
                                                          _stream(A.device, stream)))
    return C


def fp8_grouped_gemm(A, B, offsets, scale_a, scale_b, out_dtype=torch.bfloat16, C=None, stream=None, fast=False,
                     a_fmt=None, b_fmt=None):
    """MoE grouped GEMM: rows offsets[e]..offsets[e+1] of A times B[e], scaled by scale_a[e]*scale_b[e]."""
    flags = _fmt_flag(A, a_fmt, FP8_A_E5M2) | _fmt_flag(B, b_fmt, FP8_B_E5M2) | (FP8_ACC_FAST if fast else 0)
    dev = _operands(A, B, 2, 3)
    A, B = _codes(A), _codes(B)
    T, K = A.shape
    E, K2, N = B.shape
    _arg(offsets, "offsets", dev, (torch.int32,))
    _require(K2 == K and offsets.numel() == E + 1, "shape mismatch")
    _scales(dev, E, scale_a=scale_a, scale_b=scale_b)
    code = _out_code(out_dtype)
    C = _out_tensor(C, (T, N), code, A.device)
    with _on(A.device):
        _check("fp8_grouped_gemm", lib.fp8_grouped_gemm(_ptr(A), _ptr(B), _ptr(offsets), E, _ptr(scale_a),
                                                        _ptr(scale_b), _ptr(C), T, N, K, code | flags,
                                                        _stream(A.device, stream)))
    return C


def fp8_attention(Q, K, V, scale_q, scale_k, scale_v, softmax_scale=None, causal=False, out_dtype=torch.bfloat16,
                  O=None, stream=None, fast=False):
    """Multi-head attention on E4M3 codes: Q [BH, Sq, D], K and V [BH, Skv, D] (D = 64 or 128),
    per-tensor scales; softmax_scale defaults to 1/sqrt(D); returns O [BH, Sq, D] of out_dtype.
    fast=True computes Q K^T on the FP8 matrix cores (FP8_ACC_FAST)."""
    _require(isinstance(Q, torch.Tensor) and Q.is_cuda, "Q must be a GPU tensor")
    dev = Q.device
    for name, t in (("Q", Q), ("K", K), ("V", V)):
        _arg(t, name, dev, _CODES)
    _scales(dev, 1, scale_q=scale_q, scale_k=scale_k, scale_v=scale_v)
    Q, K, V = _codes(Q), _codes(K), _codes(V)
    _require(Q.dim() == 3 and K.dim() == 3 and V.dim() == 3, "Q, K, V must be [heads, seq, head_dim]")
    BH, Sq, D = Q.shape
    _require(K.shape == V.shape and K.shape[0] == BH and K.shape[2] == D, "K and V must be [heads, seq_kv, head_dim]")
    _require(Q.is_contiguous() and K.is_contiguous() and V.is_contiguous(), "Q, K, V must be contiguous")
    Skv = K.shape[1]
    if softmax_scale is None:
        softmax_scale = 1.0 / float(D) ** 0.5
    code = _out_code(out_dtype)
    O = _out_tensor(O, (BH, Sq, D), code, Q.device, "O")
    with _on(Q.device):
        _check("fp8_attention", lib.fp8_attention(_ptr(Q), _ptr(K), _ptr(V), _ptr(scale_q), _ptr(scale_k), _ptr(scale_v),
                                                  _ptr(O), BH, Sq, Skv, D, float(softmax_scale), int(bool(causal)),
                                                  code | (FP8_ACC_FAST if fast else 0), _stream(Q.device, stream)))
    return O
