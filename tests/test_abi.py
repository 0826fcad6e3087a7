"""The C-ABI library without a GPU: it loads, exports every function the
header declares, and rejects bad arguments on the host before launching
anything (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import precision_dense_linear_amd as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8gemm.h")

# Any non-null address works for the validation paths: none of these calls
# reaches a launch, so the pointers are never dereferenced.
FAKE = ctypes.c_void_p(0x100000)
FAKE_ODD = ctypes.c_void_p(0x100008)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("fp8_quantize", "fp8_quantize_e5m2", "fp8_quantize_blocked", "fp8_quantize_blocked64",
              "fp8_quantize_blocked_e8m0", "fp8_gemm_blockscaled_e8m0", "fp8_quantize_2of4", "fp8_gemm_sparse24",
              "fp8_quantize_grouped",
              "fp8_quantize_grouped_e5m2", "fp8_gemm", "fp8_gemm_ws", "fp8_gemm_blockscaled", "fp8_grouped_gemm",
              "fp8_status_string", "fp8_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(P.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(declared_functions()) == set(P.SYMBOLS)


def test_status_strings():
    assert P.status_name(0) == "FP8_OK"
    assert P.status_name(1) == "FP8_ERR_INVALID_ARG"
    assert P.status_name(2) == "FP8_ERR_UNSUPPORTED_SHAPE"
    assert P.status_name(3) == "FP8_ERR_HIP"
    assert P.status_name(99) == "FP8_ERR_UNKNOWN"


def gemm(A=FAKE, B=FAKE, sa=FAKE, sb=FAKE, C=FAKE, M=64, N=64, K=64, out=1):
    return P.lib.fp8_gemm(A, B, sa, sb, C, M, N, K, out, None)


@pytest.mark.parametrize("kw,status", [
    (dict(A=None), P.FP8_ERR_INVALID_ARG),
    (dict(A=None, M=0), P.FP8_OK),        # an empty operand may be null (M == 0: nothing is launched)
    (dict(B=None), P.FP8_ERR_INVALID_ARG),
    (dict(C=None), P.FP8_ERR_INVALID_ARG),
    (dict(sa=None), P.FP8_ERR_INVALID_ARG),
    (dict(M=-1), P.FP8_ERR_INVALID_ARG),
    (dict(K=-16), P.FP8_ERR_INVALID_ARG),
    (dict(out=7), P.FP8_ERR_INVALID_ARG),
    (dict(out=3), P.FP8_ERR_INVALID_ARG),
    (dict(out=1 | 0x800), P.FP8_ERR_INVALID_ARG),             # unknown flag bit
    (dict(out=2 | 0x200 | 0x400 | 0x100, M=0), P.FP8_OK),     # FP16 out, both E5M2, fast: accepted
    (dict(A=FAKE_ODD), P.FP8_ERR_INVALID_ARG),
    (dict(K=40), P.FP8_ERR_UNSUPPORTED_SHAPE),
    (dict(N=40), P.FP8_ERR_UNSUPPORTED_SHAPE),
    (dict(K=(1 << 23) + 16), P.FP8_ERR_UNSUPPORTED_SHAPE),
    (dict(A=None, M=1 << 40, K=1 << 40), P.FP8_ERR_UNSUPPORTED_SHAPE),  # limits come before M*K is formed
    (dict(M=1 << 31), P.FP8_ERR_UNSUPPORTED_SHAPE),
    (dict(N=1 << 21), P.FP8_ERR_UNSUPPORTED_SHAPE),
    (dict(M=0), P.FP8_OK),            # empty: nothing to enqueue
    (dict(N=0), P.FP8_OK),
])
def test_gemm_validation(kw, status):
    assert gemm(**kw) == status
    if status != P.FP8_OK:
        assert P.lib.fp8_last_error().decode() != ""


def gemm_ws(ws=FAKE, nbytes=1 << 22, M=64, N=64, K=64, out=1, **kw):
    return P.lib.fp8_gemm_ws(kw.get("A", FAKE), kw.get("B", FAKE), FAKE, FAKE, kw.get("C", FAKE), M, N, K, out,
                             ws, nbytes, None)


def test_gemm_ws_validation():
    """fp8_gemm_ws checks its workspace before anything else reaches the GPU,
    and otherwise validates exactly like fp8_gemm."""
    assert gemm_ws(nbytes=-1) == P.FP8_ERR_INVALID_ARG
    assert gemm_ws(ws=None, nbytes=8196) == P.FP8_ERR_INVALID_ARG       # null workspace with a size
    assert gemm_ws(ws=FAKE_ODD) == P.FP8_ERR_INVALID_ARG                # misaligned workspace
    assert gemm_ws(ws=None, nbytes=0, M=0) == P.FP8_OK                  # no workspace: plain fp8_gemm
    assert gemm_ws(M=0) == P.FP8_OK
    assert gemm_ws(N=40) == P.FP8_ERR_UNSUPPORTED_SHAPE
    assert gemm_ws(A=None) == P.FP8_ERR_INVALID_ARG
    assert gemm_ws(out=1 | 0x800) == P.FP8_ERR_INVALID_ARG
    assert "workspace" in (P.lib.fp8_gemm_ws(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 64, 64, 1, None, 16, None) and
                           P.lib.fp8_last_error().decode())
    # the header's sizes agree with the binding's
    text = open(HEADER).read()
    assert "#define FP8_GEMM_WS_TILE_BYTES %d" % P.FP8_GEMM_WS_TILE_BYTES in text
    assert P.FP8_GEMM_WS_TILE_BYTES == 32 * 64 * 4 + 4


def test_gemm_noalloc_validation():
    """fp8_gemm_noalloc rejects bad arguments, and returns at once for an
    empty problem, before it touches any device (its scratch set-up included)."""
    f = P.lib.fp8_gemm_noalloc
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 40, 64, 1, None) == P.FP8_ERR_UNSUPPORTED_SHAPE
    assert f(None, FAKE, FAKE, FAKE, FAKE, 64, 64, 64, 1, None) == P.FP8_ERR_INVALID_ARG
    assert f(FAKE, FAKE, None, FAKE, FAKE, 64, 64, 64, 1, None) == P.FP8_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 64, 64, 1 | 0x800, None) == P.FP8_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 64, 64, 1, None) == P.FP8_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 64, 64, 1 | P.FP8_ACC_FAST, None) == P.FP8_OK
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 0, 64, 1, None) == P.FP8_OK


def test_library_does_not_allocate():
    """No entry point allocates device memory: the library's sources call no
    allocator (scratch memory comes from the caller)."""
    csrc = os.path.join(ROOT, "precision_dense_linear_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        text = open(os.path.join(csrc, f)).read()
        for fn in ("hipMalloc", "hipFree", "hipExtMalloc", "hipMallocAsync", "hipHostMalloc"):
            assert fn not in text, "%s calls %s" % (f, fn)


def test_blockscaled_validation():
    f = P.lib.fp8_gemm_blockscaled
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 48, 64, 64, 1, None) == P.FP8_ERR_UNSUPPORTED_SHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 64, 48, 1, None) == P.FP8_ERR_UNSUPPORTED_SHAPE
    assert f(FAKE, FAKE, None, FAKE, FAKE, 64, 64, 64, 1, None) == P.FP8_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 64, 64, 1, None) == P.FP8_OK
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 64, 64, 2, None) == P.FP8_OK                 # FP16 out
    for flag in (P.FP8_A_E5M2, P.FP8_B_E5M2, P.FP8_ACC_FAST):                              # E4M3, exact only
        assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 64, 64, 1 | flag, None) == P.FP8_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 96, 64, 64, 1 | P.FP8_BLOCK64, None) == P.FP8_ERR_UNSUPPORTED_SHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 64, 96, 1 | P.FP8_BLOCK64, None) == P.FP8_ERR_UNSUPPORTED_SHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 64, 64, 2 | P.FP8_BLOCK64, None) == P.FP8_OK
    assert gemm(out=1 | P.FP8_BLOCK64) == P.FP8_ERR_INVALID_ARG                           # block-scaled only
    assert P.lib.fp8_grouped_gemm(FAKE, FAKE, FAKE, 8, FAKE, FAKE, FAKE, 64, 64, 64, 1 | P.FP8_BLOCK64, None) \
        == P.FP8_ERR_INVALID_ARG


def test_grouped_validation():
    f = P.lib.fp8_grouped_gemm
    assert f(FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, 64, 64, 64, 1, None) == P.FP8_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, 1025, FAKE, FAKE, FAKE, 64, 64, 64, 1, None) == P.FP8_ERR_INVALID_ARG
    assert f(FAKE, FAKE, None, 8, FAKE, FAKE, FAKE, 64, 64, 64, 1, None) == P.FP8_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, 8, FAKE, FAKE, FAKE, 64, 64, 40, 1, None) == P.FP8_ERR_UNSUPPORTED_SHAPE
    assert f(FAKE, FAKE, FAKE, 8, FAKE, FAKE, FAKE, 0, 64, 64, 1, None) == P.FP8_OK


def test_quantize_validation():
    L = P.lib
    assert L.fp8_quantize(None, 16, FAKE, FAKE, FAKE, None) == P.FP8_ERR_INVALID_ARG
    assert L.fp8_quantize(FAKE, -1, FAKE, FAKE, FAKE, None) == P.FP8_ERR_INVALID_ARG
    assert L.fp8_quantize(FAKE_ODD, 16, FAKE, FAKE, ctypes.c_void_p(0x200000), None) == P.FP8_ERR_INVALID_ARG
    assert L.fp8_quantize(FAKE, 16, FAKE, FAKE, FAKE, None) == P.FP8_ERR_INVALID_ARG   # scale aliases amax
    assert L.fp8_quantize_e5m2(None, 16, FAKE, FAKE, FAKE, None) == P.FP8_ERR_INVALID_ARG
    assert L.fp8_quantize_e5m2(FAKE, 16, FAKE, FAKE, FAKE, None) == P.FP8_ERR_INVALID_ARG
    assert L.fp8_quantize_grouped_e5m2(FAKE, 64, 64, FAKE, 0, FAKE, FAKE, ctypes.c_void_p(0x200000), None) \
        == P.FP8_ERR_INVALID_ARG
    assert L.fp8_quantize_blocked(FAKE, 48, 64, FAKE, FAKE, None) == P.FP8_ERR_UNSUPPORTED_SHAPE
    assert L.fp8_quantize_blocked(FAKE, 64, 64, None, FAKE, None) == P.FP8_ERR_INVALID_ARG
    assert L.fp8_quantize_blocked_e8m0(FAKE, 96, 48, 0, FAKE, FAKE, None) == P.FP8_ERR_UNSUPPORTED_SHAPE
    assert L.fp8_quantize_blocked_e8m0(FAKE, 64, 64, 2, FAKE, FAKE, None) == P.FP8_ERR_INVALID_ARG
    assert L.fp8_quantize_blocked_e8m0(FAKE, 64, 64, 1, FAKE, None, None) == P.FP8_ERR_INVALID_ARG
    f = L.fp8_gemm_blockscaled_e8m0
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 64, 48, 1, None) == P.FP8_ERR_UNSUPPORTED_SHAPE
    assert f(FAKE, FAKE, None, FAKE, FAKE, 64, 64, 64, 1, None) == P.FP8_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 64, 64, 1 | P.FP8_ACC_FAST, None) == P.FP8_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 64, 64, 2, None) == P.FP8_OK
    assert L.fp8_quantize_2of4(FAKE, 48, 64, FAKE, FAKE, FAKE, ctypes.c_void_p(0x200000), None) \
        == P.FP8_ERR_UNSUPPORTED_SHAPE
    assert L.fp8_quantize_2of4(FAKE, 64, 64, None, FAKE, FAKE, ctypes.c_void_p(0x200000), None) \
        == P.FP8_ERR_INVALID_ARG
    assert L.fp8_quantize_2of4(FAKE, 64, 64, FAKE, FAKE, FAKE, FAKE, None) == P.FP8_ERR_INVALID_ARG   # scale is amax
    f = L.fp8_gemm_sparse24
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 64, 48, 1, None) == P.FP8_ERR_UNSUPPORTED_SHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 40, 64, 1, None) == P.FP8_ERR_UNSUPPORTED_SHAPE
    assert f(FAKE, FAKE, None, FAKE, FAKE, FAKE, 64, 64, 64, 1, None) == P.FP8_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE_ODD, FAKE, FAKE, FAKE, 64, 64, 64, 1, None) == P.FP8_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 64, 64, 1 | P.FP8_ACC_FAST, None) == P.FP8_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 64, 64, 2, None) == P.FP8_OK
    assert L.fp8_quantize_blocked64(FAKE, 96, 64, FAKE, FAKE, None) == P.FP8_ERR_UNSUPPORTED_SHAPE
    assert L.fp8_quantize_blocked64(FAKE, 64, 64, None, FAKE, None) == P.FP8_ERR_INVALID_ARG
    assert L.fp8_quantize_blocked64(FAKE, 0, 64, FAKE, FAKE, None) == P.FP8_OK
    assert L.fp8_quantize_grouped(FAKE, 64, 64, FAKE, 0, FAKE, FAKE, ctypes.c_void_p(0x200000), None) \
        == P.FP8_ERR_INVALID_ARG
    assert L.fp8_quantize_grouped(FAKE, 64, 6, FAKE, 2, FAKE, FAKE, ctypes.c_void_p(0x200000), None) \
        == P.FP8_ERR_UNSUPPORTED_SHAPE


def test_binding_refuses_wrong_operand_dtype():
    import torch
    with pytest.raises(TypeError):
        P._codes(torch.zeros(4, dtype=torch.float16))
    # a float8_e5m2 tensor cannot be passed as E4M3 codes, and the format must be known
    with pytest.raises(ValueError):
        P._fmt_flag(torch.zeros(4, dtype=torch.float8_e5m2), "e4m3", P.FP8_A_E5M2)
    with pytest.raises(ValueError):
        P._fmt_flag(torch.zeros(4, dtype=torch.uint8), "e3m4", P.FP8_A_E5M2)
    assert P._fmt_flag(torch.zeros(4, dtype=torch.float8_e5m2), None, P.FP8_B_E5M2) == P.FP8_B_E5M2
    assert P._fmt_flag(torch.zeros(4, dtype=torch.uint8), "e5m2", P.FP8_A_E5M2) == P.FP8_A_E5M2
    assert P._fmt_flag(torch.zeros(4, dtype=torch.uint8), None, P.FP8_A_E5M2) == 0


def test_missing_library_fails_loudly(tmp_path):
    """The binding has no fallback: a package directory without the built
    library refuses to import (nothing runs on the CPU in its place)."""
    import shutil
    import subprocess
    import sys
    pkg = tmp_path / "precision_dense_linear_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(os.path.dirname(P.__file__), "__init__.py"), pkg / "__init__.py")
    code = ("import sys; sys.path.insert(0, %r)\n"
            "try:\n    import precision_dense_linear_amd\nexcept ImportError as e:\n    print('IMPORT-ERROR', e)\n"
            "else:\n    print('IMPORTED', precision_dense_linear_amd.__file__)\n") % str(tmp_path)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300).stdout
    assert "IMPORT-ERROR" in out and "not built" in out, out


def attention(Q=FAKE, K=FAKE, V=FAKE, sq=FAKE, sk=FAKE, sv=FAKE, O=FAKE, BH=2, Sq=64, Skv=64, D=128, scale=0.125,
              causal=0, out=1):
    return P.lib.fp8_attention(Q, K, V, sq, sk, sv, O, BH, Sq, Skv, D, scale, causal, out, None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=96), P.FP8_ERR_UNSUPPORTED_SHAPE),
    (dict(D=256), P.FP8_ERR_UNSUPPORTED_SHAPE),
    (dict(BH=-1), P.FP8_ERR_INVALID_ARG),
    (dict(Sq=-1), P.FP8_ERR_INVALID_ARG),
    (dict(out=3), P.FP8_ERR_INVALID_ARG),
    (dict(out=1 | 0x200), P.FP8_ERR_INVALID_ARG),              # operand formats: not taken here
    (dict(out=1 | 0x800), P.FP8_ERR_INVALID_ARG),
    (dict(out=1 | 0x100, Sq=0), P.FP8_OK),                     # FP8_ACC_FAST: accepted
    (dict(causal=2), P.FP8_ERR_INVALID_ARG),
    (dict(scale=0.0), P.FP8_ERR_INVALID_ARG),
    (dict(scale=-1.0), P.FP8_ERR_INVALID_ARG),
    (dict(scale=float("inf")), P.FP8_ERR_INVALID_ARG),
    (dict(scale=float("nan")), P.FP8_ERR_INVALID_ARG),
    (dict(Q=None), P.FP8_ERR_INVALID_ARG),
    (dict(K=None), P.FP8_ERR_INVALID_ARG),
    (dict(O=None), P.FP8_ERR_INVALID_ARG),
    (dict(sv=None), P.FP8_ERR_INVALID_ARG),
    (dict(V=FAKE_ODD), P.FP8_ERR_INVALID_ARG),
    (dict(Sq=1 << 24), P.FP8_ERR_UNSUPPORTED_SHAPE),           # one head past 2^31 bytes
    (dict(Skv=1 << 25, D=64), P.FP8_ERR_UNSUPPORTED_SHAPE),
    (dict(Sq=0), P.FP8_OK),                                    # nothing to write
    (dict(BH=0), P.FP8_OK),
    (dict(K=None, V=None, Skv=0, Sq=0), P.FP8_OK),
])
def test_attention_validation(kw, status):
    assert attention(**kw) == status
    if status != P.FP8_OK:
        assert P.lib.fp8_last_error().decode() != ""


def test_binding_rejects_host_tensors_before_any_call():
    """Host (CPU) tensors never reach the library: every entry point of the
    binding raises before its first HIP call, since a host pointer handed to
    a kernel would fault the GPU."""
    import torch
    x = torch.zeros(64, 64)
    c = torch.zeros(64, 64, dtype=torch.uint8)
    b3 = torch.zeros(2, 64, 64, dtype=torch.uint8)
    s = torch.ones(1)
    off = torch.tensor([0, 32, 64], dtype=torch.int32)
    calls = {
        "fp8_quantize": lambda: P.fp8_quantize(x),
        "fp8_quantize_e5m2": lambda: P.fp8_quantize_e5m2(x),
        "fp8_quantize_blocked": lambda: P.fp8_quantize_blocked(x),
        "fp8_quantize_blocked64": lambda: P.fp8_quantize_blocked64(x),
        "fp8_quantize_blocked_e8m0": lambda: P.fp8_quantize_blocked_e8m0(x),
        "fp8_quantize_grouped": lambda: P.fp8_quantize_grouped(x, off),
        "fp8_quantize_grouped_e5m2": lambda: P.fp8_quantize_grouped_e5m2(x, off),
        "fp8_quantize_2of4": lambda: P.fp8_quantize_2of4(x),
        "fp8_gemm": lambda: P.fp8_gemm(c, c, s, s),
        "fp8_gemm_ws": lambda: P.fp8_gemm(c, c, s, s, workspace=torch.zeros(16, dtype=torch.uint8)),
        "fp8_gemm_noalloc": lambda: P.fp8_gemm_noalloc(c, c, s, s),
        "fp8_gemm_blockscaled": lambda: P.fp8_gemm_blockscaled(c, c, torch.ones(2, 2), torch.ones(2, 2)),
        "fp8_gemm_blockscaled_e8m0": lambda: P.fp8_gemm_blockscaled_e8m0(c, c, torch.zeros(2, 4, dtype=torch.uint8),
                                                                         torch.zeros(2, 4, dtype=torch.uint8)),
        "fp8_gemm_sparse24": lambda: P.fp8_gemm_sparse24(c, torch.zeros(32, 64, dtype=torch.uint8),
                                                         torch.zeros(2, 64, dtype=torch.int32), s, s),
        "fp8_grouped_gemm": lambda: P.fp8_grouped_gemm(c, b3, off, torch.ones(2), torch.ones(2)),
        "fp8_attention": lambda: P.fp8_attention(b3, b3, b3, s, s, s),
    }
    for name, call in calls.items():
        with pytest.raises(ValueError, match="GPU tensor"):
            call()
