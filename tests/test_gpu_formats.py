"""GPU parity of the operand-format and output variants, through the C ABI:
E5M2 quantization (bit-exact), GEMMs on every E4M3 / E5M2 operand pair and
FP16 output ("FP8 GEMM in JAX with Triton for Blackwell": both FP8 formats on
the matrix cores, a float16 store of the accumulator), against the oracle.

Bounds as for the E4M3 GEMM: FP32 within 2e-6*sum|ab|*sa*sb of the exact
value; BF16 / FP16 within 1 ulp of the oracle's correctly rounded value (with
the cancellation allowance of tests/parity.py); small-integer operands
bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_dense_linear_amd as P
from precision_dense_linear_amd import workloads as W
from parity import check_bf16, check_f16, check_f32, to_bits

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
E4M3, E5M2, F32, BF16, F16 = oracle.E4M3, oracle.E5M2, oracle.F32, oracle.BF16, oracle.F16
TORCH_OUT = {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16}
NAME = {E4M3: "e4m3", E5M2: "e5m2"}
PAIRS = [(E4M3, E5M2), (E5M2, E4M3), (E5M2, E5M2)]


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def one():
    return torch.ones(1, dtype=torch.float32, device=DEV)


def quantize(x, fmt):
    return (P.fp8_quantize_e5m2 if fmt == E5M2 else P.fp8_quantize)(gpu(x))


def compare(C, bits, exact, sab_scaled, kind, what):
    got = to_bits(C)
    if kind == F32:
        return check_f32(got.view(np.float32), exact, sab_scaled, what)
    if kind == BF16:
        return check_bf16(got, bits, exact, sab_scaled, what)
    return check_f16(got, bits, exact, sab_scaled, what)


# ------------------------------------------------------------------ E5M2 quantize
def quantize_e5m2_and_check(x, what):
    q, s, a = P.fp8_quantize_e5m2(gpu(x))
    torch.cuda.synchronize()
    oq, os_, oa = oracle.quantize_pertensor_fmt(x, E5M2)
    assert a.item() == oa and s.item() == os_, (what, a.item(), oa, s.item(), os_)
    qh = q.cpu().numpy()
    assert np.array_equal(qh, oq), "%s: %d codes differ" % (what, int((qh != oq).sum()))


@pytest.mark.parametrize("n", [1, 3, 4, 1023, 4099 * 7, 513 * 2048 + 5])
def test_quantize_e5m2_ragged_lengths(n):
    x = np.random.default_rng(n).standard_normal(n).astype(np.float32) * 3
    quantize_e5m2_and_check(x, "n=%d" % n)


def test_quantize_e5m2_operands_and_weights():
    a, b = W.pertensor_pair(8192, 8192, 8192, seed=1)
    quantize_e5m2_and_check(a, "A 8192^2")
    _, w = W.llm_linear(16, 8192, 8192)
    quantize_e5m2_and_check(w, "weight 8192^2 N(0, 0.02)")


def test_quantize_e5m2_empty_zero_and_saturation():
    q, s, a = P.fp8_quantize_e5m2(torch.zeros(0, device=DEV))
    assert s.item() == 1.0 and a.item() == 0.0
    q, s, a = P.fp8_quantize_e5m2(torch.zeros(37, device=DEV))
    assert s.item() == 1.0 and torch.count_nonzero(q).item() == 0
    x = np.array([57344, -57344, 61440, 1e-30, -1e-30, 2.0 ** -17, 3 * 2.0 ** -17, 1.125, 1.375, 0.0, -0.0, 7.0],
                 np.float32)
    q, s, _ = P.fp8_quantize_e5m2(gpu(x))
    oq, os_, _ = oracle.quantize_pertensor_fmt(x, E5M2)
    assert s.item() == os_ and np.array_equal(q.cpu().numpy(), oq)


def test_convert_e5m2_sweep_all_fp32_patterns():
    """Every binary32 pattern with |x| <= 57344 at scale exactly 1 (amax 57344
    appended), and every 61st pattern above it with the chunk's own scale."""
    chunk = 1 << 26
    for c0 in range(0, 1 << 32, chunk):
        bits = torch.arange(c0, c0 + chunk, dtype=torch.int64, device=DEV)
        bits = torch.where(bits >= 1 << 31, bits - (1 << 32), bits).to(torch.int32)
        x = bits.view(torch.float32)
        small = x[(x.abs() <= 57344.0)]
        if small.numel():
            xs = torch.cat([small, torch.tensor([57344.0], device=DEV)])
            q, s, _ = P.fp8_quantize_e5m2(xs)
            assert s.item() == 1.0
            xh = xs.cpu().numpy()
            ref = oracle.convert_fmt(xh, E5M2)
            qh = q.cpu().numpy()
            bad = qh != ref
            assert not bad.any(), (c0, xh[bad][:4], qh[bad][:4], ref[bad][:4])
        big = x[(x.abs() > 57344.0) & torch.isfinite(x)][::61]
        if big.numel():
            quantize_e5m2_and_check(big.cpu().numpy(), "patterns above 57344 from %#x" % c0)
        print("e5m2 sweep chunk %#010x done" % c0, flush=True)


def test_quantize_grouped_e5m2():
    x, w, off = W.moe(E=4, T=1000, K=512, N=384)
    offs = np.array([0, 0, 300, 301, 1000], np.int32)
    q, s, a = P.fp8_quantize_grouped_e5m2(gpu(x), gpu(offs))
    torch.cuda.synchronize()
    oq, os_, oa = oracle.quantize_grouped_fmt(x, offs, E5M2)
    assert np.array_equal(s.cpu().numpy(), os_) and np.array_equal(a.cpu().numpy(), oa)
    assert np.array_equal(q.cpu().numpy(), oq)


# ------------------------------------------------------------------ GEMM, integer-exact
def int_codes(shape, seed, fmt, lim=8):
    """Small integers, exact in both formats (E5M2 holds every integer up to 8)."""
    v = np.random.default_rng(seed).integers(-lim, lim + 1, shape).astype(np.float32)
    dt = torch.float8_e5m2 if fmt == E5M2 else torch.float8_e4m3fn
    return torch.from_numpy(v).to(dt).view(torch.uint8).numpy()


SHAPES = [(17, 48, 48), (65, 272, 1040), (300, 256, 512), (100, 8208, 272), (300, 5648, 272), (1100, 528, 272),
          (480, 28688, 32), (37, 1040, 4112)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("fa,fb", PAIRS)
@pytest.mark.parametrize("fast", [False, True])
def test_formats_integer_exact_bit_for_bit(M, N, K, fa, fb, fast):
    """Every tile class (32x64 with and without split-K, 64x64 at 100 x 8208 and 1100 x 528, 128x128 at 300 x 5648, 256x256 at 480 x 28688),
    both accumulation modes, all three output kinds."""
    qa, qb = int_codes((M, K), M + K, fa), int_codes((K, N), N + K, fb)
    A, B = gpu(qa), gpu(qb)
    ws = P.gemm_workspace(DEV)   # (37, 1040, 4112) splits K across workgroups
    for kind in (F32, BF16, F16):
        C = P.fp8_gemm(A, B, one(), one(), TORCH_OUT[kind], fast=fast, a_fmt=NAME[fa], b_fmt=NAME[fb], workspace=ws)
        bits, _, _ = oracle.gemm_rows_fmt(qa, qb, fa, fb, 1.0, 1.0, kind)
        got = to_bits(C)
        assert np.array_equal(got, bits), "kind %d: %d mismatches" % (kind, int((got != bits).sum()))


def test_e4m3_f16_integer_exact_and_identity():
    qa, qb = int_codes((300, 512), 1, E4M3, lim=16), int_codes((512, 256), 2, E4M3, lim=16)
    C = P.fp8_gemm(gpu(qa), gpu(qb), one(), one(), torch.float16)
    bits, _, _ = oracle.gemm_rows_fmt(qa, qb, E4M3, E4M3, 1.0, 1.0, F16)
    assert np.array_equal(to_bits(C), bits)
    # identity B in E5M2 (0x3C = 1.0): C = sa*sb*A, FP32 exact
    rng = np.random.default_rng(8)
    qa = rng.integers(0, 256, (300, 256)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x38
    eye = np.zeros((256, 256), np.uint8)
    eye[np.arange(256), np.arange(256)] = 0x3C
    half = torch.tensor([0.5], device=DEV)
    C = P.fp8_gemm(gpu(qa), gpu(eye), half, half * 0.5, torch.float32, b_fmt="e5m2")
    assert np.array_equal(C.cpu().numpy(), (oracle.decode(qa) * 0.125).astype(np.float32))


def test_f16_overflow_to_infinity():
    """Sums beyond the binary16 range become +-Inf, as the oracle's rounding says."""
    K = 1024
    qa = np.full((40, K), 0x50, np.uint8)          # E4M3 8.0
    qb = np.full((K, 48), 0x48, np.uint8)          # E5M2 8.0
    qb[:, 1::2] = 0xC8                             # -8.0
    C = P.fp8_gemm(gpu(qa), gpu(qb), one(), one(), torch.float16, b_fmt="e5m2")
    bits, exact, _ = oracle.gemm_rows_fmt(qa, qb, E4M3, E5M2, 1.0, 1.0, F16)
    assert np.all(exact[:, 0] == 65536.0) and np.all(bits[:, 0] == 0x7C00) and np.all(bits[:, 1] == 0xFC00)
    assert np.array_equal(to_bits(C), bits)


# ------------------------------------------------------------------ GEMM, random data end to end
@pytest.mark.parametrize("fa,fb", PAIRS)
@pytest.mark.parametrize("M,N,K,kind", [(256, 256, 256, F32), (1024, 1024, 1024, F16), (33, 400, 208, F16),
                                        (200, 144, 400, BF16), (16, 8192, 8192, F16)])
def test_formats_random_end_to_end(fa, fb, M, N, K, kind):
    a, b = W.pertensor_pair(M, N, K, seed=M + 3 * fa + 5 * fb)
    qa, sa, _ = quantize(a, fa)
    qb, sb, _ = quantize(b, fb)
    C = P.fp8_gemm(qa, qb, sa, sb, TORCH_OUT[kind], a_fmt=NAME[fa], b_fmt=NAME[fb])
    torch.cuda.synchronize()
    oa, osa, _ = oracle.quantize_pertensor_fmt(a, fa)
    ob, osb, _ = oracle.quantize_pertensor_fmt(b, fb)
    assert np.array_equal(qa.cpu().numpy(), oa) and np.array_equal(qb.cpu().numpy(), ob)
    bits, exact, sab = oracle.gemm_rows_fmt(oa, ob, fa, fb, osa, osb, kind)
    res = compare(C, bits, exact, sab * float(osa) * float(osb), kind, "%s x %s %dx%dx%d" % (NAME[fa], NAME[fb], M, N, K))
    print(NAME[fa], NAME[fb], (M, N, K), kind, "->", res, flush=True)


def test_mixed_8192_f16_sampled_rows():
    """The 8192^3 mixed workload (A E4M3, B E5M2, FP16 out) on sampled rows."""
    a, b = W.pertensor_pair(8192, 8192, 8192, seed=0)
    qa, sa, _ = quantize(a, E4M3)
    qb, sb, _ = quantize(b, E5M2)
    C = P.fp8_gemm(qa, qb, sa, sb, torch.float16, b_fmt="e5m2")
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, 8191, np.random.default_rng(2).choice(8192, 10, replace=False)])
    oa, osa, _ = oracle.quantize_pertensor_fmt(a, E4M3)
    ob, osb, _ = oracle.quantize_pertensor_fmt(b, E5M2)
    bits, exact, sab = oracle.gemm_rows_fmt(oa, ob, E4M3, E5M2, osa, osb, F16, rows=rows)
    got = to_bits(C)[rows]
    print("mixed 8192^3 F16 ->", check_f16(got, bits, exact, sab * float(osa) * float(osb), "mixed 8192^3"))


FAST_REL = 7 * 2.0 ** -13 + 2e-6


@pytest.mark.parametrize("fa,fb", PAIRS)
def test_formats_fast_within_bound(fa, fb):
    a, b = W.pertensor_pair(1024, 1024, 1024, seed=4)
    qa, sa, _ = quantize(a, fa)
    qb, sb, _ = quantize(b, fb)
    C = P.fp8_gemm(qa, qb, sa, sb, torch.float32, fast=True, a_fmt=NAME[fa], b_fmt=NAME[fb])
    C2 = P.fp8_gemm(qa, qb, sa, sb, torch.float32, fast=True, a_fmt=NAME[fa], b_fmt=NAME[fb])
    torch.cuda.synchronize()
    assert torch.equal(C, C2)
    oa, osa, _ = oracle.quantize_pertensor_fmt(a, fa)
    ob, osb, _ = oracle.quantize_pertensor_fmt(b, fb)
    _, exact, sab = oracle.gemm_rows_fmt(oa, ob, fa, fb, osa, osb, F32)
    err = np.abs(C.cpu().numpy().astype(np.float64) - exact)
    bound = FAST_REL * sab * float(osa) * float(osb) + 1e-15 * np.abs(exact)
    assert np.all(err <= bound), "%d outputs beyond the fast bound" % int((err > bound).sum())
    print(NAME[fa], NAME[fb], "fast max err / sum|ab| =", float((err / np.maximum(sab * float(osa) * float(osb), 1e-300)).max()))


# ------------------------------------------------------------------ grouped and block-scaled
@pytest.mark.parametrize("fast", [False, True])
def test_grouped_e5m2_weights_f16(fast):
    x, w, off = W.moe(E=4, T=1000, K=512, N=384)
    E, K, N = w.shape
    goff = gpu(off.astype(np.int32))
    woff = (np.arange(E + 1) * K).astype(np.int32)
    qx, sx, _ = P.fp8_quantize_grouped(gpu(x), goff)
    qw, sw, _ = P.fp8_quantize_grouped_e5m2(gpu(w.reshape(E * K, N)), gpu(woff))
    C = P.fp8_grouped_gemm(qx, qw.view(E, K, N), goff, sx, sw, torch.float16, fast=fast, b_fmt="e5m2")
    torch.cuda.synchronize()
    ox, osx, _ = oracle.quantize_grouped(x, off)
    ow, osw, _ = oracle.quantize_grouped_fmt(w.reshape(E * K, N), woff, E5M2)
    assert np.array_equal(qw.cpu().numpy(), ow)
    got = to_bits(C)
    ow = ow.reshape(E, K, N)
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        rows = np.arange(r0, r1)
        bits, exact, sab = oracle.gemm_rows_fmt(ox, ow[e], E4M3, E5M2, osx[e], osw[e], F16, rows=rows)
        if fast:
            gv = got[rows].view(np.float16).astype(np.float64)
            bound = FAST_REL * sab * float(osx[e]) * float(osw[e]) + np.ldexp(1.0, np.frexp(np.abs(exact))[1] - 11)
            assert np.all(np.abs(gv - exact) <= bound + 2.0 ** -24)
        else:
            check_f16(got[rows], bits, exact, sab * float(osx[e]) * float(osw[e]), "expert %d" % e)


def test_blockscaled_f16_output():
    a, b = W.blockscaled_pair(256, 256, 512)
    qa, sa = P.fp8_quantize_blocked(gpu(a))
    qb, sb = P.fp8_quantize_blocked(gpu(b))
    C = P.fp8_gemm_blockscaled(qa, qb, sa, sb, torch.float16)
    torch.cuda.synchronize()
    oa, osa = oracle.quantize_blocked(a)
    ob, osb = oracle.quantize_blocked(b)
    _, exact, sab = oracle.gemm_blockscaled_rows(oa, ob, osa, osb, F32)
    bits = np.array([oracle.round_ieee_f64(float(v), F16) for v in exact.ravel()], np.uint16).reshape(exact.shape)
    print("block-scaled F16 ->", check_f16(to_bits(C), bits, exact, sab, "block-scaled F16"))
