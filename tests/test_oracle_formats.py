"""Pins of the oracle's operand-format and output variants: OCP E5M2 codes,
mixed E4M3 x E5M2 GEMMs and FP16 output ("FP8 GEMM in JAX with Triton for
Blackwell": both FP8 formats on the matrix cores, a float16 store of the
accumulator).

Each function is checked against something other than itself: the closed
form of the E5M2 fields, torch's float8_e5m2 decode and cast, numpy's
float64 -> float16 / float32 casts, the already-pinned E4M3 GEMM path, exact
rational brute force on tiny inputs, closed-form products, and invariants.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

E4M3, E5M2, F32, BF16, F16 = oracle.E4M3, oracle.E5M2, oracle.F32, oracle.BF16, oracle.F16


# ---------------------------------------------------------------- E5M2 decode
def closed_form_e5m2(c: int) -> float:
    s = -1.0 if c & 0x80 else 1.0
    e = (c >> 2) & 0x1F
    m = c & 0x3
    if e == 31:
        return s * float("inf") if m == 0 else float("nan")
    if e == 0:
        return s * m * 2.0 ** -16
    return s * 2.0 ** (e - 15) * (1 + m / 4)


def torch_e5m2_decode(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e5m2).to(torch.float64).numpy()


def torch_sat_cast_e5m2(x):
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).clamp(-57344.0, 57344.0)
    return t.to(torch.float8_e5m2).view(torch.uint8).numpy()


def test_e5m2_table_matches_closed_form_all_codes():
    t = oracle.e5m2_table()
    for c in range(256):
        ref = closed_form_e5m2(c)
        if np.isnan(ref):
            assert np.isnan(t[c]), c
        else:
            assert t[c] == ref and np.signbit(t[c]) == np.signbit(ref), (c, t[c], ref)


def test_e5m2_table_matches_torch_float8_e5m2():
    t = oracle.e5m2_table()
    ref = torch_e5m2_decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(t), nan)
    assert np.array_equal(t[~nan], ref[~nan])


def test_e5m2_invariants():
    t = oracle.e5m2_table()
    fin = t[np.isfinite(t)]
    assert list(np.nonzero(np.isnan(t))[0]) == [0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF]
    assert t[0x7C] == np.inf and t[0xFC] == -np.inf
    assert fin.max() == 57344.0 == t[0x7B] and fin.min() == -57344.0
    assert len(np.unique(fin)) == 247                               # 124 magnitudes, +-0 coincide
    assert np.all(np.diff(t[0x00:0x7D]) > 0)                        # monotone up to +Inf
    assert np.array_equal(t[0x80:0xFC], -t[0x00:0x7C])
    assert np.all(fin * 65536 == np.round(fin * 65536))             # multiples of 2^-16
    assert t[0x01] == 2.0 ** -16 and t[0x04] == 2.0 ** -14 and t[0x3C] == 1.0
    # every E5M2 value is a binary16 value (E5M2 is the top byte of binary16)
    h = (np.arange(256, dtype=np.uint16) << 8).view(np.float16).astype(np.float64)
    assert np.array_equal(h[np.isfinite(t)], fin) and np.array_equal(np.isinf(h), np.isinf(t))


# ---------------------------------------------------------------- E5M2 convert
def test_e5m2_convert_every_rounding_class_vs_torch_cast():
    """Every sign, every binary32 exponent and every value of the top 12
    mantissa bits, each with the low 11 bits 0, 1, 0x400 and 0x7FF: this
    covers each E5M2 code's kept bits, the round bit and an empty / non-empty
    sticky part on both sides of every tie (8.4M patterns; NaNs excluded)."""
    hi = np.arange(1 << 21, dtype=np.uint64) << np.uint64(11)       # sign, exponent, top 12 mantissa bits
    for low in (0, 1, 0x400, 0x7FF):
        bits = (hi | np.uint64(low)).astype(np.uint32)
        x = bits.view(np.float32)
        keep = ~np.isnan(x)
        q = oracle.convert_fmt(x, E5M2)
        ref = torch_sat_cast_e5m2(x)
        bad = (q != ref) & keep
        assert not bad.any(), (low, x[bad][:5], q[bad][:5], ref[bad][:5])


def brute_nearest_e5m2(v: float) -> int:
    t = oracle.e5m2_table()
    fv = Fraction(float(v)) if np.isfinite(v) else None
    best, bestd = None, None
    for c in range(256):
        if not np.isfinite(t[c]) or (c & 0x80) != (0x80 if np.signbit(v) else 0):
            continue
        if fv is None:
            d = -abs(Fraction(float(t[c])))            # infinity: the largest magnitude
        else:
            d = abs(Fraction(float(t[c])) - fv)
        if bestd is None or d < bestd or (d == bestd and c % 2 == 0 and best % 2 == 1):
            best, bestd = c, d
    return best


def test_e5m2_convert_brute_force_on_ties_and_neighbours():
    t = oracle.e5m2_table()
    mags = np.unique(np.abs(t[np.isfinite(t)]))
    vals = []
    for a, b in zip(mags[:-1], mags[1:]):
        mid = np.float32((a + b) / 2)
        vals += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9)), np.float32(a)]
    vals += [np.float32(57344), np.float32(61440), np.float32(61441), np.float32(1e30), np.float32(np.inf),
             np.float32(2.0 ** -17), np.float32(3 * 2.0 ** -17), np.float32(1e-45), np.float32(0.0)]
    vals = np.array(vals, np.float32)
    for v in np.concatenate([vals, -vals]):
        assert oracle.e5m2_rne_sat(float(v)) == brute_nearest_e5m2(float(v)), v


def test_e5m2_convert_hand_cases():
    assert oracle.e5m2_rne_sat(2.0 ** -17) == 0x00            # tie 0 / 2^-16 -> even
    assert oracle.e5m2_rne_sat(-(2.0 ** -17)) == 0x80
    assert oracle.e5m2_rne_sat(3 * 2.0 ** -17) == 0x02        # tie 1 / 2 (x2^-16) -> 2
    assert oracle.e5m2_rne_sat(1.125) == 0x3C                 # tie 1.0 / 1.25 -> 1.0
    assert oracle.e5m2_rne_sat(1.375) == 0x3E                 # tie 1.25 / 1.5 -> 1.5
    assert oracle.e5m2_rne_sat(61440.0) == 0x7B               # saturates (a plain cast gives Inf)
    assert oracle.e5m2_rne_sat(float("inf")) == 0x7B and oracle.e5m2_rne_sat(float("-inf")) == 0xFB


# ---------------------------------------------------------------- quantize
def test_scale_and_quantize_pertensor_e5m2_vs_torch():
    x = np.random.default_rng(3).standard_normal((300, 77)).astype(np.float32) * 5
    q, s, a = oracle.quantize_pertensor_fmt(x, E5M2)
    assert a == np.abs(x).max()
    assert s == np.float32(a) / np.float32(57344.0)
    assert np.array_equal(q, torch_sat_cast_e5m2(x / s))
    # the extreme element lands on the format's maximum
    assert np.abs(oracle.e5m2_table()[q]).max() == 57344.0
    assert oracle.scale_from_amax_fmt(0.0, E5M2) == 1.0
    # E4M3 through the format-generic entry equals the E4M3 functions
    q4, s4, a4 = oracle.quantize_pertensor_fmt(x, E4M3)
    r4, rs4, ra4 = oracle.quantize_pertensor(x)
    assert np.array_equal(q4, r4) and s4 == rs4 and a4 == ra4


def test_quantize_grouped_e5m2_reduces_to_per_group():
    x = np.random.default_rng(4).standard_normal((50, 12)).astype(np.float32)
    off = np.array([0, 7, 7, 31, 50], np.int32)
    q, s, a = oracle.quantize_grouped_fmt(x, off, E5M2)
    assert s[1] == 1.0 and a[1] == 0.0
    for g in range(4):
        if off[g + 1] > off[g]:
            rq, rs, ra = oracle.quantize_pertensor_fmt(x[off[g]:off[g + 1]], E5M2)
            assert np.array_equal(q[off[g]:off[g + 1]], rq) and s[g] == rs and a[g] == ra


# ---------------------------------------------------------------- rounding to FP16 / BF16 / FP32
def f16_bits(x: float) -> int:
    with np.errstate(over="ignore"):
        return int(np.array([x], np.float64).astype(np.float16).view(np.uint16)[0])


def test_round_ieee_f16_matches_numpy_cast():
    rng = np.random.default_rng(5)
    xs = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.uniform(-9, 5, 20000),
                         rng.uniform(-70000, 70000, 2000), [65504.0, 65519.99, 65520.0, 1e10, 2.0 ** -24,
                                                            2.0 ** -25, 3 * 2.0 ** -26, 0.0, -0.0]])
    for x in xs:
        assert oracle.round_ieee_f64(float(x), F16) == f16_bits(float(x)), x


def test_round_ieee_f16_ties_brute_force():
    # exact midpoints between neighbouring binary16 values go to the even pattern
    h = np.arange(0x0000, 0x7C00, 97, dtype=np.uint16)
    for b in h:
        lo = float(np.array([b], np.uint16).view(np.float16)[0])
        hi = float(np.array([b + 1], np.uint16).view(np.float16)[0])
        mid = (lo + hi) / 2                                   # exact in double
        want = int(b) if b % 2 == 0 else int(b) + 1
        if b + 1 == 0x7C00:
            want = 0x7C00                                      # max + half ulp overflows
        assert oracle.round_ieee_f64(mid, F16) == want, hex(b)
        assert oracle.round_ieee_f64(-mid, F16) == want | 0x8000


def test_round_ieee_f32_bf16_agree_with_pinned_rounding():
    rng = np.random.default_rng(6)
    xs = rng.standard_normal(5000) * 10.0 ** rng.uniform(-40, 38, 5000)
    for x in xs:
        assert oracle.round_ieee_f64(float(x), F32) == int(np.array([x]).astype(np.float32).view(np.uint32)[0])
        assert oracle.round_ieee_f64(float(x), BF16) == oracle.round_f64(float(x), BF16)


# ---------------------------------------------------------------- mixed-format GEMM
def all_codes(rng, shape, fmt):
    """Random codes of the format, NaN / Inf patterns replaced by 1.0."""
    q = rng.integers(0, 256, shape).astype(np.uint8)
    bad = ~np.isfinite(oracle.table(fmt)[q])
    q[bad] = 0x3C if fmt == E5M2 else 0x38
    return q


def brute_round(fr: Fraction, kind: int) -> int:
    """Nearest value of the output format to the exact rational fr, ties to
    the even pattern, by exact comparison among the neighbours of a float
    estimate; RNE overflow to infinity past max + half an ulp."""
    if kind == F16:
        dt, ut, maxbits, inf = np.float16, np.uint16, 0x7BFF, 0x7C00
    elif kind == F32:
        dt, ut, maxbits, inf = np.float32, np.uint32, 0x7F7FFFFF, 0x7F800000
    else:
        raise ValueError(kind)
    sign = 0x8000 if kind == F16 else 0x80000000
    neg = fr < 0
    a = -fr if neg else fr
    mx = Fraction(float(np.array([maxbits], ut).view(dt)[0]))
    ulp_top = mx - Fraction(float(np.array([maxbits - 1], ut).view(dt)[0]))
    if a >= mx + ulp_top / 2:
        best = inf
    else:
        est = int(np.array([min(float(a), float(mx))], np.float64).astype(dt).view(ut)[0])
        cands = [c for c in (est - 2, est - 1, est, est + 1, est + 2) if 0 <= c <= maxbits]
        best, bestd = None, None
        for c in cands:
            d = abs(Fraction(float(np.array([c], ut).view(dt)[0])) - a)
            if bestd is None or d < bestd or (d == bestd and c % 2 == 0):
                best, bestd = c, d
    return best | (sign if neg else 0)


@pytest.mark.parametrize("fa,fb", [(E4M3, E5M2), (E5M2, E4M3), (E5M2, E5M2), (E4M3, E4M3)])
@pytest.mark.parametrize("kind", [F32, F16])
def test_gemm_fmt_fraction_brute_force_tiny(fa, fb, kind):
    rng = np.random.default_rng(10 * fa + fb + 100 * kind)
    M, N, K = 3, 5, 7
    qa, qb = all_codes(rng, (M, K), fa), all_codes(rng, (K, N), fb)
    sa, sb = np.float32(0.0173), np.float32(3.91e-3) if kind == F16 else np.float32(2.5e-7)
    ta, tb = oracle.table(fa), oracle.table(fb)
    bits, exact, sab = oracle.gemm_rows_fmt(qa, qb, fa, fb, sa, sb, kind)
    for i in range(M):
        for j in range(N):
            d = sum(Fraction(float(ta[qa[i, k]])) * Fraction(float(tb[qb[k, j]])) for k in range(K))
            v = Fraction(float(sa)) * Fraction(float(sb)) * d
            if v == 0:
                continue                                         # sign of an exact zero: either
            assert int(bits[i, j]) == brute_round(v, kind), (i, j, float(v))
            assert abs(exact[i, j] - float(v)) <= 1e-15 * abs(float(v))
            s = sum(abs(Fraction(float(ta[qa[i, k]])) * Fraction(float(tb[qb[k, j]]))) for k in range(K))
            assert abs(sab[i, j] - float(s)) <= 1e-15 * float(s)


@pytest.mark.parametrize("kind", [F32, BF16])
def test_gemm_fmt_e4m3_equals_pinned_e4m3_path(kind):
    rng = np.random.default_rng(11)
    qa, qb = all_codes(rng, (40, 96), E4M3), all_codes(rng, (96, 33), E4M3)
    b1, x1, s1 = oracle.gemm_rows_fmt(qa, qb, E4M3, E4M3, 0.03, 0.7, kind)
    b2, x2, s2 = oracle.gemm_rows(qa, qb, 0.03, 0.7, kind)
    assert np.array_equal(b1, b2) and np.allclose(x1, x2, rtol=1e-15, atol=0) and np.array_equal(s1, s2)


@pytest.mark.parametrize("fa,fb", [(E4M3, E5M2), (E5M2, E4M3), (E5M2, E5M2)])
def test_gemm_fmt_vs_float64_matmul_on_a_narrow_range(fa, fb):
    """Codes with |v| in [2^-4, 2^4]: every partial sum is exact in float64,
    so numpy's matmul of the decoded operands is the exact sum (and the
    operand orientation is checked on a non-square shape)."""
    rng = np.random.default_rng(12)

    def narrow(shape, fmt):
        t = oracle.table(fmt)
        ok = np.nonzero(np.isfinite(t) & (np.abs(t) >= 2.0 ** -4) & (np.abs(t) <= 16))[0]
        return rng.choice(ok, size=shape).astype(np.uint8)

    qa, qb = narrow((9, 200), fa), narrow((200, 13), fb)
    _, exact, sab = oracle.gemm_rows_fmt(qa, qb, fa, fb, 1.0, 1.0, F32)
    A, B = oracle.table(fa)[qa], oracle.table(fb)[qb]
    assert np.array_equal(exact, A @ B)
    assert np.array_equal(sab, np.abs(A) @ np.abs(B))


def test_gemm_fmt_closed_forms():
    # identity B in E5M2 (0x3C = 1.0): C = sa*sb*A exactly representable in FP32
    rng = np.random.default_rng(13)
    qa = all_codes(rng, (6, 16), E4M3)
    eye = np.zeros((16, 16), np.uint8)
    eye[np.arange(16), np.arange(16)] = 0x3C
    bits, _, _ = oracle.gemm_rows_fmt(qa, eye, E4M3, E5M2, 0.5, 0.25, F32)
    assert np.array_equal(bits.view(np.float32), (oracle.decode(qa) * 0.125).astype(np.float32))
    # all-maximum E5M2 operands: K * 57344^2, and its FP16 overflow to +Inf
    K = 32
    qa = np.full((2, K), 0x7B, np.uint8)
    qb = np.full((K, 3), 0x7B, np.uint8)
    bits, exact, _ = oracle.gemm_rows_fmt(qa, qb, E5M2, E5M2, 1.0, 1.0, F32)
    assert np.all(exact == K * 57344.0 ** 2) and np.all(bits.view(np.float32) == np.float32(K * 57344.0 ** 2))
    b16, _, _ = oracle.gemm_rows_fmt(qa, qb, E5M2, E5M2, 1.0, 1.0, F16)
    assert np.all(b16 == 0x7C00)
    qb[:, 1] = 0xFB                                                 # -57344 -> -Inf
    b16, _, _ = oracle.gemm_rows_fmt(qa, qb, E5M2, E5M2, 1.0, 1.0, F16)
    assert np.all(b16[:, 1] == 0xFC00)
    # the smallest E5M2 subnormals: 2^-16 * 2^-16 products summed K times
    qa = np.full((1, K), 0x01, np.uint8)
    qb = np.full((K, 1), 0x01, np.uint8)
    _, exact, _ = oracle.gemm_rows_fmt(qa, qb, E5M2, E5M2, 1.0, 1.0, F32)
    assert exact[0, 0] == K * 2.0 ** -32


def test_gemm_fmt_rows_subset_and_transpose_sensitivity():
    rng = np.random.default_rng(14)
    qa, qb = all_codes(rng, (20, 48), E5M2), all_codes(rng, (48, 20), E4M3)
    full, _, _ = oracle.gemm_rows_fmt(qa, qb, E5M2, E4M3, 0.01, 0.02, F16)
    rows = np.array([19, 0, 7])
    sub, _, _ = oracle.gemm_rows_fmt(qa, qb, E5M2, E4M3, 0.01, 0.02, F16, rows=rows)
    assert np.array_equal(sub, full[rows])
    # swapping the formats of the operands changes the result (formats are per operand)
    other, _, _ = oracle.gemm_rows_fmt(qa, qb, E4M3, E5M2, 0.01, 0.02, F16)
    assert not np.array_equal(other, full)
