"""Pins of the oracle's power-of-two (E8M0) 32x32 block scales ("FP8 GEMM in
JAX with Triton for Blackwell", parameter paragraph: 32x32 microscaling;
shared exponents as the OCP MX conversion defines them), against the
defining inequality of the shared exponent, torch's saturating E4M3 cast,
the pinned FP32-scale block-scaled GEMM and rational brute force."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

F32, BF16, F16 = oracle.F32, oracle.BF16, oracle.F16


def test_e8m0_exponent_defining_inequality_and_clamps():
    rng = np.random.default_rng(1)
    vals = np.concatenate([np.float32(10.0) ** rng.uniform(-37, 38, 3000).astype(np.float32),
                           np.float32(2.0) ** np.arange(-126, 128).astype(np.float32),
                           np.array([448.0, 447.99997, 256.0, 255.99998, 1.0, 0.9999999], np.float32)])
    for a in vals.astype(np.float32):
        e = oracle.e8m0_exponent(float(a))
        lo, hi = Fraction(2) ** (e + 8), Fraction(2) ** (e + 9)
        if -127 < e < 127:
            assert lo <= Fraction(float(a)) < hi, (a, e)
        elif e == -127:
            assert Fraction(float(a)) < Fraction(2) ** (-127 + 9)
    assert oracle.e8m0_exponent(0.0) == 0
    assert oracle.e8m0_exponent(1e-45) == -127                      # subnormal amax: clamped
    assert oracle.e8m0_exponent(3.0e38) == 119                      # floor(log2) = 127


def test_quantize_blocked_e8m0_vs_torch_cast():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((96, 128)).astype(np.float32)
    x *= np.kron(np.float32(10.0) ** rng.uniform(-30, 30, (3, 4)).astype(np.float32), np.ones((32, 32), np.float32))
    x[32:64, 64:96] = 0.0
    q, sc = oracle.quantize_blocked_e8m0(x)
    assert sc[1, 2] == 127 and not q[32:64, 64:96].any()
    for bi in range(3):
        for bj in range(4):
            tile = x[bi * 32:(bi + 1) * 32, bj * 32:(bj + 1) * 32]
            e = int(sc[bi, bj]) - 127
            assert e == oracle.e8m0_exponent(float(np.abs(tile).max()))
            y = torch.from_numpy(tile.astype(np.float64) * 2.0 ** -e).float()   # exact: power of two
            ref = y.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(q[bi * 32:(bi + 1) * 32, bj * 32:(bj + 1) * 32], ref), (bi, bj)
            mags = np.abs(oracle.decode(q[bi * 32:(bi + 1) * 32, bj * 32:(bj + 1) * 32]))
            if np.abs(tile).max() > 0:
                assert 256 <= mags.max() <= 448                     # amax lands in [256, 448]


@pytest.mark.parametrize("kind", [F32, BF16])
def test_gemm_e8m0_equals_pinned_fp32_scale_path(kind):
    """E8M0 bytes b give the same sums as FP32 tile scales 2^(b-127) through
    the pinned block-scaled function (powers of two: every product exact)."""
    rng = np.random.default_rng(3)
    qa = rng.integers(0, 256, (64, 96)).astype(np.uint8)
    qb = rng.integers(0, 256, (96, 128)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x38
    qb[(qb & 0x7F) == 0x7F] = 0x38
    sa = rng.integers(100, 150, (2, 3)).astype(np.uint8)
    sb = rng.integers(100, 150, (3, 4)).astype(np.uint8)
    b1, x1, s1 = oracle.gemm_blockscaled_e8m0_rows(qa, qb, sa, sb, kind)
    fa = np.ldexp(1.0, sa.astype(np.int64) - 127).astype(np.float32)
    fb = np.ldexp(1.0, sb.astype(np.int64) - 127).astype(np.float32)
    b2, x2, s2 = oracle.gemm_blockscaled_rows(qa, qb, fa, fb, kind)
    assert np.array_equal(b1, b2) and np.array_equal(x1, x2) and np.array_equal(s1, s2)


def test_gemm_e8m0_fraction_brute_force():
    rng = np.random.default_rng(4)
    qa = rng.integers(0, 256, (64, 64)).astype(np.uint8)
    qb = rng.integers(0, 256, (64, 64)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x38
    qb[(qb & 0x7F) == 0x7F] = 0x38
    sa = rng.integers(90, 170, (2, 2)).astype(np.uint8)
    sb = rng.integers(90, 170, (2, 2)).astype(np.uint8)
    bits, exact, sab = oracle.gemm_blockscaled_e8m0_rows(qa, qb, sa, sb, F16)
    t = oracle.e4m3_table()
    for i in (0, 31, 32, 63):
        for j in (0, 31, 32, 63):
            v = sv = Fraction(0)
            for kb in range(2):
                s = Fraction(2) ** (int(sa[i // 32, kb]) + int(sb[kb, j // 32]) - 254)
                for k in range(kb * 32, kb * 32 + 32):
                    p = Fraction(float(t[qa[i, k]])) * Fraction(float(t[qb[k, j]]))
                    v += s * p
                    sv += s * abs(p)
            assert abs(exact[i, j] - float(v)) <= 1e-15 * float(sv)
            assert int(bits[i, j]) == oracle.round_ieee_f64(exact[i, j], F16)
