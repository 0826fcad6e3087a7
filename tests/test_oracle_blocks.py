"""Pins of the oracle's block-scale granularity parameter (32x32 or 64x64
tiles: "FP8 GEMM in JAX with Triton for Blackwell", parameter paragraph and
its monitoring paragraph's coarser 64x64 granularity), against the pinned
32x32 functions, numpy / torch per-tile quantization, exact rational brute
force and closed-form reductions."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

F32, BF16, F16 = oracle.F32, oracle.BF16, oracle.F16


def tiled_input(rows, cols, T, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    f = np.power(10.0, rng.uniform(-2, 2, (rows // T, cols // T))).astype(np.float32)
    return x * np.kron(f, np.ones((T, T), np.float32))


def test_quantize_t32_equals_pinned_blocked():
    x = tiled_input(96, 160, 32, 1)
    q, s = oracle.quantize_blocked_t(x, 32)
    rq, rs = oracle.quantize_blocked(x)
    assert np.array_equal(q, rq) and np.array_equal(s, rs)


def test_quantize_t64_vs_numpy_tiles_and_torch_cast():
    x = tiled_input(128, 192, 64, 2)
    q, s = oracle.quantize_blocked_t(x, 64)
    assert s.shape == (2, 3)
    for bi in range(2):
        for bj in range(3):
            tile = x[bi * 64:(bi + 1) * 64, bj * 64:(bj + 1) * 64]
            amax = np.float32(np.abs(tile).max())
            assert s[bi, bj] == amax / np.float32(448.0)
            ref = torch.from_numpy(tile / s[bi, bj]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(q[bi * 64:(bi + 1) * 64, bj * 64:(bj + 1) * 64], ref)


@pytest.mark.parametrize("kind", [F32, BF16])
def test_gemm_t32_equals_pinned_blockscaled(kind):
    a, b = tiled_input(64, 96, 32, 3), tiled_input(96, 128, 32, 4)
    qa, sa = oracle.quantize_blocked(a)
    qb, sb = oracle.quantize_blocked(b)
    b1, x1, s1 = oracle.gemm_blockscaled_rows_t(qa, qb, sa, sb, 32, kind)
    b2, x2, s2 = oracle.gemm_blockscaled_rows(qa, qb, sa, sb, kind)
    assert np.array_equal(b1, b2) and np.array_equal(x1, x2) and np.array_equal(s1, s2)


@pytest.mark.parametrize("kind", [F32, F16])
def test_gemm_t64_fraction_brute_force(kind):
    a, b = tiled_input(128, 192, 64, 5), tiled_input(192, 128, 64, 6)
    qa, sa = oracle.quantize_blocked_t(a, 64)
    qb, sb = oracle.quantize_blocked_t(b, 64)
    rows = np.array([0, 63, 64, 127])
    bits, exact, sab = oracle.gemm_blockscaled_rows_t(qa, qb, sa, sb, 64, kind, rows=rows)
    t = oracle.e4m3_table()
    for r, i in enumerate(rows):
        for j in (0, 1, 63, 64, 100, 127):
            v = Fraction(0)
            sv = Fraction(0)
            for kb in range(3):
                s = Fraction(float(sa[i // 64, kb])) * Fraction(float(sb[kb, j // 64]))
                p = sum(Fraction(float(t[qa[i, k]])) * Fraction(float(t[qb[k, j]])) for k in range(kb * 64, kb * 64 + 64))
                pa = sum(abs(Fraction(float(t[qa[i, k]])) * Fraction(float(t[qb[k, j]]))) for k in range(kb * 64, kb * 64 + 64))
                v += s * p
                sv += s * pa
            assert abs(exact[r, j] - float(v)) <= 1e-14 * float(sv)
            assert abs(sab[r, j] - float(sv)) <= 1e-14 * float(sv)
            assert int(bits[r, j]) == oracle.round_ieee_f64(exact[r, j], kind)


def test_gemm_t64_unit_scales_reduce_to_plain_gemm():
    rng = np.random.default_rng(7)
    qa = rng.integers(0, 256, (64, 128)).astype(np.uint8)
    qb = rng.integers(0, 256, (128, 192)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x38
    qb[(qb & 0x7F) == 0x7F] = 0x38
    ones_a = np.ones((1, 2), np.float32)
    ones_b = np.ones((2, 3), np.float32)
    bits, exact, _ = oracle.gemm_blockscaled_rows_t(qa, qb, ones_a, ones_b, 64, F32)
    rbits, rexact, _ = oracle.gemm_rows(qa, qb, 1.0, 1.0, F32)
    assert np.array_equal(exact, rexact) and np.array_equal(bits, rbits)


def test_gemm_t64_equals_t32_with_expanded_scales():
    """64x64 scales expanded to their four 32x32 sub-tiles give the same sum
    through the 32-deep-block function (up to FP64 summation order)."""
    a, b = tiled_input(128, 128, 64, 8), tiled_input(128, 192, 64, 9)
    qa, sa = oracle.quantize_blocked_t(a, 64)
    qb, sb = oracle.quantize_blocked_t(b, 64)
    _, x64, s64 = oracle.gemm_blockscaled_rows_t(qa, qb, sa, sb, 64, F32)
    e = np.ones((2, 2), np.float32)
    _, x32, s32 = oracle.gemm_blockscaled_rows_t(qa, qb, np.kron(sa, e), np.kron(sb, e), 32, F32)
    assert np.all(np.abs(x64 - x32) <= 1e-14 * s64)
    assert np.allclose(s64, s32, rtol=1e-14, atol=0)
