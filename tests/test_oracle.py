"""Pins of the CPU oracle against things other than itself.

Each test checks an oracle function against what the pages state (tests/golden),
a closed form, a library routine (torch's float8_e4m3fn and bfloat16 casts,
numpy's float64 -> float32 cast and float64 matmul), exact rational brute force
on tiny inputs, or an invariant -- chosen so that a dropped term, a wrong sign
or index, or a transposed operand in the oracle fails at least one of them.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_sat_cast(x: np.ndarray) -> np.ndarray:
    """Library routine: clamp to +-448, then torch's RNE cast to float8_e4m3fn."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ---------------------------------------------------------------- decode
def closed_form_e4m3(c: int) -> float:
    s = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * 2.0 ** (e - 7) * (1 + m / 8)


def test_decode_table_matches_closed_form_all_codes():
    t = oracle.e4m3_table()
    for c in range(256):
        ref = closed_form_e4m3(c)
        if np.isnan(ref):
            assert np.isnan(t[c]), c
        else:
            assert t[c] == ref and np.signbit(t[c]) == np.signbit(ref), (c, t[c], ref)


def test_decode_table_matches_torch_float8_e4m3fn():
    t = oracle.e4m3_table()
    ref = torch_e4m3_decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(t), nan)
    assert np.array_equal(t[~nan], ref[~nan])


def test_decode_invariants_and_page_constants():
    g = json.load(open(os.path.join(GOLDEN, "pages_constants.json")))
    t = oracle.e4m3_table()
    fin = t[~np.isnan(t)]
    assert list(np.nonzero(np.isnan(t))[0]) == [0x7F, 0xFF]        # NaN patterns only, no Inf
    assert fin.max() == g["e4m3_max_finite"] == t[0x7E]            # the pages' +-448
    assert fin.min() == -g["e4m3_max_finite"] == t[0xFE]
    assert len(np.unique(fin)) == 253                               # +0 and -0 coincide
    assert np.all(np.diff(t[0x00:0x7F]) > 0)                        # monotone in the code
    assert np.array_equal(t[0x80:0xFF], -t[0x00:0x7F])              # sign-magnitude
    assert np.all(fin * 512 == np.round(fin * 512))                 # multiples of 2^-9
    assert t[0x01] == 2.0 ** -9 and t[0x08] == 2.0 ** -6            # min subnormal / normal
    assert t[0x38] == 1.0


# ---------------------------------------------------------------- convert
def test_convert_exhaustive_all_fp32_patterns_vs_torch_cast():
    """Every one of the 2^32 binary32 bit patterns (NaNs excluded: outside the contract)."""
    chunk = 1 << 26
    for c0 in range(0, 1 << 32, chunk):
        bits = np.arange(c0, c0 + chunk, dtype=np.uint64).astype(np.uint32)
        x = bits.view(np.float32)
        keep = ~np.isnan(x)
        q = oracle.convert(x)
        ref = torch_sat_cast(x)
        bad = (q != ref) & keep
        assert not bad.any(), (c0, x[bad][:5], q[bad][:5], ref[bad][:5])


def brute_force_nearest_code(v: float) -> int:
    """Nearest finite E4M3 value by exact rational search over all 254 finite codes;
    ties to the even code; beyond +-448 the nearest finite value is +-448."""
    t = oracle.e4m3_table()
    fv = Fraction(float(v))
    best, bestd = None, None
    for c in range(256):
        if np.isnan(t[c]):
            continue
        if (c & 0x80) != (0x80 if np.signbit(v) else 0):
            continue
        d = abs(Fraction(float(t[c])) - fv)
        if bestd is None or d < bestd or (d == bestd and c % 2 == 0 and best % 2 == 1):
            best, bestd = c, d
    return best


def test_convert_brute_force_on_ties_and_neighbours():
    t = oracle.e4m3_table()
    mags = np.unique(np.abs(t[~np.isnan(t)]))
    vals = []
    for a, b in zip(mags[:-1], mags[1:]):
        mid = np.float32((a + b) / 2)        # midpoints are binary32-exact
        vals += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9)), np.float32(a)]
    vals += [np.float32(448), np.float32(464), np.float32(465), np.float32(1e30), np.float32(2.0 ** -10),
             np.float32(3 * 2.0 ** -10), np.float32(1e-45), np.float32(0.0)]
    vals = np.array(vals, np.float32)
    vals = np.concatenate([vals, -vals])
    for v in vals:
        assert oracle.e4m3_rne_sat(float(v)) == brute_force_nearest_code(float(v)), v


def test_convert_hand_cases():
    assert oracle.e4m3_rne_sat(2.0 ** -10) == 0x00      # tie between 0 and 2^-9 -> even (0)
    assert oracle.e4m3_rne_sat(-(2.0 ** -10)) == 0x80    # sign kept on zero
    assert oracle.e4m3_rne_sat(3 * 2.0 ** -10) == 0x02   # tie between 1 and 2 (x2^-9) -> 2
    assert oracle.e4m3_rne_sat(1.0625) == 0x38           # tie 1.0 / 1.125 -> 1.0
    assert oracle.e4m3_rne_sat(1.1875) == 0x3A           # tie 1.125 / 1.25 -> 1.25
    assert oracle.e4m3_rne_sat(464.0) == 0x7E            # saturates
    assert oracle.e4m3_rne_sat(1e30) == 0x7E and oracle.e4m3_rne_sat(-1e30) == 0xFE
    assert oracle.e4m3_rne_sat(float("inf")) == 0x7E


# ---------------------------------------------------------------- quantize
def test_amax_and_scale():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(100003) * 3).astype(np.float32)
    a = oracle.amax(x)
    assert a == np.abs(x).max()
    s = oracle.scale_from_amax(a)
    assert s == np.float32(a) / np.float32(448.0)          # one binary32 division (numpy)
    assert oracle.scale_from_amax(0.0) == 1.0
    assert oracle.scale_from_amax(448.0) == 1.0


def test_quantize_pertensor_double_rounding_reading():
    # fl32(x/s) is exactly 184 (a tie between 176 and 192 -> 192, even code) although the
    # exact quotient is just below 184 (single rounding would give 176).  The oracle takes
    # the binary32 quotient, as a binary32 value handed to an FP8 convert is.
    x = np.float32(1265.850341796875)
    s = np.float32(6.879621505737305)
    assert Fraction(float(x)) / Fraction(float(s)) < 184
    q = oracle.quantize_with_scale(np.array([x], np.float32), s)[0]
    assert oracle.e4m3_table()[q] == 192.0


def test_quantize_pertensor_vs_torch():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((97, 131)) * 11).astype(np.float32)
    q, s, a = oracle.quantize_pertensor(x)
    assert a == np.abs(x).max()
    assert s == np.float32(a) / np.float32(448)
    assert np.array_equal(q, torch_sat_cast(x / s))
    assert oracle.e4m3_table()[q].__abs__().max() == 448.0   # the amax element maps to 448


def test_quantize_zero_tensor():
    q, s, a = oracle.quantize_pertensor(np.zeros((4, 4), np.float32))
    assert a == 0 and s == 1.0 and not q.any()


def test_quantize_blocked_vs_numpy_tiles():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((96, 160))).astype(np.float32)
    x *= np.repeat(np.repeat(rng.uniform(0.01, 100, (3, 5)).astype(np.float32), 32, 0), 32, 1)
    x[32:64, 64:96] = 0.0                                       # one all-zero tile
    q, ts = oracle.quantize_blocked(x)
    tam = np.abs(x).reshape(3, 32, 5, 32).max(axis=(1, 3))
    sc = np.where(tam == 0, np.float32(1), tam / np.float32(448)).astype(np.float32)
    assert np.array_equal(ts, sc)
    assert ts[1, 2] == 1.0
    full = np.repeat(np.repeat(sc, 32, 0), 32, 1)
    assert np.array_equal(q, torch_sat_cast(x / full))


def test_quantize_blocked_equal_amax_reduces_to_pertensor():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((64, 64)).astype(np.float32)
    x[::32, ::32] = 7.5                                         # every tile has amax 7.5
    q1, ts = oracle.quantize_blocked(x)
    q2, s, _ = oracle.quantize_pertensor(x)
    assert np.all(ts == s) and np.array_equal(q1, q2)


def test_quantize_grouped():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((50, 24)) * np.arange(1, 51)[:, None]).astype(np.float32)
    off = np.array([0, 10, 10, 33, 50], np.int32)              # group 1 is empty
    q, s, a = oracle.quantize_grouped(x, off)
    assert s[1] == 1.0 and a[1] == 0.0
    for g in (0, 2, 3):
        qg, sg, ag = oracle.quantize_pertensor(x[off[g]:off[g + 1]])
        assert sg == s[g] and ag == a[g]
        assert np.array_equal(qg, q[off[g]:off[g + 1]])


# ---------------------------------------------------------------- rounding
def bf16_values_sorted():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ok = np.isfinite(v) & (bits < 0x8000)                       # non-negative finite
    return v[ok], bits[ok]


def brute_round_bf16(x: Fraction) -> int:
    """Nearest BF16 to an exact rational by search over all BF16 values (torch decode); ties even."""
    vals, bits = bf16_values_sorted()
    s = 0x8000 if x < 0 else 0
    ax = abs(x)
    i = int(np.searchsorted(vals, float(ax)))
    best = None
    for j in range(max(0, i - 2), min(len(vals), i + 2)):
        d = abs(Fraction(float(vals[j])) - ax)
        if best is None or d < best[0] or (d == best[0] and bits[j] % 2 == 0):
            best = (d, int(bits[j]))
    # beyond the largest finite value by at least half a step: infinity
    maxv = Fraction(float(vals[-1]))
    if ax >= maxv + Fraction(2) ** (127 - 8):
        return s | 0x7F80
    return s | best[1]


def brute_round_f32(x: Fraction) -> int:
    f = np.float32(float(x))
    cands = [f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))]
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        d = abs(Fraction(float(c)) - x)
        b = int(np.array(c, np.float32).view(np.uint32))
        if best is None or d < best[0] or (d == best[0] and b % 2 == 0):
            best = (d, b)
    return best[1]


def test_round_f64_to_f32_matches_numpy_cast():
    rng = np.random.default_rng(12)
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-160, 140, 20000))
    x = np.concatenate([x, [1e-50, 3e38, 3.5e38, 1.401298464324817e-45 * 0.5000001, 0.0, -0.0]])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float32).view(np.uint32)
    got = np.array([oracle.round_f64(v, oracle.F32) for v in x], np.uint32)
    assert np.array_equal(got, ref)


def test_round_f64_to_bf16_brute_force():
    rng = np.random.default_rng(13)
    x = list(rng.standard_normal(3000) * np.exp2(rng.integers(-130, 120, 3000)))
    # near-ties: BF16 midpoints and their double neighbours
    for m in rng.integers(0x3F00, 0x4100, 200):
        lo = float(torch.tensor([m], dtype=torch.int16).view(torch.bfloat16).float())
        hi = float(torch.tensor([m + 1], dtype=torch.int16).view(torch.bfloat16).float())
        mid = (lo + hi) / 2
        x += [mid, np.nextafter(mid, 0), np.nextafter(mid, 10), -mid]
    x += [1 + 2 ** -8 + 2 ** -30]   # a double-rounding trap: exact RNE gives 1 + 2^-7
    for v in x:
        assert oracle.round_f64(v, oracle.BF16) == brute_round_bf16(Fraction(v)), v
    assert oracle.round_f64(1 + 2 ** -8 + 2 ** -30, oracle.BF16) == 0x3F81


def test_round_scaled_exact_vs_fraction():
    rng = np.random.default_rng(14)
    for _ in range(3000):
        sa = np.float32(rng.uniform(0.5, 2) * 2.0 ** rng.integers(-20, 5))
        sb = np.float32(rng.uniform(0.5, 2) * 2.0 ** rng.integers(-20, 5))
        d = int(rng.integers(-(2 ** 52), 2 ** 52)) >> int(rng.integers(0, 50))
        exact = Fraction(float(sa)) * Fraction(float(sb)) * d / 2 ** 18
        assert oracle.round_scaled(d, sa, sb, oracle.F32) == brute_round_f32(exact)
        assert oracle.round_scaled(d, sa, sb, oracle.BF16) == brute_round_bf16(exact)


def test_round_scaled_f32_exact_values_match_torch_bf16_cast():
    # when sa*sb*d*2^-18 is a binary32 number, rounding it to BF16 is torch's RNE cast
    rng = np.random.default_rng(15)
    d = rng.integers(-(2 ** 24), 2 ** 24, 5000)
    f = (d.astype(np.float64) * 2.0 ** -18).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.round_scaled(int(v), 1.0, 1.0, oracle.BF16) for v in d], np.uint16)
    assert np.array_equal(got, ref)
    got32 = np.array([oracle.round_scaled(int(v), 1.0, 1.0, oracle.F32) for v in d], np.uint32)
    assert np.array_equal(got32, f.view(np.uint32))


# ---------------------------------------------------------------- GEMM
def all_code_matrix(rng, shape):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38                                # no NaN codes in GEMM inputs
    return c


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (8, 4, 16), (17, 9, 33), (64, 48, 40)])
def test_gemm_integer_loop_vs_numpy_float64_matmul(M, N, K):
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    qa, qb = all_code_matrix(rng, (M, K)), all_code_matrix(rng, (K, N))
    D = oracle.gemm_dot_i64(qa, qb)
    ref = oracle.decode(qa) @ oracle.decode(qb)                  # float64 matmul: exact here
    assert np.array_equal(D.astype(np.float64) * 2.0 ** -18, ref)
    dot, sab = oracle.gemm_rows_f64(qa, qb)
    assert np.array_equal(dot, ref)
    assert np.array_equal(sab, np.abs(oracle.decode(qa)) @ np.abs(oracle.decode(qb)))


def test_gemm_fraction_brute_force_tiny():
    rng = np.random.default_rng(16)
    qa, qb = all_code_matrix(rng, (2, 3)), all_code_matrix(rng, (3, 4))
    t = oracle.e4m3_table()
    sa, sb = np.float32(0.0137), np.float32(3.7)
    bits, exact, _ = oracle.gemm_rows(qa, qb, sa, sb, oracle.F32)
    for i in range(2):
        for j in range(4):
            v = sum(Fraction(float(t[qa[i, k]])) * Fraction(float(t[qb[k, j]])) for k in range(3))
            v *= Fraction(float(sa)) * Fraction(float(sb))
            assert bits[i, j] == brute_round_f32(v)


def test_gemm_closed_forms():
    rng = np.random.default_rng(17)
    K, N = 96, 40
    qb = all_code_matrix(rng, (K, N))
    ones = np.full((3, K), 0x38, np.uint8)                      # every a = 1.0
    dot, _ = oracle.gemm_rows_f64(ones, qb)
    assert np.array_equal(dot[1], oracle.decode(qb).sum(axis=0))
    neg = np.full((1, K), 0xB8, np.uint8)                       # every a = -1.0
    dotn, _ = oracle.gemm_rows_f64(neg, qb)
    assert np.array_equal(dotn[0], -oracle.decode(qb).sum(axis=0))
    # identity B (code 0x38 on the diagonal): C = sa*sb*A
    qa = all_code_matrix(rng, (5, 32))
    eye = np.zeros((32, 32), np.uint8)
    eye[np.arange(32), np.arange(32)] = 0x38
    sa, sb = np.float32(0.25), np.float32(0.5)
    bits, _, _ = oracle.gemm_rows(qa, eye, sa, sb, oracle.F32)
    assert np.array_equal(bits.view(np.float32), (oracle.decode(qa) * 0.125).astype(np.float32))


def test_gemm_not_transposed():
    # non-square: a transposed operand cannot even produce the right shape/values
    rng = np.random.default_rng(18)
    qa, qb = all_code_matrix(rng, (6, 10)), all_code_matrix(rng, (10, 3))
    bits, exact, _ = oracle.gemm_rows(qa, qb, 1.0, 1.0, oracle.F32)
    assert bits.shape == (6, 3)
    assert np.array_equal(exact, oracle.decode(qa) @ oracle.decode(qb))


@pytest.mark.parametrize("kind", [0, 1])
def test_gemm_rows_rounding_and_sampled_agree(kind):
    rng = np.random.default_rng(19 + kind)
    qa, qb = all_code_matrix(rng, (20, 64)), all_code_matrix(rng, (64, 12))
    sa, sb = np.float32(0.011), np.float32(0.0031)
    bits, exact, sab = oracle.gemm_rows(qa, qb, sa, sb, kind)
    D = oracle.gemm_dot_i64(qa, qb)
    for i in range(20):
        for j in range(12):
            assert bits[i, j] == oracle.round_scaled(int(D[i, j]), sa, sb, kind)
    ii = rng.integers(0, 20, 50)
    jj = rng.integers(0, 12, 50)
    b2, e2, s2 = oracle.gemm_sampled(qa, qb, sa, sb, kind, ii, jj)
    assert np.array_equal(b2, bits[ii, jj].astype(np.uint32))
    assert np.array_equal(e2, exact[ii, jj]) and np.array_equal(s2, sab[ii, jj])
    rows = np.array([19, 0, 7])
    b3, _, _ = oracle.gemm_rows(qa, qb, sa, sb, kind, rows=rows)
    assert np.array_equal(b3, bits[rows])


def test_gemm_exact_for_long_k():
    # K = 8192 with all-max codes: the largest sums the workloads can reach stay exact in FP64
    K = 8192
    qa = np.full((1, K), 0x7E, np.uint8)
    qb = np.full((K, 2), 0x7E, np.uint8)
    qb[::2, 1] = 0xFE
    dot, sab = oracle.gemm_rows_f64(qa, qb)
    assert dot[0, 0] == K * 448.0 * 448.0 and dot[0, 1] == 0.0 and sab[0, 1] == K * 448.0 * 448.0


# ---------------------------------------------------------------- block-scaled
def test_blockscaled_power_of_two_scales_reduce_to_pertensor():
    rng = np.random.default_rng(20)
    M, N, K = 64, 96, 128
    qa, qb = all_code_matrix(rng, (M, K)), all_code_matrix(rng, (K, N))
    s_a = np.full((M // 32, K // 32), 2.0 ** -3, np.float32)
    s_b = np.full((K // 32, N // 32), 2.0 ** -5, np.float32)
    for kind in (0, 1):
        b1, _, _ = oracle.gemm_blockscaled_rows(qa, qb, s_a, s_b, kind)
        b2, _, _ = oracle.gemm_rows(qa, qb, 2.0 ** -3, 2.0 ** -5, kind)
        assert np.array_equal(b1, b2)


def test_blockscaled_fraction_brute_force():
    rng = np.random.default_rng(21)
    M = N = K = 64
    qa, qb = all_code_matrix(rng, (M, K)), all_code_matrix(rng, (K, N))
    s_a = (10.0 ** rng.uniform(-2, 2, (2, 2)) / 448).astype(np.float32)
    s_b = (10.0 ** rng.uniform(-2, 2, (2, 2)) / 448).astype(np.float32)
    bits, c64, sab = oracle.gemm_blockscaled_rows(qa, qb, s_a, s_b, oracle.BF16)
    t = oracle.e4m3_table()
    A = [[Fraction(float(t[v])) for v in row] for row in qa]
    B = [[Fraction(float(t[v])) for v in row] for row in qb]
    for (i, j) in [(0, 0), (5, 40), (33, 7), (63, 63), (40, 33), (17, 50)]:
        v = Fraction(0)
        for kb in range(2):
            p = sum(A[i][k] * B[k][j] for k in range(kb * 32, kb * 32 + 32))
            v += Fraction(float(s_a[i // 32, kb])) * Fraction(float(s_b[kb, j // 32])) * p
        assert bits[i, j] == brute_round_bf16(v), (i, j)
        assert abs(Fraction(float(c64[i, j])) - v) <= abs(v) * Fraction(1, 2 ** 45)
    # numpy float64 formulation of the same definition
    da, db = oracle.decode(qa), oracle.decode(qb)
    ref = sum(np.repeat(s_a[:, kb], 32)[:, None].astype(np.float64) * (da[:, kb * 32:(kb + 1) * 32] @ db[kb * 32:(kb + 1) * 32])
              * np.repeat(s_b[kb], 32)[None, :].astype(np.float64) for kb in range(2))
    assert np.allclose(c64, ref, rtol=1e-12, atol=1e-300)


# ---------------------------------------------------------------- grouped
def test_grouped_reduces_to_per_expert_gemms_and_handles_empty_expert():
    rng = np.random.default_rng(22)
    T, K, N, E = 40, 64, 24, 4
    qx = all_code_matrix(rng, (T, K))
    qw = np.stack([all_code_matrix(rng, (K, N)) for _ in range(E)])
    off = np.array([0, 13, 13, 30, 40])
    sx = np.array([0.5, 1.0, 0.02, 0.7], np.float32)
    sw = np.array([0.01, 1.0, 0.3, 0.004], np.float32)
    bits, exact, _ = oracle.grouped_gemm_rows(qx, qw, off, sx, sw, oracle.BF16)
    for e in range(E):
        if off[e + 1] == off[e]:
            continue
        b, _, _ = oracle.gemm_rows(qx[off[e]:off[e + 1]], qw[e], sx[e], sw[e], oracle.BF16)
        assert np.array_equal(bits[off[e]:off[e + 1]], b)
    # one expert covering all rows is the plain per-tensor GEMM
    b1, _, _ = oracle.grouped_gemm_rows(qx, qw[:1], [0, T], sx[:1], sw[:1], oracle.F32)
    b2, _, _ = oracle.gemm_rows(qx, qw[0], sx[0], sw[0], oracle.F32)
    assert np.array_equal(b1, b2)


def test_gemm_rows_rejects_fp16_output():
    # gemm_rows rounds to FP32 or BF16; FP16 output goes through gemm_rows_fmt
    q = np.zeros((2, 16), np.uint8)
    with pytest.raises(ValueError):
        oracle.gemm_rows(q, q.T.copy(), 1.0, 1.0, oracle.F16)


def test_gemm_blockscaled_rows_rejects_fp16_output():
    q = np.zeros((32, 32), np.uint8)
    sc = np.ones((1, 1), np.float32)
    with pytest.raises(ValueError):
        oracle.gemm_blockscaled_rows(q, q, sc, sc, oracle.F16)
