"""A seeded sweep of random GEMM shapes across the dispatch's class
boundaries, through the C ABI, bit for bit against the oracle.

Each case draws M (1 to 1500, weighted towards the class edges 16, 64 and
1024), N and K (multiples of 16), the two operand formats, the output type,
the accumulation mode and whether a split-K workspace is given; the codes
are small integers (|v| <= 8, exact in both formats), so every partial sum
is an integer below 2^24 and any summation order gives the oracle's value:
the GPU must match it bit for bit whichever tile class, split or skinny
path the shape lands on.  Also: the same call twice gives the same bits
(determinism), and no output outside C is touched (a guard row after C).
The grouped (MoE) form likewise: random expert counts (empty experts
included, rows per expert across the class edges), random K and N, unit
per-expert scales; and the block-scaled (power-of-two FP32 tile scales,
32 or 64 tiles), E8M0 and 2:4-sparse GEMMs on random shapes of their
granularity; and attention on random head counts, sequence lengths, head
dimensions, masks, modes and output types, within the bound its header
states (tests/test_gpu_attention.py)."""
import numpy as np
import pytest
import torch

import oracle
import precision_dense_linear_amd as P
from parity import to_bits

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
E4M3, E5M2 = oracle.E4M3, oracle.E5M2
NAME = {E4M3: "e4m3", E5M2: "e5m2"}
OUT = {oracle.F32: torch.float32, oracle.BF16: torch.bfloat16, oracle.F16: torch.float16}
EDGES = [1, 15, 16, 17, 31, 63, 64, 65, 127, 128, 129, 255, 1023, 1024, 1025]


def int_codes(shape, rng, fmt, lim=8):
    v = rng.integers(-lim, lim + 1, shape).astype(np.float32)
    dt = torch.float8_e5m2 if fmt == E5M2 else torch.float8_e4m3fn
    return torch.from_numpy(v).to(dt).view(torch.uint8).numpy()


def draw(i):
    rng = np.random.default_rng(1000 + i)
    M = int(rng.choice(EDGES)) if rng.random() < 0.5 else int(rng.integers(1, 1501))
    N = 16 * int(rng.integers(1, 300))
    K = 16 * int(rng.integers(0, 160))
    # keep each case's exact check and oracle time small
    while M * N * K > 1 << 30:
        K //= 2
        K -= K % 16
    fa, fb = (E4M3, E5M2)[int(rng.integers(0, 2))], (E4M3, E5M2)[int(rng.integers(0, 2))]
    kind = (oracle.F32, oracle.BF16, oracle.F16)[int(rng.integers(0, 3))]
    return M, N, K, fa, fb, kind, bool(rng.integers(0, 2)), bool(rng.integers(0, 2)), rng


@pytest.mark.parametrize("case", range(400))
def test_random_shape_bit_for_bit(case):
    M, N, K, fa, fb, kind, fast, ws, rng = draw(case)
    print("case %d: %dx%dx%d %s x %s kind %d fast=%s ws=%s" % (case, M, N, K, NAME[fa], NAME[fb], kind, fast, ws),
          flush=True)
    qa, qb = int_codes((M, K), rng, fa), int_codes((K, N), rng, fb)
    A, B = torch.from_numpy(qa).to(DEV), torch.from_numpy(qb).to(DEV)
    one = torch.ones(1, device=DEV)
    work = P.gemm_workspace(DEV) if ws else None
    # C is the first M rows of a buffer with one guard row after it
    buf = torch.full((M + 1, N), 7.0, dtype=OUT[kind], device=DEV)
    C = buf[:M]
    P.fp8_gemm(A, B, one, one, OUT[kind], C=C, a_fmt=NAME[fa], b_fmt=NAME[fb], workspace=work, fast=fast)
    first = to_bits(C)
    P.fp8_gemm(A, B, one, one, OUT[kind], C=C, a_fmt=NAME[fa], b_fmt=NAME[fb], workspace=work, fast=fast)
    again = to_bits(C)
    assert np.array_equal(first, again), "not deterministic"
    assert torch.all(buf[M] == 7.0).item(), "wrote past C"
    bits, exact, _ = oracle.gemm_rows_fmt(qa, qb, fa, fb, 1.0, 1.0, kind)
    assert np.abs(exact).max(initial=0.0) < 2 ** 24
    assert np.array_equal(first, bits), "%d of %d outputs differ" % (int((first != bits).sum()), first.size)


@pytest.mark.parametrize("case", range(120))
def test_random_grouped_bit_for_bit(case):
    rng = np.random.default_rng(5000 + case)
    E = int(rng.integers(1, 13))
    per = int(rng.choice([8, 40, 100, 700, 1500]))
    counts = rng.integers(0, 2 * per + 1, E)
    counts[rng.random(E) < 0.15] = 0
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    T = int(off[-1])
    N = 16 * int(rng.integers(1, 100))
    K = 16 * int(rng.integers(1, 64))
    while T * N * K > 1 << 30 and K > 16:   # keep the oracle's share of the case small
        K = max(16, (K // 2) - (K // 2) % 16)
    while T * N * K > 1 << 30 and N > 16:
        N = max(16, (N // 2) - (N // 2) % 16)
    kind = (oracle.F32, oracle.BF16)[int(rng.integers(0, 2))]
    fast = bool(rng.integers(0, 2))
    print("grouped case %d: E=%d T=%d N=%d K=%d kind %d fast=%s counts %s" % (case, E, T, N, K, kind, fast,
                                                                            counts.tolist()), flush=True)
    qx, qw = int_codes((T, K), rng, E4M3), int_codes((E, K, N), rng, E4M3)
    ones = torch.ones(E, device=DEV)
    buf = torch.full((T + 1, N), 7.0, dtype=OUT[kind], device=DEV)
    C = buf[:T]
    P.fp8_grouped_gemm(torch.from_numpy(qx).to(DEV), torch.from_numpy(qw).to(DEV), torch.from_numpy(
        off.astype(np.int32)).to(DEV), ones, ones, OUT[kind], C=C, fast=fast)
    got = to_bits(C)
    assert torch.all(buf[T] == 7.0).item(), "wrote past C"
    if T == 0:
        return
    bits, exact, _ = oracle.grouped_gemm_rows(qx, qw, off, np.ones(E, np.float32), np.ones(E, np.float32), kind,
                                              rows=np.arange(T))
    assert np.abs(exact).max(initial=0.0) < 2 ** 24
    assert np.array_equal(got, bits), "%d of %d outputs differ" % (int((got != bits).sum()), got.size)


def pot_scales(shape, rng, lo=0, hi=3):
    """Power-of-two tile scales 2^e, e in [lo, hi]: with small-integer codes
    every scaled partial sum stays an integer below 2^24 (exact in FP32)."""
    return np.ldexp(1.0, rng.integers(lo, hi + 1, shape)).astype(np.float32)


@pytest.mark.parametrize("case", range(60))
def test_random_blockscaled_bit_for_bit(case):
    rng = np.random.default_rng(7000 + case)
    T = (32, 64)[int(rng.integers(0, 2))]
    M, N, K = (T * int(rng.integers(1, n)) for n in (40 if T == 32 else 20, 40 if T == 32 else 20,
                                                     32 if T == 32 else 16))
    kind = (oracle.F32, oracle.BF16, oracle.F16)[int(rng.integers(0, 3))]
    print("block-scaled case %d: T=%d %dx%dx%d kind %d" % (case, T, M, N, K, kind), flush=True)
    qa, qb = int_codes((M, K), rng, E4M3), int_codes((K, N), rng, E4M3)
    sa, sb = pot_scales((M // T, K // T), rng), pot_scales((K // T, N // T), rng)
    C = P.fp8_gemm_blockscaled(torch.from_numpy(qa).to(DEV), torch.from_numpy(qb).to(DEV),
                               torch.from_numpy(sa).to(DEV), torch.from_numpy(sb).to(DEV), OUT[kind], block=T)
    bits, exact, _ = oracle.gemm_blockscaled_rows_t(qa, qb, sa, sb, T, kind)
    assert np.abs(exact).max(initial=0.0) < 2 ** 24
    got = to_bits(C)
    assert np.array_equal(got, bits), "%d of %d outputs differ" % (int((got != bits).sum()), got.size)


def k_major_exps(e):
    """[tiles_mn, K/32] exponent bytes -> the library's [K/32, pitch(tiles_mn)] layout (padding 127)."""
    t, kb = e.shape
    out = np.full((kb, (t + 3) // 4 * 4), 127, np.uint8)
    out[:, :t] = e.T
    return out


@pytest.mark.parametrize("case", range(60))
def test_random_e8m0_bit_for_bit(case):
    rng = np.random.default_rng(8000 + case)
    M, N, K = (32 * int(rng.integers(1, n)) for n in (40, 40, 32))
    kind = (oracle.F32, oracle.BF16, oracle.F16)[int(rng.integers(0, 3))]
    print("E8M0 case %d: %dx%dx%d kind %d" % (case, M, N, K, kind), flush=True)
    qa, qb = int_codes((M, K), rng, E4M3), int_codes((K, N), rng, E4M3)
    ea = rng.integers(127, 130, (M // 32, K // 32)).astype(np.uint8)     # 2^0 .. 2^2
    eb = rng.integers(127, 130, (K // 32, N // 32)).astype(np.uint8)
    C = P.fp8_gemm_blockscaled_e8m0(torch.from_numpy(qa).to(DEV), torch.from_numpy(qb).to(DEV),
                                    torch.from_numpy(k_major_exps(ea)).to(DEV),
                                    torch.from_numpy(k_major_exps(eb.T.copy())).to(DEV), OUT[kind])
    bits, exact, _ = oracle.gemm_blockscaled_e8m0_rows(qa, qb, ea, eb, kind)
    assert np.abs(exact).max(initial=0.0) < 2 ** 24
    got = to_bits(C)
    assert np.array_equal(got, bits), "%d of %d outputs differ" % (int((got != bits).sum()), got.size)


@pytest.mark.parametrize("case", range(60))
def test_random_sparse24_bit_for_bit(case):
    rng = np.random.default_rng(9000 + case)
    M = int(rng.choice(EDGES)) if rng.random() < 0.5 else int(rng.integers(1, 1501))
    N, K = 16 * int(rng.integers(1, 150)), 32 * int(rng.integers(1, 40))
    kind = (oracle.F32, oracle.BF16)[int(rng.integers(0, 2))]
    print("sparse case %d: %dx%dx%d kind %d" % (case, M, N, K, kind), flush=True)
    qa, qb = int_codes((M, K), rng, E4M3), int_codes((K, N), rng, E4M3)
    # 2:4 along K: zero two random entries of every group of 4 (code 0x00)
    g = qb.reshape(K // 4, 4, N)
    drop = np.argsort(rng.random((K // 4, 4, N)), axis=1)[:, :2, :]
    np.put_along_axis(g, drop, 0, axis=1)
    qb = g.reshape(K, N)
    vals, idx = oracle.compress_2of4(qb)
    one = torch.ones(1, device=DEV)
    C = P.fp8_gemm_sparse24(torch.from_numpy(qa).to(DEV), torch.from_numpy(vals).to(DEV),
                            torch.from_numpy(idx.view(np.int32)).to(DEV), one, one, OUT[kind])
    bits, exact, _ = oracle.gemm_rows(qa, qb, 1.0, 1.0, kind)
    assert np.abs(exact).max(initial=0.0) < 2 ** 24
    got = to_bits(C)
    assert np.array_equal(got, bits), "%d of %d outputs differ" % (int((got != bits).sum()), got.size)


@pytest.mark.parametrize("case", range(40))
def test_random_attention_within_bound(case):
    from test_gpu_attention import run_case   # the header's bound, against the float64 oracle
    rng = np.random.default_rng(11000 + case)
    BH = int(rng.integers(1, 6))
    Sq, Skv = int(rng.integers(1, 700)), int(rng.integers(1, 900))
    D = (64, 128)[int(rng.integers(0, 2))]
    causal, fast = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    out = (torch.float32, torch.bfloat16, torch.float16)[int(rng.integers(0, 3))]
    print("attention case %d: BH=%d Sq=%d Skv=%d D=%d causal=%s fast=%s %s" % (case, BH, Sq, Skv, D, causal, fast, out),
          flush=True)
    run_case(BH, Sq, Skv, D, causal, out, seed=12000 + case, fast=fast)
