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
per-expert scales."""
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


@pytest.mark.parametrize("case", range(100))
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


@pytest.mark.parametrize("case", range(30))
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
