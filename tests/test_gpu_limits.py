"""Edge cases at the sizes the C ABI allows at most, through the C ABI,
against the oracle: K = 2^23, N = 2^20, 1024 experts, and a per-tensor
quantization of more than 2^31 elements (64-bit indexing)."""
import numpy as np
import pytest
import torch

import oracle
import precision_dense_linear_amd as P
from parity import to_bits

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def unit_codes(shape, seed, p_zero=0.3):
    """Codes of -1, 0, +1: every partial sum of K <= 2^23 products is an
    integer below 2^24, exact in FP32 in any order."""
    rng = np.random.default_rng(seed)
    v = rng.choice(np.array([0x38, 0x00, 0xB8], np.uint8), size=shape, p=[(1 - p_zero) / 2, p_zero, (1 - p_zero) / 2])
    return v


@pytest.mark.parametrize("fast", [False, True])
def test_max_k(fast):
    M, N, K = 33, 32, 1 << 23
    qa, qb = unit_codes((M, K), 1), unit_codes((K, N), 2)
    one = torch.ones(1, device=DEV)
    bits, exact, _ = oracle.gemm_rows(qa, qb, 1.0, 1.0, oracle.F32)
    assert np.abs(exact).max() < 2 ** 24
    for ws in (P.gemm_workspace(DEV), None):     # split over 8 workgroups, and unsplit
        C = P.fp8_gemm(gpu(qa), gpu(qb), one, one, torch.float32, fast=fast, workspace=ws)
        assert np.array_equal(to_bits(C), bits)


def test_k_beyond_max_rejected():
    A = torch.zeros((1, (1 << 23) + 16), dtype=torch.uint8, device=DEV)
    B = torch.zeros(((1 << 23) + 16, 16), dtype=torch.uint8, device=DEV)
    one = torch.ones(1, device=DEV)
    with pytest.raises(P.FP8Error):
        P.fp8_gemm(A, B, one, one, torch.float32)


def test_max_n():
    M, N, K = 16, 1 << 20, 64
    qa, qb = unit_codes((M, K), 3), unit_codes((K, N), 4)
    one = torch.ones(1, device=DEV)
    C = P.fp8_gemm(gpu(qa), gpu(qb), one, one, torch.bfloat16)
    bits, _, _ = oracle.gemm_rows(qa, qb, 1.0, 1.0, oracle.BF16)
    assert np.array_equal(to_bits(C), bits)


def test_1024_experts_most_empty():
    E, T, K, N = 1024, 3000, 64, 48
    rng = np.random.default_rng(5)
    counts = np.zeros(E, np.int64)
    counts[rng.choice(E, 40, replace=False)] = rng.multinomial(T, np.ones(40) / 40)
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(counts)
    qa = unit_codes((T, K), 6)
    qb = unit_codes((E, K, N), 7)
    sa = (2.0 ** rng.integers(-3, 4, E)).astype(np.float32)
    sb = (2.0 ** rng.integers(-3, 4, E)).astype(np.float32)
    C = P.fp8_grouped_gemm(gpu(qa), gpu(qb), gpu(off), gpu(sa), gpu(sb), torch.float32)
    bits, _, _ = oracle.grouped_gemm_rows(qa, qb, off, sa, sb, oracle.F32)
    assert np.array_equal(to_bits(C), bits)


def test_quantize_beyond_2_31_elements_sampled():
    n = (1 << 31) + 7
    x = torch.randn(n, device=DEV)
    x[n - 1] = 7.5                               # the extreme element sits in the float tail
    q, s, a = P.fp8_quantize(x)
    torch.cuda.synchronize()
    assert a.item() == 7.5 and s.item() == np.float32(7.5) / np.float32(448.0)
    rng = np.random.default_rng(8)
    starts = np.r_[0, (1 << 31) - 4096, n - 4096, rng.integers(0, n - 4096, 6)]
    for st in starts:
        xs = x[st:st + 4096].cpu().numpy()
        ref = oracle.quantize_with_scale(xs, s.item())
        assert np.array_equal(q[st:st + 4096].cpu().numpy(), ref), st
    assert q[n - 1].item() == 0x7E                # 448
