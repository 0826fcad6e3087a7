"""GPU parity of the block-scaled GEMM with power-of-two 32x32 tile scales
applied by the FP8 matrix cores ("FP8 GEMM in JAX with Triton for
Blackwell", parameter paragraph: 32x32 microscaling), through the C ABI:
the E8M0 quantizer bit-exact (both exponent layouts), the GEMM within the
FP8-matrix-core bound of include/fp8gemm.h, and bit for bit where every
partial sum is exact."""
import numpy as np
import pytest
import torch

import oracle
import precision_dense_linear_amd as P
from precision_dense_linear_amd import workloads as W
from parity import bf16_ulp, f16_ulp, to_bits

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
F32, BF16, F16 = oracle.F32, oracle.BF16, oracle.F16
TORCH_OUT = {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16}
FAST_REL = 7 * 2.0 ** -13 + 2e-6


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def values(C):
    if C.dtype == torch.float32:
        return C.cpu().numpy().astype(np.float64)
    return C.float().cpu().numpy().astype(np.float64)


def check_fast_bound(C, exact, sab, what):
    got = values(C)
    out_ulp = {torch.float32: 0.0, torch.bfloat16: None, torch.float16: None}[C.dtype]
    if C.dtype == torch.bfloat16:
        out_ulp = bf16_ulp(exact)
    elif C.dtype == torch.float16:
        out_ulp = f16_ulp(exact)
    bound = FAST_REL * sab + out_ulp + 1e-15 * np.abs(exact)
    err = np.abs(got - exact)
    bad = ~(err <= bound)
    if C.dtype == torch.float16:
        # past the binary16 range the output is +-Inf; accept it wherever the
        # value the bound allows reaches the overflow threshold (65520)
        reach = np.abs(exact) + FAST_REL * sab >= 65520.0
        bad &= ~(np.isinf(got) & (np.sign(got) == np.sign(exact)) & reach)
    assert not bad.any(), "%s: %d of %d outputs beyond the bound" % (what, int(bad.sum()), err.size)
    return float((err / np.maximum(sab, 1e-300)).max())


@pytest.mark.parametrize("shape", [(32, 32), (96, 160), (8192, 8192)])
def test_quantize_e8m0_bit_exact_both_layouts(shape):
    a, _ = W.blockscaled_pair(shape[0], 32, shape[1], seed=2)
    oq, osc = oracle.quantize_blocked_e8m0(a)
    for k_major in (False, True):
        q, e = P.fp8_quantize_blocked_e8m0(gpu(a), k_major=k_major)
        torch.cuda.synchronize()
        ref = osc.T if k_major else osc
        eh = e.cpu().numpy()
        assert eh.shape[1] % 4 == 0 and np.all(eh[:, ref.shape[1]:] == 127)      # padded rows
        assert np.array_equal(eh[:, :ref.shape[1]], ref)
        qh = q.cpu().numpy()
        assert np.array_equal(qh, oq), "%d codes differ" % int((qh != oq).sum())


def test_quantize_e8m0_zero_tile_and_extremes():
    a, _ = W.blockscaled_pair(64, 32, 96, seed=3)
    a[:32, 32:64] = 0.0
    a[32:, :32] *= np.float32(1e-38)          # tile amax subnormal-range: exponent clamps at -127
    a[32:, 64:] *= np.float32(1e30)
    q, e = P.fp8_quantize_blocked_e8m0(gpu(a))
    torch.cuda.synchronize()
    oq, osc = oracle.quantize_blocked_e8m0(a)
    assert osc[0, 1] == 127
    assert np.array_equal(e.cpu().numpy()[:, :3], osc) and np.array_equal(q.cpu().numpy(), oq)


def padded(e):
    """An exponent array with its rows padded to a multiple of 4 bytes (127)."""
    out = np.full((e.shape[0], (e.shape[1] + 3) // 4 * 4), 127, np.uint8)
    out[:, :e.shape[1]] = e
    return out


def end_to_end(M, N, K, kind, seed, rows=None, what=""):
    a, b = W.blockscaled_pair(M, N, K, seed=seed)
    qa, ea = P.fp8_quantize_blocked_e8m0(gpu(a), k_major=True)
    qb, eb = P.fp8_quantize_blocked_e8m0(gpu(b))
    C = P.fp8_gemm_blockscaled_e8m0(qa, qb, ea, eb, TORCH_OUT[kind])
    torch.cuda.synchronize()
    oa, osa = oracle.quantize_blocked_e8m0(a)
    ob, osb = oracle.quantize_blocked_e8m0(b)
    _, exact, sab = oracle.gemm_blockscaled_e8m0_rows(oa, ob, osa, osb, kind, rows=rows)
    got = C if rows is None else C[torch.from_numpy(np.asarray(rows)).to(DEV)]
    worst = check_fast_bound(got, exact, sab, what)
    print(what, "max err / sum|ab| =", worst, flush=True)


@pytest.mark.parametrize("M,N,K", [(32, 32, 32), (64, 64, 64), (96, 160, 224), (256, 256, 256), (1056, 1024, 512),
                                   (1152, 1088, 352)])
@pytest.mark.parametrize("kind", [F32, BF16, F16])
def test_e8m0_gemm_within_bound(M, N, K, kind):
    end_to_end(M, N, K, kind, seed=M + N + K, what="e8m0 %dx%dx%d" % (M, N, K))


def test_e8m0_gemm_8192_sampled():
    rows = np.unique(np.r_[0, 8191, np.random.default_rng(7).choice(8192, 10, replace=False)])
    end_to_end(8192, 8192, 8192, BF16, seed=0, rows=rows, what="e8m0 8192^3 BF16")


@pytest.mark.parametrize("M,N,K", [(64, 64, 256), (288, 96, 224), (1088, 1056, 256)])
def test_e8m0_gemm_exact_cases_bit_for_bit(M, N, K):
    """Small-integer codes and tile exponents within +-2 of 127: every block
    sum and every FP32 partial sum is exact, so the scaled matrix cores must
    reproduce the oracle bit for bit -- which also pins which exponent each
    lane and K block receives."""
    rng = np.random.default_rng(M + K)
    va = rng.integers(-8, 9, (M, K)).astype(np.float32)
    vb = rng.integers(-8, 9, (K, N)).astype(np.float32)
    qa = torch.from_numpy(va).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    qb = torch.from_numpy(vb).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    sa = rng.integers(125, 130, (M // 32, K // 32)).astype(np.uint8)
    sb = rng.integers(125, 130, (K // 32, N // 32)).astype(np.uint8)
    bits, exact, _ = oracle.gemm_blockscaled_e8m0_rows(qa, qb, sa, sb, F32)
    C = P.fp8_gemm_blockscaled_e8m0(gpu(qa), gpu(qb), gpu(padded(sa.T)), gpu(padded(sb)), torch.float32)
    got = to_bits(C)
    assert np.array_equal(got, bits), "%d mismatches" % int((got != bits).sum())


def test_e8m0_unit_exponents_equal_plain_fast_gemm():
    rng = np.random.default_rng(11)
    va = rng.integers(-16, 17, (256, 512)).astype(np.float32)
    vb = rng.integers(-16, 17, (512, 256)).astype(np.float32)
    qa = torch.from_numpy(va).to(torch.float8_e4m3fn).view(torch.uint8).to(DEV)
    qb = torch.from_numpy(vb).to(torch.float8_e4m3fn).view(torch.uint8).to(DEV)
    ea = torch.full((16, 8), 127, dtype=torch.uint8, device=DEV)    # [K/32][pitch(M/32)]
    eb = torch.full((16, 8), 127, dtype=torch.uint8, device=DEV)
    C = P.fp8_gemm_blockscaled_e8m0(qa, qb, ea, eb, torch.float32)
    one = torch.ones(1, device=DEV)
    C2 = P.fp8_gemm(qa, qb, one, one, torch.float32)
    assert torch.equal(C, C2)


def test_e8m0_k_zero_writes_zeros():
    A = torch.zeros((64, 0), dtype=torch.uint8, device=DEV)
    B = torch.zeros((0, 64), dtype=torch.uint8, device=DEV)
    e = torch.zeros((0, 4), dtype=torch.uint8, device=DEV)
    C = torch.full((64, 64), float("nan"), device=DEV)
    P.fp8_gemm_blockscaled_e8m0(A, B, e, e, torch.float32, C=C)
    torch.cuda.synchronize()
    assert torch.count_nonzero(C).item() == 0
