"""GPU tests of the FP8_ACC_FAST accumulation mode (native FP8 matrix cores).

Its contract (include/fp8gemm.h): per group of 8 products the extra error is
below 7 * 2^-13 * max|a*b| <= 7 * 2^-13 * sum|a*b| of the group, on top of the
FP32 accumulation; so |C - C_exact| <= (7*2^-13 + 2e-6) * sum_k|a*b| * sa * sb
(plus one BF16 ulp of rounding for BF16 output).  Small-integer operands keep
every product inside the 13-bit window, so there the mode is exact and must
match the oracle bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_dense_linear_amd as P
from precision_dense_linear_amd import workloads as W
from parity import bf16_to_f64, bf16_ulp, to_bits

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
FAST_REL = 7 * 2.0 ** -13 + 2e-6


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def one():
    return torch.ones(1, dtype=torch.float32, device=DEV)


@pytest.mark.parametrize("M,N,K", [(17, 48, 48), (65, 272, 1040), (300, 256, 512), (1100, 528, 272)])
@pytest.mark.parametrize("kind", [oracle.F32, oracle.BF16])
def test_fast_integer_exact(M, N, K, kind):
    rng = np.random.default_rng(M + N + K)
    va = rng.integers(-16, 17, (M, K)).astype(np.float32)
    vb = rng.integers(-16, 17, (K, N)).astype(np.float32)
    qa = torch.from_numpy(va).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    qb = torch.from_numpy(vb).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    C = P.fp8_gemm(gpu(qa), gpu(qb), one(), one(), torch.float32 if kind == oracle.F32 else torch.bfloat16, fast=True)
    bits, _, _ = oracle.gemm_rows(qa, qb, 1.0, 1.0, kind)
    assert np.array_equal(to_bits(C), bits)


def check_fast(C, exact, sab_scaled, what):
    bits = to_bits(C)
    got = bits.view(np.float32).astype(np.float64) if C.dtype == torch.float32 else bf16_to_f64(bits)
    bound = FAST_REL * sab_scaled + (0 if C.dtype == torch.float32 else bf16_ulp(exact)) + 1e-15 * np.abs(exact)
    err = np.abs(got - exact)
    assert np.all(err <= bound), "%s: %d outputs beyond the FP8_ACC_FAST bound" % (what, int((err > bound).sum()))
    return float((err / np.maximum(sab_scaled, 1e-300)).max())


@pytest.mark.parametrize("shape,out", [((256, 256, 256), torch.float32), ((1024, 1024, 1024), torch.bfloat16)])
def test_fast_workloads_within_bound(shape, out):
    M, N, K = shape
    a, b = W.pertensor_pair(M, N, K, seed=0)
    qa, sa, _ = P.fp8_quantize(gpu(a))
    qb, sb, _ = P.fp8_quantize(gpu(b))
    C = P.fp8_gemm(qa, qb, sa, sb, out, fast=True)
    C2 = P.fp8_gemm(qa, qb, sa, sb, out, fast=True)
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.uint8), C2.view(torch.uint8))        # deterministic
    oa, osa, _ = oracle.quantize_pertensor(a)
    ob, osb, _ = oracle.quantize_pertensor(b)
    _, exact, sab = oracle.gemm_rows(oa, ob, osa, osb, oracle.F32)
    worst = check_fast(C, exact, sab * float(osa) * float(osb), "%s fast" % (shape,))
    print(shape, "max |err| / sum|ab| =", worst)


@pytest.mark.parametrize("M,N", [(16, 8192), (128, 28672), (4096, 28672)])
def test_fast_llm_within_bound(M, N):
    a, w = W.llm_linear(M, N, 8192)
    qa, sa, _ = P.fp8_quantize(gpu(a))
    qw, sw, _ = P.fp8_quantize(gpu(w))
    C = P.fp8_gemm(qa, qw, sa, sw, torch.bfloat16, fast=True)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, M - 1, np.random.default_rng(M).choice(M, size=min(8, M), replace=False)])
    oa, osa, _ = oracle.quantize_pertensor(a)
    ow, osw, _ = oracle.quantize_pertensor(w)
    _, exact, sab = oracle.gemm_rows(oa, ow, osa, osw, oracle.F32, rows=rows)
    check_fast(C[torch.from_numpy(rows).to(DEV)], exact, sab * float(osa) * float(osw), "LLM M=%d fast" % M)


def test_fast_grouped_matches_per_expert_fast_gemm():
    x, w, off = W.moe(E=4, T=1000, K=512, N=384)
    E, K, N = w.shape
    goff = gpu(off.astype(np.int32))
    qx, sx, _ = P.fp8_quantize_grouped(gpu(x), goff)
    qw, sw, _ = P.fp8_quantize_grouped(gpu(w.reshape(E * K, N)), gpu((np.arange(E + 1) * K).astype(np.int32)))
    C = P.fp8_grouped_gemm(qx, qw.view(E, K, N), goff, sx, sw, torch.float32, fast=True)
    torch.cuda.synchronize()
    ox, osx, _ = oracle.quantize_grouped(x, off)
    ow, osw, _ = oracle.quantize_grouped(w.reshape(E * K, N), np.arange(E + 1) * K)
    _, exact, sab = oracle.grouped_gemm_rows(ox, ow.reshape(E, K, N), off, osx, osw, oracle.F32)
    e = np.searchsorted(off, np.arange(x.shape[0]), side="right") - 1
    check_fast(C, exact, sab * (osx[e].astype(np.float64) * osw[e])[:, None], "grouped fast")
