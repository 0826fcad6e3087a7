"""GPU parity of the 2:4-sparse weight path ("FP8 GEMM in JAX with Triton for
Blackwell", opening section: sparsity support, about 2x at 50% weight
sparsity) through the C ABI: pruning + quantization + compression bit-exact
with the oracle, and the sparse-matrix-core GEMM against the oracle's exact
GEMM of the pruned codes -- bit for bit where every sum is exact, else within
the FP8 matrix-core bound."""
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


def oracle_sparse_weights(w):
    """The oracle's pruned codes, scale, amax and compressed form of w."""
    q, s, a = oracle.quantize_pertensor(oracle.prune_2of4(w))
    vals, idx = oracle.compress_2of4(q)
    return q, s, a, vals, idx


@pytest.mark.parametrize("K,N", [(32, 64), (96, 1000), (64, 48), (8192, 8192)])
def test_quantize_2of4_bit_exact(K, N):
    w = W.gaussian((K, N), 0.02, K + N, "sparse-w")
    w[:4, 0] = [0.0, 0.0, 0.0, 0.0]                 # an all-zero group
    w[4:8, 1] = [0.0, 1e-30, 0.0, 0.0]             # a kept value that rounds to zero
    vals, idx, s, a = P.fp8_quantize_2of4(gpu(w))
    torch.cuda.synchronize()
    q, os_, oa, ovals, oidx = oracle_sparse_weights(w)
    assert s.item() == os_ and a.item() == oa
    assert np.array_equal(vals.cpu().numpy(), ovals), "%d values differ" % int((vals.cpu().numpy() != ovals).sum())
    assert np.array_equal(idx.cpu().numpy().view(np.uint32), oidx)


def sparse_int_operands(M, N, K, seed):
    rng = np.random.default_rng(seed)
    va = rng.integers(-16, 17, (M, K)).astype(np.float32)
    vb = oracle.prune_2of4(rng.integers(-16, 17, (K, N)).astype(np.float32))
    qa = torch.from_numpy(va).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    qb = torch.from_numpy(vb).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    vals, idx = oracle.compress_2of4(qb)
    return qa, qb, vals, idx


@pytest.mark.parametrize("M,N,K", [(64, 64, 64), (32, 48, 32), (300, 256, 512), (1100, 528, 352), (2048, 1024, 1024)])
@pytest.mark.parametrize("kind", [F32, BF16, F16])
def test_sparse_integer_exact_bit_for_bit(M, N, K, kind):
    """Small-integer operands: every product sum is exact, so the sparse
    matrix cores must reproduce the oracle's dense GEMM of the pruned codes
    bit for bit (both tile classes, ragged tiles, K ending in half a slice)."""
    qa, qb, vals, idx = sparse_int_operands(M, N, K, M + N + K)
    one = torch.ones(1, device=DEV)
    C = P.fp8_gemm_sparse24(gpu(qa), gpu(vals), gpu(idx.view(np.int32)), one, one, TORCH_OUT[kind])
    bits, _, _ = oracle.gemm_rows(qa, qb, 1.0, 1.0, kind) if kind != F16 else \
        oracle.gemm_rows_fmt(qa, qb, oracle.E4M3, oracle.E4M3, 1.0, 1.0, F16)
    got = to_bits(C)
    assert np.array_equal(got, bits), "%d mismatches" % int((got != bits).sum())


def check_fast(C, exact, sab, what):
    got = C.float().cpu().numpy().astype(np.float64)
    ulp = 0.0 if C.dtype == torch.float32 else (bf16_ulp(exact) if C.dtype == torch.bfloat16 else f16_ulp(exact))
    bound = FAST_REL * sab + ulp + 1e-15 * np.abs(exact)
    bad = ~(np.abs(got - exact) <= bound)
    assert not bad.any(), "%s: %d of %d outputs beyond the bound" % (what, int(bad.sum()), bad.size)
    return float((np.abs(got - exact) / np.maximum(sab, 1e-300)).max())


def end_to_end(M, N, K, kind, rows=None, seed=0):
    a, w = W.llm_linear(M, N, K, seed=seed)
    qa, sa, _ = P.fp8_quantize(gpu(a))
    vals, idx, sw, _ = P.fp8_quantize_2of4(gpu(w))
    C = P.fp8_gemm_sparse24(qa, vals, idx, sa, sw, TORCH_OUT[kind])
    torch.cuda.synchronize()
    oa, osa, _ = oracle.quantize_pertensor(a)
    q, osw, _, _, _ = oracle_sparse_weights(w)
    _, exact, sab = oracle.gemm_rows(oa, q, osa, osw, F32, rows=rows)
    got = C if rows is None else C[torch.from_numpy(rows).to(DEV)]
    return check_fast(got, exact, sab * float(osa) * float(osw), "sparse %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K,kind", [(256, 256, 256, F32), (1024, 1024, 1024, BF16), (96, 400, 224, F16),
                                        (1536, 512, 2048, BF16)])
def test_sparse_random_within_bound(M, N, K, kind):
    print("worst err / sum|ab| =", end_to_end(M, N, K, kind, seed=M))


def test_sparse_llm_4096_sampled():
    rows = np.unique(np.r_[0, 4095, np.random.default_rng(3).choice(4096, 8, replace=False)]).astype(np.int64)
    print("worst err / sum|ab| =", end_to_end(4096, 28672, 8192, BF16, rows=rows))


def test_sparse_k_zero_writes_zeros():
    A = torch.zeros((64, 0), dtype=torch.uint8, device=DEV)
    vals = torch.zeros((0, 64), dtype=torch.uint8, device=DEV)
    idx = torch.zeros((0, 64), dtype=torch.int32, device=DEV)
    one = torch.ones(1, device=DEV)
    C = torch.full((64, 64), float("nan"), device=DEV)
    P.fp8_gemm_sparse24(A, vals, idx, one, one, torch.float32, C=C)
    torch.cuda.synchronize()
    assert torch.count_nonzero(C).item() == 0
