"""GPU parity of the 64x64 block-scaled path (the coarser scale granularity
of "FP8 GEMM in JAX with Triton for Blackwell", monitoring paragraph)
through the C ABI: 64x64-tile quantization bit-exact, the GEMM with 64-deep
K blocks within the bounds of tests/parity.py against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import precision_dense_linear_amd as P
from precision_dense_linear_amd import workloads as W
from parity import check_bf16, check_f16, check_f32, to_bits

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
F32, BF16, F16 = oracle.F32, oracle.BF16, oracle.F16
TORCH_OUT = {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16}


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def compare(C, bits, exact, sab, kind, what):
    got = to_bits(C)
    if kind == F32:
        return check_f32(got.view(np.float32), exact, sab, what)
    return (check_bf16 if kind == BF16 else check_f16)(got, bits, exact, sab, what)


@pytest.mark.parametrize("shape", [(64, 64), (192, 320), (8192, 8192)])
def test_quantize_blocked64_bit_exact(shape):
    a, _ = W.blockscaled_pair(shape[0], 64, shape[1], seed=3, tile=64)
    q, ts = P.fp8_quantize_blocked64(gpu(a))
    torch.cuda.synchronize()
    oq, ots = oracle.quantize_blocked_t(a, 64)
    assert np.array_equal(ts.cpu().numpy(), ots)
    qh = q.cpu().numpy()
    assert np.array_equal(qh, oq), "%d codes differ" % int((qh != oq).sum())


def test_quantize_blocked64_zero_tile():
    a, _ = W.blockscaled_pair(128, 64, 128, seed=4, tile=64)
    a[64:, :64] = 0.0
    q, ts = P.fp8_quantize_blocked64(gpu(a))
    torch.cuda.synchronize()
    assert ts[1, 0].item() == 1.0 and torch.count_nonzero(q[64:, :64]).item() == 0
    oq, ots = oracle.quantize_blocked_t(a, 64)
    assert np.array_equal(q.cpu().numpy(), oq) and np.array_equal(ts.cpu().numpy(), ots)


def end_to_end(M, N, K, kind, seed, rows=None, what=""):
    a, b = W.blockscaled_pair(M, N, K, seed=seed, tile=64)
    qa, ta = P.fp8_quantize_blocked64(gpu(a))
    qb, tb = P.fp8_quantize_blocked64(gpu(b))
    C = P.fp8_gemm_blockscaled(qa, qb, ta, tb, TORCH_OUT[kind], block=64)
    torch.cuda.synchronize()
    oa, ota = oracle.quantize_blocked_t(a, 64)
    ob, otb = oracle.quantize_blocked_t(b, 64)
    bits, exact, sab = oracle.gemm_blockscaled_rows_t(oa, ob, ota, otb, 64, kind, rows=rows)
    got = C if rows is None else C[torch.from_numpy(np.asarray(rows)).to(DEV)]
    res = compare(got, bits, exact, sab, kind, what)
    print(what, "->", res, flush=True)


@pytest.mark.parametrize("M,N,K", [(64, 64, 64), (256, 256, 256), (192, 320, 448), (384, 128, 1088)])
@pytest.mark.parametrize("kind", [F32, BF16, F16])
def test_blockscaled64_small(M, N, K, kind):
    end_to_end(M, N, K, kind, seed=M + N + K, what="block64 %dx%dx%d" % (M, N, K))


def test_blockscaled64_8192_sampled():
    rows = np.unique(np.r_[0, 8191, np.random.default_rng(6).choice(8192, 10, replace=False)])
    end_to_end(8192, 8192, 8192, BF16, seed=0, rows=rows, what="block64 8192^3 BF16")


def test_blockscaled64_unit_scales_integer_exact():
    """Integer codes with unit tile scales: every partial and every fold is
    exact, so the result equals the plain GEMM bit for bit."""
    rng = np.random.default_rng(9)
    M, N, K = 192, 256, 320
    va = rng.integers(-16, 17, (M, K)).astype(np.float32)
    vb = rng.integers(-16, 17, (K, N)).astype(np.float32)
    qa = torch.from_numpy(va).to(torch.float8_e4m3fn).view(torch.uint8)
    qb = torch.from_numpy(vb).to(torch.float8_e4m3fn).view(torch.uint8)
    ones_a = torch.ones((M // 64, K // 64), device=DEV)
    ones_b = torch.ones((K // 64, N // 64), device=DEV)
    C = P.fp8_gemm_blockscaled(qa.to(DEV), qb.to(DEV), ones_a, ones_b, torch.float32, block=64)
    bits, _, _ = oracle.gemm_rows(qa.numpy(), qb.numpy(), 1.0, 1.0, F32)
    assert np.array_equal(to_bits(C), bits)


def test_blockscaled64_rejects_shapes_not_multiple_of_64():
    A = torch.zeros((96, 64), dtype=torch.uint8, device=DEV)
    B = torch.zeros((64, 64), dtype=torch.uint8, device=DEV)
    s = torch.ones((2, 1), device=DEV)
    with pytest.raises(P.FP8Error):
        P.fp8_gemm_blockscaled(A, B, s, s, torch.float32, block=64)
