"""The binding's tensor checks with GPU operands: a wrong output tensor (type,
size, layout), a scale or offsets array of the wrong type, size or device,
and operands on two devices are refused before any launch, and the same
call with correct tensors still runs and matches the oracle."""
import numpy as np
import pytest
import torch

import oracle
import precision_dense_linear_amd as P
from parity import to_bits

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def codes(shape, seed):
    rng = np.random.default_rng(seed)
    v = rng.integers(-4, 5, shape).astype(np.float32)
    return torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_gemm_refuses_bad_tensors():
    M, N, K = 96, 160, 64
    qa, qb = codes((M, K), 1), codes((K, N), 2)
    A, B = torch.from_numpy(qa).to(DEV), torch.from_numpy(qb).to(DEV)
    one = torch.ones(1, device=DEV)
    bad = {
        "C of the wrong type": dict(C=torch.empty((M, N), dtype=torch.float16, device=DEV)),
        "C too small": dict(C=torch.empty((M - 1, N), dtype=torch.bfloat16, device=DEV)),
        "C not contiguous": dict(C=torch.empty((N, M), dtype=torch.bfloat16, device=DEV).t()),
        "C on the host": dict(C=torch.empty((M, N), dtype=torch.bfloat16)),
    }
    for what, kw in bad.items():
        with pytest.raises(ValueError):
            P.fp8_gemm(A, B, one, one, torch.bfloat16, **kw)
    for scale_a in (torch.ones(1), torch.ones(1, device=DEV, dtype=torch.float64), torch.ones(0, device=DEV)):
        with pytest.raises(ValueError):
            P.fp8_gemm(A, B, scale_a, one, torch.bfloat16)
    with pytest.raises(ValueError):
        P.fp8_gemm(A, B.cpu(), one, one, torch.bfloat16)
    with pytest.raises(ValueError):
        P.fp8_gemm(A, B, one, one, torch.bfloat16, workspace=torch.zeros(16, dtype=torch.uint8))
    C = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=DEV)
    P.fp8_gemm(A, B, one, one, torch.bfloat16, C=C)
    bits, _, _ = oracle.gemm_rows(qa, qb, 1.0, 1.0, oracle.BF16)
    assert np.array_equal(to_bits(C), bits)


def test_grouped_and_quantize_refuse_bad_tensors():
    T, K, N, E = 100, 64, 48, 3
    qa, qb = codes((T, K), 3), codes((E, K, N), 4)
    A, B = torch.from_numpy(qa).to(DEV), torch.from_numpy(qb).to(DEV)
    off = torch.tensor([0, 40, 40, T], dtype=torch.int32, device=DEV)
    s = torch.ones(E, device=DEV)
    for kw in (dict(offsets=off.long()), dict(offsets=off.cpu()), dict(scale_a=torch.ones(E - 1, device=DEV))):
        args = dict(offsets=off, scale_a=s, scale_b=s)
        args.update(kw)
        with pytest.raises(ValueError):
            P.fp8_grouped_gemm(A, B, args["offsets"], args["scale_a"], args["scale_b"], torch.float32)
    C = P.fp8_grouped_gemm(A, B, off, s, s, torch.float32)
    bits, _, _ = oracle.grouped_gemm_rows(qa, qb, off.cpu().numpy(), s.cpu().numpy(), s.cpu().numpy(), oracle.F32)
    assert np.array_equal(to_bits(C), bits)
    x = torch.randn(64, 64, device=DEV)
    for kw in (dict(q=torch.empty(64 * 64 - 1, dtype=torch.uint8, device=DEV)), dict(scale=torch.empty(1)),
               dict(amax=torch.empty(1, dtype=torch.float64, device=DEV))):
        with pytest.raises(ValueError):
            P.fp8_quantize(x, **kw)
    with pytest.raises(ValueError):
        P.fp8_quantize_blocked(x, tile_scales=torch.empty(3, device=DEV))
    with pytest.raises(ValueError):
        P.fp8_attention(*(torch.zeros(2, 10, 64, dtype=torch.uint8, device=DEV),) * 3, torch.ones(1), s[:1], s[:1])
