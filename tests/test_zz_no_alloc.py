"""fp8_gemm_noalloc, the per-tensor GEMM whose split-K partial sums live in
the library's own static device array, through the C ABI: its outputs must
equal, bit for bit, those of fp8_gemm_ws with a caller workspace of the same
size (the same kernels and split counts), on two calls in a row, the second
with a smaller input -- for split shapes and an unsplit one, both
accumulation modes, FP32 and BF16 output -- and one case is checked against
the oracle to the FP32 bound."""
import numpy as np
import pytest
import torch

import oracle
import precision_dense_linear_amd as P
from precision_dense_linear_amd import workloads as W
from parity import check_f32, to_bits

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def operands(M, N, K, seed):
    a, b = W.pertensor_pair(M, N, K, seed=seed)
    qa, sa, _ = P.fp8_quantize(torch.from_numpy(a).to(DEV))
    qb, sb, _ = P.fp8_quantize(torch.from_numpy(b).to(DEV))
    return (qa, qb, sa, sb), (a, b)


# (first call, second call with a smaller input): 16 tiles of 32 x 64 x 8
# splits then the skinny class (M <= 16: 256-column tiles) with 2 tiles x 8
# splits; 64 tiles x 8 splits then skinny 2 tiles x 2; an unsplit
# 128 x 128-tile shape then a split 32 x 64 one; skinny 32 tiles x 8 splits
# (all 512 split tiles) then 4 tiles x 16 splits
PAIRS = [((20, 1024, 8192), (16, 512, 4096)), ((64, 2048, 2304), (1, 512, 1024)),
         ((300, 5648, 272), (40, 256, 1040)), ((16, 8192, 8192), (3, 1024, 4112))]


@pytest.mark.parametrize("first,second", PAIRS)
@pytest.mark.parametrize("fast", [False, True])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_noalloc_equals_workspace_variant(first, second, fast, out):
    print("noalloc %s then %s fast=%s out=%s" % (first, second, fast, out), flush=True)
    ws = P.gemm_workspace(DEV)
    for shape, seed in ((first, 1), (second, 2)):
        ops, _ = operands(*shape, seed=seed)
        ref = P.fp8_gemm(*ops, out, fast=fast, workspace=ws)
        got = P.fp8_gemm_noalloc(*ops, out, fast=fast)
        again = P.fp8_gemm_noalloc(*ops, out, fast=fast)
        torch.cuda.synchronize()
        for c in (got, again):
            assert np.array_equal(to_bits(c), to_bits(ref)), "%s: %d outputs differ from fp8_gemm_ws" % (
                shape, int((to_bits(c) != to_bits(ref)).sum()))


def test_noalloc_against_oracle():
    M, N, K = 48, 3072, 8192     # 48 tiles of 32 x 64, K split 8 ways
    ops, (a, b) = operands(M, N, K, seed=5)
    C = P.fp8_gemm_noalloc(*ops, torch.float32)
    oa, osa, _ = oracle.quantize_pertensor(a)
    ob, osb, _ = oracle.quantize_pertensor(b)
    _, exact, sab = oracle.gemm_rows(oa, ob, osa, osb, oracle.F32)
    print("noalloc vs oracle:", check_f32(to_bits(C).view(np.float32), exact, sab * float(osa) * float(osb),
                                           "fp8_gemm_noalloc 48x3072x8192"))
