"""The skinny GEMM class (plain GEMM, M <= 16 rows) through the C ABI: bit
for bit on small-integer codes (every partial sum exact in FP32, so any
order gives the oracle's value) over ragged M, N and K (K ending inside a
32-byte stage; K is a multiple of 16), both FP8 formats per operand,
every output type, in both accumulation modes, with K split across 2 to 16
workgroups (fp8_gemm_ws, two workspace sizes) and unsplit (enough column
tiles, a ragged last one); random end-to-end cases within the FP32 / BF16
bounds, including the 16 x 8192 x 8192 LLM layer; K = 0."""
import numpy as np
import pytest
import torch

import oracle
import precision_dense_linear_amd as P
from precision_dense_linear_amd import workloads as W
from parity import check_bf16, check_f32, to_bits

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
E4M3, E5M2 = oracle.E4M3, oracle.E5M2
NAME = {E4M3: "e4m3", E5M2: "e5m2"}
OUT = {oracle.F32: torch.float32, oracle.BF16: torch.bfloat16, oracle.F16: torch.float16}


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def one():
    return torch.ones(1, dtype=torch.float32, device=DEV)


def int_codes(shape, seed, fmt, lim=8):
    v = np.random.default_rng(seed).integers(-lim, lim + 1, shape).astype(np.float32)
    dt = torch.float8_e5m2 if fmt == E5M2 else torch.float8_e4m3fn
    return torch.from_numpy(v).to(dt).view(torch.uint8).numpy()


# (M, N, K): splits with the default workspace -- (3, 48, 1040) 2, (5, 96,
# 2000) 3, (16, 16384, 1024) 2, (7, 8192, 4112) 8, (16, 1024, 8192) 16;
# (4, 33040, 96) 130 tiles unsplit, the last 16 columns wide; (1, 16, 16)
# and (16, 272, 64) too little K for the class (32 x 64 tiles instead).
SHAPES = [(1, 16, 16), (3, 48, 1040), (16, 1024, 8192), (7, 8192, 4112), (16, 272, 64), (5, 96, 2000),
          (16, 16384, 1024), (4, 33040, 96)]
WS = {"none": 0, "default": P.FP8_GEMM_WORKSPACE_BYTES, "large": 2048 * P.FP8_GEMM_WS_TILE_BYTES}


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_skinny_integer_exact_bit_for_bit(M, N, K):
    works = {w: P.gemm_workspace(DEV, nbytes=n) if n else None for w, n in WS.items()}
    for fa, fb in ((E4M3, E4M3), (E5M2, E4M3), (E4M3, E5M2)):
        qa, qb = int_codes((M, K), M + K + fa, fa), int_codes((K, N), N + K + fb, fb)
        A, B = gpu(qa), gpu(qb)
        for kind in (oracle.F32, oracle.BF16, oracle.F16):
            bits, exact, _ = oracle.gemm_rows_fmt(qa, qb, fa, fb, 1.0, 1.0, kind)
            assert np.abs(exact).max() < 2 ** 24
            for w, work in works.items():
                for fast in (False, True):
                    C = P.fp8_gemm(A, B, one(), one(), OUT[kind], a_fmt=NAME[fa], b_fmt=NAME[fb], workspace=work,
                                   fast=fast)
                    got = to_bits(C)
                    assert np.array_equal(got, bits), "%s x %s kind %d ws %s fast %s: %d mismatches" % (
                        NAME[fa], NAME[fb], kind, w, fast, int((got != bits).sum()))


@pytest.mark.parametrize("M,N,K", [(16, 8192, 8192), (9, 1040, 4112), (1, 4096, 8192)])
@pytest.mark.parametrize("ws", [False, True])
def test_skinny_random_within_bounds(M, N, K, ws):
    a, b = W.llm_linear(M, N, K) if (M, N, K) == (16, 8192, 8192) else W.pertensor_pair(M, N, K, seed=M + N + K)
    qa, sa, _ = P.fp8_quantize(gpu(a))
    qb, sb, _ = P.fp8_quantize(gpu(b))
    work = P.gemm_workspace(DEV) if ws else None
    Cf = P.fp8_gemm(qa, qb, sa, sb, torch.float32, workspace=work)
    Cb = P.fp8_gemm(qa, qb, sa, sb, torch.bfloat16, workspace=work)
    Cb2 = P.fp8_gemm(qa, qb, sa, sb, torch.bfloat16, workspace=work)
    assert torch.equal(Cb.view(torch.int16), Cb2.view(torch.int16))
    oa, osa, _ = oracle.quantize_pertensor(a)
    ob, osb, _ = oracle.quantize_pertensor(b)
    bits, exact, sab = oracle.gemm_rows(oa, ob, osa, osb, oracle.F32)
    sc = sab * float(osa) * float(osb)
    print("skinny %dx%dx%d ws=%s F32 ->" % (M, N, K, ws), check_f32(to_bits(Cf).view(np.float32), exact, sc, "F32"))
    bbits, _, _ = oracle.gemm_rows(oa, ob, osa, osb, oracle.BF16)
    print("  BF16 ->", check_bf16(to_bits(Cb), bbits, exact, sc, "BF16"), flush=True)


def test_skinny_k_zero_writes_zeros():
    A = torch.zeros((5, 0), dtype=torch.uint8, device=DEV)
    B = torch.zeros((0, 64), dtype=torch.uint8, device=DEV)
    C = torch.full((5, 64), float("nan"), device=DEV)
    P.fp8_gemm(A, B, one(), one(), torch.float32, C=C, workspace=P.gemm_workspace(DEV))
    assert torch.count_nonzero(C).item() == 0
