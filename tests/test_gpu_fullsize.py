"""Every output of the large configurations against the oracle, through the
C ABI: the 8192^3 per-tensor GEMM (BF16 out), the 4096 x 28672 x 8192 LLM
linear layer, the 8192^3 block-scaled GEMM with 32x32 tile scales and the MoE
grouped GEMM (8 experts, 16384 tokens).  Each runs the whole path on both
sides from the same seeded FP32 inputs (GPU quantize -> GPU GEMM against
oracle quantize -> oracle GEMM) and holds every output to the BF16 rule of
tests/parity.py (the count of outputs passing only under its cancellation
allowance held to that file's ceiling).
The oracle's exact sums take about 20-45 s of CPU per configuration here."""
import numpy as np
import pytest
import torch

import oracle
import precision_dense_linear_amd as P
from precision_dense_linear_amd import workloads as W
from parity import check_bf16, to_bits

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def pertensor_all_outputs(a, b, what):
    qa, sa, _ = P.fp8_quantize(gpu(a))
    qb, sb, _ = P.fp8_quantize(gpu(b))
    C = P.fp8_gemm(qa, qb, sa, sb, torch.bfloat16)
    got = to_bits(C)
    del qa, qb, C
    oa, osa, _ = oracle.quantize_pertensor(a)
    ob, osb, _ = oracle.quantize_pertensor(b)
    bits, exact, sab = oracle.gemm_rows(oa, ob, osa, osb, oracle.BF16)
    res = check_bf16(got, bits, exact, sab * float(osa) * float(osb), what)
    print(what, "-> max ulp %d, allowance %d" % res, flush=True)


def test_headline_8192_all_outputs():
    print("full-size 8192^3 per-tensor BF16", flush=True)
    a, b = W.pertensor_pair(8192, 8192, 8192, seed=0)
    pertensor_all_outputs(a, b, "8192^3 BF16, all outputs")


def test_llm_4096x28672x8192_all_outputs():
    print("full-size LLM 4096x28672x8192 BF16", flush=True)
    a, w = W.llm_linear(4096, 28672, 8192)
    pertensor_all_outputs(a, w, "LLM 4096x28672x8192, all outputs")


def test_blockscaled_8192_all_outputs():
    print("full-size block-scaled 8192^3 BF16", flush=True)
    a, b = W.blockscaled_pair(8192, 8192, 8192, seed=0)
    qa, ta = P.fp8_quantize_blocked(gpu(a))
    qb, tb = P.fp8_quantize_blocked(gpu(b))
    got = to_bits(P.fp8_gemm_blockscaled(qa, qb, ta, tb, torch.bfloat16))
    del qa, qb
    oa, ota = oracle.quantize_blocked(a)
    ob, otb = oracle.quantize_blocked(b)
    bits, exact, sab = oracle.gemm_blockscaled_rows(oa, ob, ota, otb, oracle.BF16)
    res = check_bf16(got, bits, exact, sab, "block-scaled 8192^3, all outputs")
    print("block-scaled 8192^3 -> max ulp %d, allowance %d" % res, flush=True)


def test_moe_all_rows():
    print("full-size MoE 8 experts x 16384 tokens BF16", flush=True)
    x, w, off = W.moe()
    E, K, N = w.shape
    goff = gpu(off.astype(np.int32))
    qx, sx, _ = P.fp8_quantize_grouped(gpu(x), goff)
    qw, sw, _ = P.fp8_quantize_grouped(gpu(w.reshape(E * K, N)), gpu((np.arange(E + 1) * K).astype(np.int32)))
    got = to_bits(P.fp8_grouped_gemm(qx, qw.view(E, K, N), goff, sx, sw, torch.bfloat16))
    del qx, qw
    ox, osx, _ = oracle.quantize_grouped(x, off)
    ow, osw, _ = oracle.quantize_grouped(w.reshape(E * K, N), np.arange(E + 1) * K)
    bits, exact, sab = oracle.grouped_gemm_rows(ox, ow.reshape(E, K, N), off, osx, osw, oracle.BF16)
    e = np.searchsorted(off, np.arange(x.shape[0]), side="right") - 1
    res = check_bf16(got, bits, exact, sab * (osx[e].astype(np.float64) * osw[e])[:, None], "MoE, all rows")
    print("MoE -> max ulp %d, allowance %d" % res, flush=True)
