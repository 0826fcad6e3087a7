"""GPU parity of the FP8 GEMMs with the CPU oracle, through the C ABI.

End-to-end cases run the whole path on both sides from the same seeded FP32
inputs: GPU quantize -> GPU GEMM against oracle quantize -> oracle GEMM.
Bounds: FP32 output within 2e-6*sum|ab|*sa*sb of the exact value; BF16 output
within 1 ulp of the oracle's correctly rounded value (tests/parity.py).
Full-size configurations are checked on sampled rows the oracle computes one
by one; small ones (spanning several tiles and a ragged tail) on every output.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_dense_linear_amd as P
from precision_dense_linear_amd import workloads as W
from parity import check_bf16, check_f32, to_bits

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
F32, BF16 = oracle.F32, oracle.BF16


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def scalar(v):
    return torch.tensor([v], dtype=torch.float32, device=DEV)


def sample_rows(M, n, seed):
    r = np.random.default_rng(seed).choice(M, size=min(n, M), replace=False)
    return np.unique(np.concatenate([r, [0, M - 1]])).astype(np.int64)


def compare(C, bits, exact, sab_scaled, kind, rows, what):
    got = to_bits(C)[rows] if rows is not None else to_bits(C)
    if kind == F32:
        return check_f32(got.view(np.float32), exact, sab_scaled, what)
    return check_bf16(got, bits, exact, sab_scaled, what)


def pertensor_end_to_end(a, b, kind, rows=None, what="", workspace=None):
    qa, sa, _ = P.fp8_quantize(gpu(a))
    qb, sb, _ = P.fp8_quantize(gpu(b))
    C = P.fp8_gemm(qa, qb, sa, sb, torch.float32 if kind == F32 else torch.bfloat16, workspace=workspace)
    torch.cuda.synchronize()
    oa, osa, _ = oracle.quantize_pertensor(a)
    ob, osb, _ = oracle.quantize_pertensor(b)
    bits, exact, sab = oracle.gemm_rows(oa, ob, osa, osb, kind, rows)
    res = compare(C, bits, exact, sab * float(osa) * float(osb), kind, rows, what)
    print(what, "->", res, flush=True)
    return C


# ------------------------------------------------------------------ configurations
def test_pertensor_256_f32():
    a, b = W.pertensor_pair(256, 256, 256, seed=0)
    pertensor_end_to_end(a, b, F32, what="256^3 FP32")


def test_pertensor_1024_bf16_and_determinism():
    a, b = W.pertensor_pair(1024, 1024, 1024, seed=0)
    C1 = pertensor_end_to_end(a, b, BF16, what="1024^3 BF16")
    C2 = pertensor_end_to_end(a, b, BF16, what="1024^3 BF16 again")
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))


@pytest.mark.parametrize("M,N", [(16, 8192), (128, 28672), (4096, 28672)])
def test_llm_linear_k8192_bf16(M, N):
    a, w = W.llm_linear(M, N, 8192)
    rows = None if M <= 16 else sample_rows(M, 12, M)
    pertensor_end_to_end(a, w, BF16, rows=rows, what="LLM M=%d N=%d K=8192" % (M, N))


def test_headline_8192_bf16_sampled():
    a, b = W.pertensor_pair(8192, 8192, 8192, seed=0)
    pertensor_end_to_end(a, b, BF16, rows=sample_rows(8192, 14, 1), what="8192^3 BF16")


# ------------------------------------------------------------------ exactness / edges
def int_codes(shape, seed, lim=16):
    v = np.random.default_rng(seed).integers(-lim, lim + 1, shape).astype(np.float32)
    return torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy(), v


@pytest.mark.parametrize("M,N,K", [(1, 16, 16), (17, 48, 48), (64, 64, 128), (65, 272, 1040),
                                   (255, 528, 256), (300, 256, 512), (100, 8208, 272), (300, 5648, 272),
                                   (480, 28688, 80), (1025, 64, 384), (1100, 528, 272)])
@pytest.mark.parametrize("kind", [F32, BF16])
def test_integer_exact_bit_for_bit(M, N, K, kind):
    """Small-integer operands with unit scales: every partial sum is an integer
    below 2^24, so FP32 accumulation is exact in any order and the GPU must
    match the oracle bit for bit (tiles of every shape class, ragged tails;
    480 x 28688 has enough 256 x 256 tiles to be run with that class,
    300 x 5648 enough 128 x 128 tiles for that one; the other shapes have
    too few of either: 100 x 8208 and 1100 x 528 go to the 64 x 64 class,
    the rest to the 32 x 64 class)."""
    qa, va = int_codes((M, K), M * 7 + K)
    qb, vb = int_codes((K, N), N * 13 + K)
    C = P.fp8_gemm(gpu(qa), gpu(qb), scalar(1.0), scalar(1.0), torch.float32 if kind == F32 else torch.bfloat16)
    bits, exact, _ = oracle.gemm_rows(qa, qb, 1.0, 1.0, kind)
    assert np.array_equal(exact, va.astype(np.float64) @ vb.astype(np.float64))
    got = to_bits(C)
    assert np.array_equal(got, bits), "%d mismatches" % int((got != bits).sum())


def test_identity_b_gives_scaled_a():
    rng = np.random.default_rng(8)
    qa = rng.integers(0, 256, (300, 256)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x38
    eye = np.zeros((256, 256), np.uint8)
    eye[np.arange(256), np.arange(256)] = 0x38
    C = P.fp8_gemm(gpu(qa), gpu(eye), scalar(0.5), scalar(0.25), torch.float32)
    ref = (oracle.decode(qa) * 0.125).astype(np.float32)
    assert np.array_equal(C.cpu().numpy(), ref)


def test_k_zero_writes_zeros_and_m_zero_is_noop():
    A = torch.zeros((40, 0), dtype=torch.uint8, device=DEV)
    B = torch.zeros((0, 32), dtype=torch.uint8, device=DEV)
    C = torch.full((40, 32), float("nan"), device=DEV)
    P.fp8_gemm(A, B, scalar(1.0), scalar(1.0), torch.float32, C=C)
    assert torch.count_nonzero(C).item() == 0
    C2 = torch.full((0, 32), 1.0, device=DEV)
    P.fp8_gemm(torch.zeros((0, 64), dtype=torch.uint8, device=DEV), torch.zeros((64, 32), dtype=torch.uint8, device=DEV),
               scalar(1.0), scalar(1.0), torch.float32, C=C2)


@pytest.mark.parametrize("M,N,K", [(33, 96, 160), (200, 144, 400), (1500, 400, 208)])
def test_random_ragged_f32(M, N, K):
    a, b = W.pertensor_pair(M, N, K, seed=M + N + K)
    pertensor_end_to_end(a, b, F32, what="ragged %dx%dx%d" % (M, N, K))


# ------------------------------------------------------------------ split-K
# fp8_gemm_ws: M <= 64 with few 32 x 64 tiles splits K over workgroups.  With
# 256 CUs the shapes below take 2, 8, 4 and 8 splits; the K stage counts (4,
# 17, 9, 32) give even and uneven K ranges, the last one ending in a partial
# stage.
SPLITK_SHAPES = [(1, 512, 1024), (37, 1040, 4112), (64, 2048, 2304), (20, 96, 8192)]


@pytest.mark.parametrize("M,N,K", SPLITK_SHAPES)
@pytest.mark.parametrize("fast", [False, True])
@pytest.mark.parametrize("kind", [F32, BF16])
def test_splitk_integer_exact_bit_for_bit(M, N, K, fast, kind):
    """Integer operands make the sum exact in any order, so every split's
    partial, the fixed-order sum and the ragged row/column edges must give
    the oracle's value bit for bit -- with the workspace (split) and without
    it (one workgroup per tile)."""
    qa, va = int_codes((M, K), M * 5 + K, lim=8)
    qb, vb = int_codes((K, N), N * 3 + K, lim=8)
    bits, exact, _ = oracle.gemm_rows(qa, qb, 1.0, 1.0, kind)
    for ws in (P.gemm_workspace(DEV), None):
        C = P.fp8_gemm(gpu(qa), gpu(qb), scalar(1.0), scalar(1.0), torch.float32 if kind == F32 else torch.bfloat16,
                       fast=fast, workspace=ws)
        got = to_bits(C)
        assert np.array_equal(got, bits), "%d mismatches (workspace: %s)" % (int((got != bits).sum()), ws is not None)


@pytest.mark.parametrize("M,N,K", [(48, 3072, 8192), (37, 1040, 4112)])
def test_splitk_random_f32(M, N, K):
    a, b = W.pertensor_pair(M, N, K, seed=M * N + K)
    pertensor_end_to_end(a, b, F32, what="split-K %dx%dx%d" % (M, N, K), workspace=P.gemm_workspace(DEV))


def test_splitk_small_workspace_limits_the_splits():
    """A workspace of only a few split tiles bounds tiles x splits: 16 tiles
    with room for 40 split tiles run 2 splits each (a third would not fit),
    and room for 31 leaves the call unsplit; both exact on integer codes."""
    M, N, K = 20, 1024, 8192
    qa, _ = int_codes((M, K), 11, lim=8)
    qb, _ = int_codes((K, N), 12, lim=8)
    bits, _, _ = oracle.gemm_rows(qa, qb, 1.0, 1.0, F32)
    for tiles in (40, 31):
        ws = P.gemm_workspace(DEV, tiles * P.FP8_GEMM_WS_TILE_BYTES)
        C = P.fp8_gemm(gpu(qa), gpu(qb), scalar(1.0), scalar(1.0), torch.float32, workspace=ws)
        assert np.array_equal(to_bits(C), bits)
        assert torch.count_nonzero(ws[tiles * 8192:]).item() == 0    # counters back at zero


def test_splitk_repeated_calls_other_shapes_and_two_streams():
    """Each launch leaves the per-tile arrival counters at zero: repeated
    calls, a call with a different tile count in between, and calls on two
    streams at once (each with its own workspace) give identical bits."""
    def operands(M, N, K, seed):
        a, b = W.pertensor_pair(M, N, K, seed=seed)
        qa, sa, _ = P.fp8_quantize(gpu(a))
        qb, sb, _ = P.fp8_quantize(gpu(b))
        return qa, qb, sa, sb

    ws1, ws2 = P.gemm_workspace(DEV), P.gemm_workspace(DEV)
    x = operands(40, 4096, 4096, 3)   # 128 tiles, 4 splits
    y = operands(16, 1024, 8192, 4)   # 16 tiles, 8 splits
    Cx = P.fp8_gemm(*x, torch.float32, workspace=ws1)
    Cy = P.fp8_gemm(*y, torch.bfloat16, workspace=ws1)
    torch.cuda.synchronize()
    for _ in range(3):
        assert torch.equal(P.fp8_gemm(*x, torch.float32, workspace=ws1), Cx)
        assert torch.equal(P.fp8_gemm(*y, torch.bfloat16, workspace=ws1).view(torch.int16), Cy.view(torch.int16))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for _ in range(4):
        with torch.cuda.stream(s1):
            o1 = P.fp8_gemm(*x, torch.float32, workspace=ws1)
        with torch.cuda.stream(s2):
            o2 = P.fp8_gemm(*y, torch.bfloat16, workspace=ws2)
        outs.append((o1, o2))
    torch.cuda.synchronize()
    for o1, o2 in outs:
        assert torch.equal(o1, Cx)
        assert torch.equal(o2.view(torch.int16), Cy.view(torch.int16))
    a, b = W.pertensor_pair(40, 4096, 4096, seed=3)
    pertensor_end_to_end(a, b, F32, what="split-K 40x4096x4096 (oracle)", workspace=ws1)


# ------------------------------------------------------------------ block-scaled
def blockscaled_end_to_end(a, b, kind, rows=None, what=""):
    qa, ta = P.fp8_quantize_blocked(gpu(a))
    qb, tb = P.fp8_quantize_blocked(gpu(b))
    C = P.fp8_gemm_blockscaled(qa, qb, ta, tb, torch.float32 if kind == F32 else torch.bfloat16)
    torch.cuda.synchronize()
    oa, ota = oracle.quantize_blocked(a)
    ob, otb = oracle.quantize_blocked(b)
    bits, exact, sab = oracle.gemm_blockscaled_rows(oa, ob, ota, otb, kind, rows)
    res = compare(C, bits, exact, sab, kind, rows, what)
    print(what, "->", res, flush=True)


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (96, 160, 224), (384, 128, 1056)])
@pytest.mark.parametrize("kind", [F32, BF16])
def test_blockscaled_small(M, N, K, kind):
    a, b = W.blockscaled_pair(M, N, K, seed=M + K)
    blockscaled_end_to_end(a, b, kind, what="block-scaled %dx%dx%d" % (M, N, K))


def test_blockscaled_zero_tiles():
    a, b = W.blockscaled_pair(128, 128, 128, seed=5)
    a[:32, 32:64] = 0.0
    b[64:96, :] = 0.0
    blockscaled_end_to_end(a, b, BF16, what="block-scaled with zero tiles")


def test_blockscaled_8192_tile_factors_sampled():
    a, b = W.blockscaled_pair(8192, 8192, 8192, seed=0)
    blockscaled_end_to_end(a, b, BF16, rows=sample_rows(8192, 10, 2), what="block-scaled 8192^3 BF16")


# ------------------------------------------------------------------ grouped (MoE)
def grouped_end_to_end(x, w, off, kind, rows=None, what=""):
    E, K, N = w.shape
    T = x.shape[0]
    goff = gpu(off.astype(np.int32))
    qx, sx, _ = P.fp8_quantize_grouped(gpu(x), goff)
    qw, sw, _ = P.fp8_quantize_grouped(gpu(w.reshape(E * K, N)), gpu((np.arange(E + 1) * K).astype(np.int32)))
    C = torch.full((T, N), float("nan"), dtype=torch.float32 if kind == F32 else torch.bfloat16, device=DEV)
    P.fp8_grouped_gemm(qx, qw.view(E, K, N), goff, sx, sw, C.dtype, C=C)
    torch.cuda.synchronize()
    ox, osx, _ = oracle.quantize_grouped(x, off)
    ow, osw, _ = oracle.quantize_grouped(w.reshape(E * K, N), np.arange(E + 1) * K)
    ow = ow.reshape(E, K, N)
    lo, hi = int(off[0]), int(off[-1])
    sel = np.arange(lo, hi) if rows is None else rows
    bits, exact, sab = oracle.grouped_gemm_rows(ox, ow, off, osx, osw, kind, rows=sel)
    expert = np.searchsorted(off, sel, side="right") - 1
    scale = osx[expert].astype(np.float64) * osw[expert].astype(np.float64)
    res = compare(C, bits, exact, sab * scale[:, None], kind, sel, what)
    print(what, "->", res, flush=True)
    # rows outside every expert's range are never written
    outside = np.setdiff1d(np.arange(T), np.arange(lo, hi))
    if outside.size:
        assert torch.isnan(C[torch.from_numpy(outside).to(DEV)].float()).all()
    return C


def test_grouped_small_with_empty_expert_and_outside_rows():
    rng = np.random.default_rng(6)
    T, K, N, E = 300, 192, 96, 5
    x = rng.standard_normal((T, K)).astype(np.float32)
    w = (rng.standard_normal((E, K, N)) * 0.02).astype(np.float32)
    grouped_end_to_end(x, w, np.array([0, 70, 70, 171, 290, 300]), F32, what="grouped, empty expert")
    grouped_end_to_end(x, w, np.array([10, 70, 70, 171, 260, 280]), BF16, what="grouped, rows outside")


def test_grouped_single_expert_equals_gemm():
    a, b = W.pertensor_pair(333, 128, 256, seed=9)
    off = np.array([0, 333])
    C = grouped_end_to_end(a, b[None], off, F32, what="grouped single expert")
    qa, sa, _ = P.fp8_quantize(gpu(a))
    qb, sb, _ = P.fp8_quantize(gpu(b))
    C2 = P.fp8_gemm(qa, qb, sa, sb, torch.float32)
    assert torch.equal(C, C2)


@pytest.mark.parametrize("kind", [F32, BF16])
def test_grouped_large_experts_ragged_ends(kind):
    """Over 1024 rows per expert on average (the 256 x 256 tile class): expert
    ends at every kind of position inside a 256-row tile (0, under 128, 127,
    128 and over 128 rows past the last whole tile), an empty expert, a
    ragged N; every output compared."""
    rng = np.random.default_rng(31)
    counts = np.array([1100, 0, 1280, 1919, 1408, 550])  # remainders 76, -, 0, 127, 128, 38
    off = np.concatenate([[0], np.cumsum(counts)])
    T, K, N, E = int(off[-1]), 320, 272, len(counts)
    x = rng.standard_normal((T, K)).astype(np.float32)
    w = (rng.standard_normal((E, K, N)) * 0.02).astype(np.float32)
    grouped_end_to_end(x, w, off, kind, what="grouped, large experts, ragged ends")


def test_grouped_moe_8_experts_16384_tokens_sampled():
    x, w, off = W.moe()
    rows = np.concatenate([sample_rows(int(off[e + 1] - off[e]), 3, e) + off[e] for e in range(8)])
    grouped_end_to_end(x, w, off, BF16, rows=np.unique(rows), what="MoE 8 experts Zipf(1.2) T=16384")
