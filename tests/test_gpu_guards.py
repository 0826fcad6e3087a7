"""Canary guards and poisoned outputs for every entry point, through the C
ABI: each output sits between two 4 KiB guard regions inside one buffer, the
output itself filled with NaN bit patterns (NaN codes for FP8 outputs)
before the call.  After the call the guards must be untouched, every output
element written (no NaN left), and the result equal, bit for bit, to the
same call into a fresh tensor.  Shapes are ragged (partial tiles in M, N,
K where the entry point allows them) and span the tile classes, the skinny
kernel and split K."""
import numpy as np
import pytest
import torch

import precision_dense_linear_amd as P

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
GUARD = 4096   # bytes on each side

POISON = {torch.uint8: 0x7F, torch.int32: 0x7FC00001, torch.float32: 0x7FC00001, torch.bfloat16: 0x7FC1,
          torch.float16: 0x7E01}
BITS = {torch.uint8: torch.uint8, torch.int32: torch.int32, torch.float32: torch.int32, torch.bfloat16: torch.int16,
        torch.float16: torch.int16}


class Guarded:
    """A tensor of `shape` and `dtype` between two poisoned guard regions."""

    def __init__(self, shape, dtype):
        self.esz = torch.empty(0, dtype=dtype).element_size()
        self.g = GUARD // self.esz
        self.n = int(np.prod(shape))
        bits = BITS[dtype]
        pat = POISON[dtype]
        if bits == torch.int16 and pat >= 0x8000:
            pat -= 0x10000
        self.buf = torch.full((2 * self.g + self.n,), pat, dtype=bits, device=DEV)
        self.pat = pat
        self.t = self.buf[self.g:self.g + self.n].view(dtype).view(shape)

    def check(self, what):
        b = self.buf
        assert torch.all(b[:self.g] == self.pat).item(), "%s: guard before the output written" % what
        assert torch.all(b[self.g + self.n:] == self.pat).item(), "%s: guard after the output written" % what
        if self.t.dtype == torch.uint8:
            left = int(((self.t & 0x7F) == 0x7F).sum().item())
        elif self.t.dtype == torch.int32:
            left = int((self.t == self.pat).sum().item())
        else:
            left = int(torch.isnan(self.t.float()).sum().item())
        assert left == 0, "%s: %d of %d output elements not written" % (what, left, self.n)


def same(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def rand_codes(shape, seed):
    x = torch.randn(shape, generator=torch.Generator().manual_seed(seed)).to(DEV)
    q, s, _ = P.fp8_quantize(x)
    return q, s


@pytest.mark.parametrize("M,N,K,ws,fast", [(5, 8192, 2048, True, False), (5, 272, 48, False, False),
                                            (40, 336, 400, True, True), (100, 4160, 528, False, False),
                                            (300, 1040, 272, False, True), (1100, 528, 96, False, False),
                                            (600, 9232, 64, False, False), (2000, 7152, 64, False, True)])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16, torch.float16])
def test_gemm_guards(M, N, K, ws, fast, out):
    A, sa = rand_codes((M, K), 1)
    B, sb = rand_codes((K, N), 2)
    work = P.gemm_workspace(DEV) if ws else None
    g = Guarded((M, N), out)
    P.fp8_gemm(A, B, sa, sb, out, C=g.t, workspace=work, fast=fast)
    g.check("fp8_gemm %dx%dx%d" % (M, N, K))
    assert same(g.t, P.fp8_gemm(A, B, sa, sb, out, workspace=work, fast=fast))
    if ws:
        g2 = Guarded((M, N), out)
        P.fp8_gemm_noalloc(A, B, sa, sb, out, C=g2.t, fast=fast)
        g2.check("fp8_gemm_noalloc")
        assert same(g2.t, g.t)


def test_grouped_gemm_guards():
    E, K, N = 5, 96, 272
    counts = [0, 77, 300, 1, 130]
    T = sum(counts)
    off = torch.tensor(np.r_[0, np.cumsum(counts)], dtype=torch.int32, device=DEV)
    A, _ = rand_codes((T, K), 3)
    B, _ = rand_codes((E, K, N), 4)
    s = torch.rand(E, device=DEV) + 0.5
    for out in (torch.float32, torch.bfloat16):
        g = Guarded((T, N), out)
        P.fp8_grouped_gemm(A, B, off, s, s, out, C=g.t)
        g.check("fp8_grouped_gemm")
        assert same(g.t, P.fp8_grouped_gemm(A, B, off, s, s, out))


@pytest.mark.parametrize("block", [32, 64])
def test_blockscaled_guards(block):
    M, N, K = 192, 320, 256
    xa = torch.randn(M, K, device=DEV)
    xb = torch.randn(K, N, device=DEV)
    qfn = P.fp8_quantize_blocked if block == 32 else P.fp8_quantize_blocked64
    ga, gsa = Guarded((M, K), torch.uint8), Guarded((M // block, K // block), torch.float32)
    qfn(xa, q=ga.t, tile_scales=gsa.t)
    ga.check("blocked quantize codes")
    gsa.check("blocked quantize scales")
    qb, sb = qfn(xb)
    g = Guarded((M, N), torch.bfloat16)
    P.fp8_gemm_blockscaled(ga.t, qb, gsa.t, sb, torch.bfloat16, C=g.t, block=block)
    g.check("fp8_gemm_blockscaled")
    assert same(g.t, P.fp8_gemm_blockscaled(ga.t, qb, gsa.t, sb, torch.bfloat16, block=block))


def test_e8m0_guards():
    M, N, K = 160, 288, 128
    xa = torch.randn(M, K, device=DEV)
    xb = torch.randn(K, N, device=DEV)
    pitch = lambda n: (n + 3) // 4 * 4
    ga, gea = Guarded((M, K), torch.uint8), Guarded((K // 32, pitch(M // 32)), torch.uint8)
    P.fp8_quantize_blocked_e8m0(xa, k_major=True, q=ga.t, tile_exps=gea.t)
    ga.check("e8m0 quantize codes")
    assert torch.all(gea.buf[:gea.g] == gea.pat).item() and torch.all(gea.buf[gea.g + gea.n:] == gea.pat).item()
    qb, eb = P.fp8_quantize_blocked_e8m0(xb)
    g = Guarded((M, N), torch.float32)
    P.fp8_gemm_blockscaled_e8m0(ga.t, qb, gea.t, eb, torch.float32, C=g.t)
    g.check("fp8_gemm_blockscaled_e8m0")
    assert same(g.t, P.fp8_gemm_blockscaled_e8m0(ga.t, qb, gea.t, eb, torch.float32))


def test_sparse_guards():
    M, N, K = 200, 272, 192
    A, sa = rand_codes((M, K), 5)
    w = torch.randn(K, N, device=DEV)
    gv, gi = Guarded((K // 2, N), torch.uint8), Guarded((K // 32, N), torch.int32)
    _, _, sb, _ = P.fp8_quantize_2of4(w, vals=gv.t, idx=gi.t)
    gv.check("2:4 values")
    gi.check("2:4 positions")
    g = Guarded((M, N), torch.bfloat16)
    P.fp8_gemm_sparse24(A, gv.t, gi.t, sa, sb, torch.bfloat16, C=g.t)
    g.check("fp8_gemm_sparse24")
    assert same(g.t, P.fp8_gemm_sparse24(A, gv.t, gi.t, sa, sb, torch.bfloat16))


def test_quantize_guards():
    for n in (1, 15, 4099, 1 << 20 | 3):
        x = torch.randn(n, device=DEV)
        for fn in (P.fp8_quantize, P.fp8_quantize_e5m2):
            gq, gs, ga = Guarded((n,), torch.uint8), Guarded((1,), torch.float32), Guarded((1,), torch.float32)
            fn(x, q=gq.t, scale=gs.t, amax=ga.t)
            for g, w in ((gq, "codes"), (gs, "scale"), (ga, "amax")):
                g.check("%s n=%d %s" % (fn.__name__, n, w))
            assert same(gq.t, fn(x)[0])
    rows, cols = 300, 96
    x = torch.randn(rows, cols, device=DEV)
    off = torch.tensor([0, 0, 120, 121, rows], dtype=torch.int32, device=DEV)
    gq, gs, ga = Guarded((rows, cols), torch.uint8), Guarded((4,), torch.float32), Guarded((4,), torch.float32)
    P.fp8_quantize_grouped(x, off, q=gq.t, scales=gs.t, amax=ga.t)
    gq.check("grouped codes")
    assert torch.all(gs.buf[:gs.g] == gs.pat).item() and torch.all(gs.buf[gs.g + gs.n:] == gs.pat).item()
    assert torch.all(ga.buf[:ga.g] == ga.pat).item() and torch.all(ga.buf[ga.g + ga.n:] == ga.pat).item()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("fast", [False, True])
def test_attention_guards(causal, fast):
    BH, Sq, Skv, D = 3, 200, 333, 64
    q, sq = rand_codes((BH, Sq, D), 6)
    k, sk = rand_codes((BH, Skv, D), 7)
    v, sv = rand_codes((BH, Skv, D), 8)
    for out in (torch.float32, torch.bfloat16):
        g = Guarded((BH, Sq, D), out)
        P.fp8_attention(q, k, v, sq, sk, sv, 0.125, causal, out, O=g.t, fast=fast)
        g.check("fp8_attention causal=%s fast=%s" % (causal, fast))
        assert same(g.t, P.fp8_attention(q, k, v, sq, sk, sv, 0.125, causal, out, fast=fast))
