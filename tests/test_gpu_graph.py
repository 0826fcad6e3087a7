"""Graph capture of the hot path, through the C ABI.

The per-tensor step (quantize A, quantize B, FP8 GEMM), the block-scaled step,
the grouped (MoE) step and the attention step (quantize Q, K, V, attention)
are captured in a HIP graph (torch.cuda.CUDAGraph)
and the graph is replayed several times, with eager work between the replays
(new input values, stale values planted in every output and accumulator).
Every replay must equal, bit for bit, the same calls run eagerly on the same
inputs: the kernels are deterministic, the amax accumulators are cleared by a
fill kernel inside the captured sequence (no memset nodes), and the split-K
workspace is the caller's: nothing is called before the capture.
"""
import numpy as np
import pytest
import torch

import precision_dense_linear_amd as P
from precision_dense_linear_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
NAN = float("nan")


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def empty_like_codes(x):
    return torch.empty(x.shape, dtype=torch.uint8, device=DEV)


def replay_against_eager(inputs, make_state, step, outputs, perturb, replays=3):
    """Capture step(state_g) on a side stream, then per replay: perturb the
    inputs eagerly, plant stale values, replay, run step(state_e) eagerly and
    compare every output of the two states bit for bit."""
    st_g, st_e = make_state(), make_state()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(st_g)
    torch.cuda.synchronize()
    for i in range(replays):
        perturb(inputs, i)
        for k in outputs:
            t = st_g[k]
            t.fill_(NAN) if t.is_floating_point() else t.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        step(st_e)
        torch.cuda.synchronize()
        for k in outputs:
            a, b = st_g[k], st_e[k]
            if a.is_floating_point():
                a, b = a.view(torch.int16 if a.element_size() == 2 else torch.int32), \
                    b.view(torch.int16 if b.element_size() == 2 else torch.int32)
            assert torch.equal(a, b), "replay %d: %s differs from the eager result" % (i, k)
    return st_g


def perturb_pair(inputs, i):
    A, B = inputs
    A.mul_((-1.5, 0.25, 3.0)[i % 3])
    B.add_((0.125, -0.5, 0.0)[i % 3])


# 256x256 tiles; 128x128 tiles; 32x64 tiles with split-K; 64x64 tiles (two shapes); the skinny class (M <= 16)
# with K split 8 ways
@pytest.mark.parametrize("M,N,K", [(480, 28688, 80), (300, 5648, 272), (40, 4096, 4096), (1024, 1024, 1024),
                                   (1100, 528, 272), (16, 8192, 4096)])
@pytest.mark.parametrize("fast", [False, True])
def test_graph_pertensor_step(M, N, K, fast):
    print("graph per-tensor %dx%dx%d fast=%s" % (M, N, K, fast), flush=True)
    a, b = W.pertensor_pair(M, N, K, seed=M + 3 * N + K)
    A, B = gpu(a), gpu(b)

    def make_state():
        return {"qa": empty_like_codes(A), "qb": empty_like_codes(B),
                "sa": torch.empty(1, device=DEV), "aa": torch.empty(1, device=DEV),
                "sb": torch.empty(1, device=DEV), "ab": torch.empty(1, device=DEV),
                "C": torch.empty((M, N), dtype=torch.bfloat16, device=DEV), "ws": P.gemm_workspace(DEV)}

    def step(st):
        P.fp8_quantize(A, st["qa"], st["sa"], st["aa"])
        P.fp8_quantize(B, st["qb"], st["sb"], st["ab"])
        P.fp8_gemm(st["qa"], st["qb"], st["sa"], st["sb"], torch.bfloat16, C=st["C"], fast=fast, workspace=st["ws"])

    st = replay_against_eager((A, B), make_state, step, ["qa", "qb", "sa", "sb", "aa", "ab", "C"], perturb_pair)
    assert torch.isfinite(st["C"].float()).all()


def test_graph_blockscaled_step():
    M = N = K = 256
    print("graph block-scaled %dx%dx%d" % (M, N, K), flush=True)
    a, b = W.blockscaled_pair(M, N, K, seed=17)
    A, B = gpu(a), gpu(b)

    def make_state():
        return {"qa": empty_like_codes(A), "qb": empty_like_codes(B),
                "sa": torch.empty((M // 32, K // 32), device=DEV), "sb": torch.empty((K // 32, N // 32), device=DEV),
                "C": torch.empty((M, N), dtype=torch.bfloat16, device=DEV)}

    def step(st):
        P.fp8_quantize_blocked(A, st["qa"], st["sa"])
        P.fp8_quantize_blocked(B, st["qb"], st["sb"])
        P.fp8_gemm_blockscaled(st["qa"], st["qb"], st["sa"], st["sb"], torch.bfloat16, C=st["C"])

    replay_against_eager((A, B), make_state, step, ["qa", "qb", "sa", "sb", "C"], perturb_pair)


def test_graph_grouped_step():
    E, K, N = 4, 256, 384
    counts = np.array([300, 0, 77, 323])
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = int(off[-1])
    print("graph grouped E=%d T=%d K=%d N=%d" % (E, T, K, N), flush=True)
    rng = np.random.default_rng(23)
    X = gpu(rng.standard_normal((T, K)).astype(np.float32))
    Wt = gpu((0.02 * rng.standard_normal((E * K, N))).astype(np.float32))
    offs = gpu(off)
    woffs = gpu((np.arange(E + 1) * K).astype(np.int32))

    def make_state():
        return {"qx": empty_like_codes(X), "qw": empty_like_codes(Wt),
                "sx": torch.empty(E, device=DEV), "ax": torch.empty(E, device=DEV),
                "sw": torch.empty(E, device=DEV), "aw": torch.empty(E, device=DEV),
                "C": torch.empty((T, N), dtype=torch.bfloat16, device=DEV)}

    def step(st):
        P.fp8_quantize_grouped(X, offs, st["qx"], st["sx"], st["ax"])
        P.fp8_quantize_grouped(Wt, woffs, st["qw"], st["sw"], st["aw"])
        P.fp8_grouped_gemm(st["qx"], st["qw"].view(E, K, N), offs, st["sx"], st["sw"], torch.bfloat16, C=st["C"])

    replay_against_eager((X, Wt), make_state, step, ["qx", "qw", "sx", "sw", "ax", "aw", "C"], perturb_pair)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("fast", [False, True])
def test_graph_attention_step(causal, fast):
    BH, Sq, Skv, D = 4, 300, 333, 128
    print("graph attention BH=%d Sq=%d Skv=%d D=%d causal=%s fast=%s" % (BH, Sq, Skv, D, causal, fast), flush=True)
    rng = np.random.default_rng(29)
    Q, K, V = (gpu(rng.standard_normal(s).astype(np.float32)) for s in ((BH, Sq, D), (BH, Skv, D), (BH, Skv, D)))

    def make_state():
        st = {"q" + n: empty_like_codes(x) for n, x in (("q", Q), ("k", K), ("v", V))}
        for n in ("sq", "aq", "sk", "ak", "sv", "av"):
            st[n] = torch.empty(1, device=DEV)
        st["O"] = torch.empty((BH, Sq, D), dtype=torch.bfloat16, device=DEV)
        return st

    def step(st):
        P.fp8_quantize(Q, st["qq"], st["sq"], st["aq"])
        P.fp8_quantize(K, st["qk"], st["sk"], st["ak"])
        P.fp8_quantize(V, st["qv"], st["sv"], st["av"])
        P.fp8_attention(st["qq"], st["qk"], st["qv"], st["sq"], st["sk"], st["sv"], causal=causal, fast=fast,
                        O=st["O"])

    def perturb(inputs, i):
        q, k, v = inputs
        q.mul_((-1.5, 0.25, 3.0)[i % 3])
        k.add_((0.125, -0.5, 0.0)[i % 3])
        v.mul_((2.0, -1.0, 0.5)[i % 3])

    replay_against_eager((Q, K, V), make_state, step, ["qq", "qk", "qv", "sq", "sk", "sv", "O"], perturb)
