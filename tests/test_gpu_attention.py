"""GPU parity of fp8_attention with the float64 oracle (oracle/attention.py),
through the C ABI, on the same seeded inputs quantized per tensor on both
sides.  Every output is held to the bound the header derives from the
kernel's arithmetic (probabilities rounded to BF16: 2^-9 each, twice through
the normalisation; FP32 accumulation over the keys; score errors of the FP32
first product; one ulp of output rounding):

    |O - O_exact| <= (1.01 (2^-8 + 4 dS) + 2^-23 (2 seq_kv + 16)) wabs
                     + 2^-22 |O_exact| + ulp_out(|O_exact| + that)

with wabs = scale_v * sum_j w_j |V[j, d]| and dS = 2^-24 (D max_j A + 6 max_j |S|)
from the oracle; with Q K^T on the FP8 matrix cores (fast=True) dS grows by
(7 * 2^-13 + 2^-21) max_j A, the FP8_ACC_FAST truncation per group of 8
products.  Shapes: ragged query and key counts on both head
dimensions, causal and not, all output types; the LLM shape (32 heads,
sequence 4096, head dimension 128) on every output; decode (one query);
queries without visible keys; no keys at all; equal scores (the mean of V);
negative scales and a scale product that underflows binary32; scores that
grow along the keys (the running max moves in the middle of the key loop)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import attention as OA
import precision_dense_linear_amd as P
from parity import bf16_to_f64, bf16_ulp, f16_to_f64, f16_ulp, to_bits

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def quantized(shape, seed):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    q, s, _ = P.fp8_quantize(gpu(x))
    oq, os_, _ = oracle.quantize_pertensor(x)
    return q, s, oq, os_


def check(O, Oex, wabs, sabs, smax, Skv, D, what, fast=False):
    if O.dtype == torch.float32:
        got = O.cpu().numpy().astype(np.float64)
        ulp = np.maximum(np.abs(Oex) * 2.0 ** -23, 2.0 ** -149)
    elif O.dtype == torch.bfloat16:
        got = bf16_to_f64(to_bits(O))
        ulp = None
    else:
        got = f16_to_f64(to_bits(O))
        ulp = None
    dS = 2.0 ** -24 * (D * sabs + 6 * smax)[..., None]
    if fast:    # Q K^T on the FP8 matrix cores: the FP8_ACC_FAST truncation per group of 8 products
        dS = dS + (7 * 2.0 ** -13 + 2.0 ** -21) * sabs[..., None]
        assert dS.max() < 0.6, "the bound's linearisation needs dS < 0.6 (max %g)" % dS.max()
    f32 = (1.01 * (2.0 ** -8 + 4 * dS) + 2.0 ** -23 * (2 * Skv + 16)) * wabs + 2.0 ** -22 * np.abs(Oex)
    at = np.abs(Oex) + f32
    if ulp is None:
        ulp = bf16_ulp(at) if O.dtype == torch.bfloat16 else f16_ulp(at)
    bound = f32 + ulp
    err = np.abs(got - Oex)
    ratio = err / bound
    bad = ~(err <= bound)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, ratio, 0)), err.shape)
        raise AssertionError("%s: %d of %d outputs outside the bound; worst %s: got %r exact %r bound %r"
                             % (what, int(bad.sum()), err.size, i, got[i], Oex[i], bound[i]))
    rel = err / np.maximum(wabs, 1e-300)
    print("%s: max err/bound %.3f, max err/wabs %.3g" % (what, ratio.max(), rel.max()), flush=True)


def run_case(BH, Sq, Skv, D, causal, out, seed, scale=None, fast=False):
    q, sq, oq, osq = quantized((BH, Sq, D), seed)
    k, sk, ok, osk = quantized((BH, Skv, D), seed + 1)
    v, sv, ov, osv = quantized((BH, Skv, D), seed + 2)
    ss = 1.0 / np.sqrt(D) if scale is None else scale
    O = P.fp8_attention(q, k, v, sq, sk, sv, float(np.float32(ss)), causal, out, fast=fast)
    torch.cuda.synchronize()
    Oex, wabs, sabs, smax = OA.attention(oq, ok, ov, osq, osk, osv, float(np.float32(ss)), causal)
    check(O, Oex, wabs, sabs, smax, Skv, D, "attention BH=%d Sq=%d Skv=%d D=%d causal=%s %s fast=%s" % (
        BH, Sq, Skv, D, causal, out, fast), fast=fast)
    return O


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Sq,Skv", [(200, 333), (128, 64), (77, 77), (300, 130)])
@pytest.mark.parametrize("fast", [False, True])
def test_ragged_shapes(Sq, Skv, D, causal, fast):
    run_case(3, Sq, Skv, D, causal, torch.bfloat16, seed=Sq + Skv + D, fast=fast)


@pytest.mark.parametrize("out", [torch.float32, torch.float16])
@pytest.mark.parametrize("fast", [False, True])
def test_output_types(out, fast):
    run_case(2, 257, 513, 128, True, out, seed=7, fast=fast)
    run_case(2, 190, 100, 64, False, out, seed=8, fast=fast)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("fast", [False, True])
def test_llm_32_heads_4096_all_outputs(causal, fast):
    print("attention 32 x 4096 x 4096 x 128 causal=%s fast=%s" % (causal, fast), flush=True)
    O1 = run_case(32, 4096, 4096, 128, causal, torch.bfloat16, seed=11, fast=fast)
    O2 = run_case(32, 4096, 4096, 128, causal, torch.bfloat16, seed=11, fast=fast)
    assert torch.equal(O1.view(torch.int16), O2.view(torch.int16))      # deterministic


def test_decode_one_query_and_long_keys():
    run_case(8, 1, 4097, 128, False, torch.bfloat16, seed=21)
    run_case(8, 1, 4097, 128, True, torch.float32, seed=22)
    run_case(8, 1, 4097, 128, True, torch.float32, seed=23, fast=True)


def test_queries_without_keys_and_no_keys():
    O = run_case(2, 100, 40, 64, True, torch.float32, seed=31)     # causal: the first 60 queries see no key
    assert torch.count_nonzero(O[:, :60]).item() == 0
    q, sq, _, _ = quantized((2, 50, 64), 32)
    empty = torch.zeros((2, 0, 64), dtype=torch.uint8, device=DEV)
    O = torch.full((2, 50, 64), float("nan"), device=DEV)
    P.fp8_attention(q, empty, empty, sq, sq, sq, 0.125, False, torch.float32, O=O)
    assert torch.count_nonzero(O).item() == 0


@pytest.mark.parametrize("fast", [False, True])
def test_negative_and_underflowing_scale_products(fast):
    q, sq, oq, osq = quantized((2, 150, 128), 51)
    k, sk, ok, osk = quantized((2, 200, 128), 52)
    v, sv, ov, osv = quantized((2, 200, 128), 53)
    ss = float(np.float32(1 / np.sqrt(128)))
    tiny = np.float32(1e-30)
    dtiny = torch.full((1,), float(tiny), device=DEV)
    for causal in (False, True):
        # a negative scale product (the kernel moves the sign onto Q's codes)
        O = P.fp8_attention(q, k, v, -sq, sk, -sv, ss, causal, torch.bfloat16, fast=fast)
        Oex, wabs, sabs, smax = OA.attention(oq, ok, ov, -osq, osk, -osv, ss, causal)
        check(O, Oex, wabs, sabs, smax, 200, 128, "negative scales causal=%s fast=%s" % (causal, fast), fast=fast)
        # scale_q * scale_k underflows to 0 in binary32: every visible score
        # is (all but) zero, so each query averages the V rows it sees
        O = P.fp8_attention(q, k, v, dtiny, dtiny, sv, ss, causal, torch.float32, fast=fast)
        Oex, wabs, sabs, smax = OA.attention(oq, ok, ov, tiny, tiny, osv, ss, causal)
        check(O, Oex, wabs, sabs, smax, 200, 128, "underflowing scales causal=%s fast=%s" % (causal, fast), fast=fast)


def test_equal_scores_give_the_mean_of_v():
    BH, Sq, Skv, D = 2, 130, 200, 128
    q = torch.zeros((BH, Sq, D), dtype=torch.uint8, device=DEV)
    one = torch.ones(1, device=DEV)
    v, sv, ov, osv = quantized((BH, Skv, D), 41)
    k, sk, _, _ = quantized((BH, Skv, D), 42)
    O = P.fp8_attention(q, k, v, one, sk, sv, 0.1, False, torch.float32).cpu().numpy()
    mean = oracle.decode(ov).mean(axis=1) * float(osv)            # every probability is exactly 1
    assert np.allclose(O, np.broadcast_to(mean[:, None, :], O.shape), rtol=0,
                       atol=2.0 ** -20 * float(np.abs(oracle.decode(ov)).max()) * float(osv))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("ss,fast", [(0.25, False), (1.0, False), (4.0, False), (0.25, True)])
def test_scores_growing_along_the_keys(ss, fast, causal):
    """Key rows scaled up along the sequence (x1 to x4), so a query's running
    max keeps growing from block to block -- by a few log2 units at the
    smallest score scale, by far more than the largest finite exponential at
    the largest -- and the lazily kept exponent offsets must be moved (and the
    accumulators rescaled) in the middle of the key loop."""
    BH, Sq, Skv, D = 2, 130, 700, 128
    rng = np.random.default_rng(61)
    xq = rng.standard_normal((BH, Sq, D)).astype(np.float32)
    ramp = (1.0 + 3.0 * np.arange(Skv) / (Skv - 1)).astype(np.float32)
    xk = (rng.standard_normal((BH, Skv, D)) * ramp[None, :, None]).astype(np.float32)
    xv = rng.standard_normal((BH, Skv, D)).astype(np.float32)
    (q, sq, _), (k, sk, _), (v, sv, _) = (P.fp8_quantize(gpu(x)) for x in (xq, xk, xv))
    (oq, osq, _), (ok, osk, _), (ov, osv, _) = (oracle.quantize_pertensor(x) for x in (xq, xk, xv))
    s32 = float(np.float32(ss))
    O = P.fp8_attention(q, k, v, sq, sk, sv, s32, causal, torch.float32, fast=fast)
    torch.cuda.synchronize()
    Oex, wabs, sabs, smax = OA.attention(oq, ok, ov, osq, osk, osv, s32, causal)
    check(O, Oex, wabs, sabs, smax, Skv, D, "growing scores ss=%g causal=%s fast=%s" % (ss, causal, fast), fast=fast)
