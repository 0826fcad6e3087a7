"""Pins of the attention oracle (oracle/attention.py) to facts outside it:
a pure-Python brute force with exact dot products (fractions) and math.exp,
closed forms (equal scores give the mean of the visible V rows; one dominant
score gives that V row; a causal first row sees only key 0; a query with no
visible key gives 0), torch's float64 scaled_dot_product_attention on the
decoded inputs (a library routine), and invariances (permuting the keys
together with the values; the output scales with scale_v; only the product
of the score scales matters).  Shapes are tiny or small: CPU only."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as OA


def codes(shape, seed, lim=448.0):
    """Random finite E4M3 codes from scaled N(0, 1) values."""
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    x *= np.float32(lim / max(1e-30, float(np.abs(x).max())))
    return oracle.convert(x).reshape(shape)


def brute_force(qq, qk, qv, sq, sk, sv, scale, causal):
    """Scalar loops: exact dot products (Fraction), math.exp, float sums."""
    Q, K, V = (oracle.decode(a) for a in (qq, qk, qv))
    BH, Sq, D = Q.shape
    Skv = K.shape[1]
    out = np.zeros((BH, Sq, D))
    c = Fraction(float(sq)) * Fraction(float(sk)) * Fraction(float(scale))
    for h in range(BH):
        for i in range(Sq):
            keys = [j for j in range(Skv) if not causal or j <= i + (Skv - Sq)]
            if not keys:
                continue
            s = {j: float(c * sum(Fraction(float(Q[h, i, d])) * Fraction(float(K[h, j, d])) for d in range(D)))
                 for j in keys}
            m = max(s.values())
            e = {j: math.exp(s[j] - m) for j in keys}
            tot = math.fsum(e.values())
            for d in range(D):
                out[h, i, d] = math.fsum(e[j] * float(V[h, j, d]) for j in keys) / tot * float(sv)
    return out


@pytest.mark.parametrize("Sq,Skv,causal", [(3, 5, False), (5, 5, True), (4, 7, True), (6, 3, True)])
def test_brute_force_tiny(Sq, Skv, causal):
    BH, D = 2, 8
    qq, qk, qv = codes((BH, Sq, D), 1), codes((BH, Skv, D), 2), codes((BH, Skv, D), 3)
    sq, sk, sv, scale = np.float32(0.0123), np.float32(0.0071), np.float32(0.5), 0.35
    O, wabs, sabs, smax = OA.attention(qq, qk, qv, sq, sk, sv, scale, causal)
    ref = brute_force(qq, qk, qv, sq, sk, sv, scale, causal)
    assert np.allclose(O, ref, rtol=1e-13, atol=1e-13 * float(np.abs(ref).max()))
    assert np.all(wabs + 1e-12 >= np.abs(O)) and np.all(sabs + 1e-12 >= smax)


def test_equal_scores_give_the_mean_of_v():
    BH, Sq, Skv, D = 2, 6, 9, 16
    qq = np.zeros((BH, Sq, D), np.uint8)                  # Q = 0: every score is 0
    qk, qv = codes((BH, Skv, D), 4), codes((BH, Skv, D), 5)
    O, _, _, _ = OA.attention(qq, qk, qv, 1.0, 1.0, 0.25, 1.0, False)
    V = oracle.decode(qv)
    tol = 1e-14 * float(np.abs(V).max())              # float64 rounding of the weighted sums
    assert np.allclose(O, np.broadcast_to(V.mean(axis=1, keepdims=True) * 0.25, O.shape), rtol=0, atol=tol)
    Oc, _, _, _ = OA.attention(qq, qk, qv, 1.0, 1.0, 0.25, 1.0, True)        # causal, Sq < Skv
    for i in range(Sq):
        n = i + (Skv - Sq) + 1
        assert np.allclose(Oc[:, i], V[:, :n].mean(axis=1) * 0.25, rtol=0, atol=tol)


def test_one_dominant_score_gives_its_v_row():
    BH, Skv, D = 1, 10, 32
    one = oracle.convert(np.array([448.0], np.float32))[0]
    qq = np.full((BH, 1, D), one, np.uint8)
    qk = np.zeros((BH, Skv, D), np.uint8)
    qk[0, 6] = one                                       # score 448^2 * 32 against 0 for every other key
    qv = codes((BH, Skv, D), 6)
    O, _, _, _ = OA.attention(qq, qk, qv, 1.0, 1.0, 2.0, 1.0, False)
    assert np.array_equal(O[0, 0], oracle.decode(qv)[0, 6] * 2.0)


def test_causal_first_row_and_rows_without_keys():
    BH, D = 2, 16
    qq, qk, qv = codes((BH, 8, D), 7), codes((BH, 8, D), 8), codes((BH, 8, D), 9)
    O, _, _, _ = OA.attention(qq, qk, qv, 0.01, 0.02, 3.0, 0.1, True)
    assert np.array_equal(O[:, 0], oracle.decode(qv)[:, 0] * 3.0)           # query 0 sees key 0 only
    O2, wabs, _, _ = OA.attention(qq, qk[:, :5], qv[:, :5], 0.01, 0.02, 3.0, 0.1, True)
    assert np.all(O2[:, :3] == 0) and np.all(wabs[:, :3] == 0)              # 8 queries, 5 keys: 3 see none
    assert np.array_equal(O2[:, 3], oracle.decode(qv)[:, 0] * 3.0)


@pytest.mark.parametrize("causal,Sq,Skv", [(False, 33, 70), (True, 48, 48), (True, 20, 45)])
def test_matches_torch_sdpa_float64(causal, Sq, Skv):
    BH, D = 3, 64
    qq, qk, qv = codes((BH, Sq, D), 10), codes((BH, Skv, D), 11), codes((BH, Skv, D), 12)
    sq, sk, sv, scale = 0.004, 0.003, 0.7, 1 / 8
    O, _, _, _ = OA.attention(qq, qk, qv, sq, sk, sv, scale, causal)
    q = torch.from_numpy(oracle.decode(qq) * sq)
    k = torch.from_numpy(oracle.decode(qk) * sk)
    v = torch.from_numpy(oracle.decode(qv) * sv)
    mask = torch.ones(Sq, Skv, dtype=torch.bool).tril(diagonal=Skv - Sq) if causal else None
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale).numpy()
    assert np.allclose(O, ref, rtol=1e-12, atol=1e-12 * float(np.abs(ref).max()))


def test_key_permutation_and_scale_invariances():
    BH, Sq, Skv, D = 2, 12, 40, 32
    qq, qk, qv = codes((BH, Sq, D), 13), codes((BH, Skv, D), 14), codes((BH, Skv, D), 15)
    O, _, _, _ = OA.attention(qq, qk, qv, 0.02, 0.01, 1.0, 0.2, False)
    perm = np.random.default_rng(16).permutation(Skv)
    Op, _, _, _ = OA.attention(qq, qk[:, perm], qv[:, perm], 0.02, 0.01, 1.0, 0.2, False)
    assert np.allclose(Op, O, rtol=1e-14, atol=1e-14 * float(np.abs(O).max()))
    O3, _, _, _ = OA.attention(qq, qk, qv, 0.04, 0.005, 0.5, 0.2, False)    # same score scale, half scale_v
    assert np.allclose(O3, O * 0.5, rtol=1e-14, atol=1e-14 * float(np.abs(O).max()))


def test_negative_scale_equals_negated_q_codes():
    # S = c * (Q K^T): a negative scale_q is the same as Q with every sign bit
    # flipped (E4M3 sign-magnitude codes) and the positive scale; the error
    # scales stay non-negative
    BH, Sq, Skv, D = 2, 9, 30, 64
    qq, qk, qv = codes((BH, Sq, D), 17), codes((BH, Skv, D), 18), codes((BH, Skv, D), 19)
    for causal in (False, True):
        On, wn, an, mn = OA.attention(qq, qk, qv, -0.03, 0.02, -0.5, 0.125, causal)
        Op, wp, ap, mp = OA.attention(qq ^ np.uint8(0x80), qk, qv, 0.03, 0.02, 0.5, 0.125, causal)
        assert np.array_equal(On, -Op) and np.array_equal(wn, wp) and np.array_equal(an, ap) and np.array_equal(mn, mp)
        assert np.all(wn >= 0) and np.all(an >= 0)


def test_flops_counts_visible_pairs():
    assert OA.flops(2, 4, 4, 8, False) == 4.0 * 2 * 16 * 8
    assert OA.flops(2, 4, 4, 8, True) == 4.0 * 2 * 10 * 8
