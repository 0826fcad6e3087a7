"""CPU oracle of FP8 multi-head attention -- test infrastructure only.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the product library never does and
shares no code with it.

What it computes ("Leveraging CUTLASS kernel naming in Triton for a 100
TFLOPS FP8 tensor-core speed-up in multi-head attention", blog.hotdry.top:
the fp8_mha_kernel sketch -- Q K^T as an FP8 dot product, then the softmax
and the accumulation of V fused into the same kernel -- and its parameter
list -- 32 heads, sequence length 4096).  The page leaves the softmax out
("softmax logic" placeholder); it is read as standard scaled dot-product
attention.  For every head h and query row i:

    S[i, j] = (scale_q * scale_k * softmax_scale) * sum_d Q[h, i, d] * K[h, j, d]
    P[i, j] = exp(S[i, j] - max_j' S[i, j']) / sum_j' exp(S[i, j'] - max_j' S[i, j'])
    O[h, i, d] = scale_v * sum_j P[i, j] * V[h, j, d]

over the keys j visible to i: all of them, or with ``causal`` those with
j <= i + (seq_kv - seq_q) (the last query sees every key).  A query that
sees no key has O = 0.  Q, K, V are E4M3 codes (per-tensor scales, as the
GEMM pages quantize, amax / 448), decoded exactly; the dot products of
decoded codes are exact in float64 (each product is a multiple of 2^-18
below 2^18, a sum of at most 2^10 of them stays below 2^53), the softmax and
the second product are evaluated in float64.
"""
from __future__ import annotations

import numpy as np


def _decode(q: np.ndarray) -> np.ndarray:
    from . import decode
    return decode(np.ascontiguousarray(q, dtype=np.uint8))


def visible(seq_q: int, seq_kv: int, causal: bool) -> np.ndarray:
    """Bool [seq_q, seq_kv]: key j is visible to query i."""
    if not causal:
        return np.ones((seq_q, seq_kv), bool)
    i = np.arange(seq_q)[:, None]
    j = np.arange(seq_kv)[None, :]
    return j <= i + (seq_kv - seq_q)


def attention(qq, qk, qv, scale_q, scale_k, scale_v, softmax_scale, causal=False):
    """qq [BH, Sq, D], qk and qv [BH, Skv, D] E4M3 codes (uint8); returns
    float64 arrays:
      O      [BH, Sq, D]  the attention output;
      wabs   [BH, Sq, D]  |scale_v| * sum_j P[i, j] * |V[h, j, d]| (the scale of
                          the second product's rounding errors);
      sabs   [BH, Sq]     max over visible j of |scale_q * scale_k *
                          softmax_scale| * sum_d |Q[h, i, d] * K[h, j, d]|
                          (the scale of the first product's);
      smax   [BH, Sq]     max over visible j of |S[i, j]|."""
    Q, K, V = _decode(qq), _decode(qk), _decode(qv)
    BH, Sq, D = Q.shape
    Skv = K.shape[1]
    assert K.shape == (BH, Skv, D) and V.shape == (BH, Skv, D)
    c = float(scale_q) * float(scale_k) * float(softmax_scale)
    vis = visible(Sq, Skv, causal)
    any_vis = vis.any(axis=1)
    O = np.zeros((BH, Sq, D))
    wabs = np.zeros((BH, Sq, D))
    sabs = np.zeros((BH, Sq))
    smax = np.zeros((BH, Sq))
    for h in range(BH):
        dots = Q[h] @ K[h].T                      # exact sums of exact products
        S = np.where(vis, dots * c, -np.inf)
        m = np.where(any_vis, S.max(axis=1, initial=-np.inf), 0.0)
        E = np.where(vis, np.exp(S - m[:, None]), 0.0)
        L = E.sum(axis=1)
        W = np.divide(E, L[:, None], out=np.zeros_like(E), where=L[:, None] > 0)
        O[h] = (W @ V[h]) * float(scale_v)
        wabs[h] = (W @ np.abs(V[h])) * abs(float(scale_v))
        A = np.where(vis, (np.abs(Q[h]) @ np.abs(K[h]).T) * abs(c), 0.0)
        sabs[h] = A.max(axis=1, initial=0.0)
        smax[h] = np.where(vis, np.abs(S), 0.0).max(axis=1, initial=0.0)
    return O, wabs, sabs, smax


def flops(BH: int, seq_q: int, seq_kv: int, D: int, causal: bool) -> float:
    """Multiply-add flops of the two products over the visible pairs."""
    pairs = float(visible(seq_q, seq_kv, causal).sum()) if causal else float(seq_q) * seq_kv
    return 4.0 * BH * pairs * D
