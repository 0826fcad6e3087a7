"""Seeded synthetic inputs for the scaled FP8 GEMM workloads.

This module only draws random numbers and lays them out; it holds no
quantization, rounding or GEMM arithmetic, so that the HIP path and the CPU
oracle can both be fed from it without sharing any of the method.

Every generator is deterministic in ``seed``: each tensor gets its own
numpy ``Generator(PCG64)`` stream, derived from (seed, tensor name).

Workloads (shapes follow the LLM linear layers and MoE experts the pages
motivate the FP8 GEMM with):

* ``pertensor_pair``  -- A (M x K), B (K x N), entries N(0, 1).
* ``llm_linear``      -- activations A N(0, 1) with 1% outlier channels
                         (columns of A, i.e. K indices) scaled by 20, the same
                         channel set for every M; weights B N(0, 0.02).
* ``blockscaled_pair``-- A, B N(0, 1), each 32 x 32 tile multiplied by its own
                         factor 10^U(-2, 2).
* ``moe``             -- E experts, T routed tokens with Zipf(s) expert
                         popularity (p_e proportional to (e+1)^-s, one i.i.d.
                         draw per token, rows grouped by expert), X (T x K)
                         N(0, 1), W (E x K x N) N(0, 0.02).
* ``attention_qkv``   -- Q [heads, seq_q, D], K and V [heads, seq_kv, D],
                         entries N(0, 1) (the attention page's LLM setting:
                         32 heads, sequence 4096, head dimension 128).
"""
from __future__ import annotations

import zlib

import numpy as np


def rng(seed: int, name: str) -> np.random.Generator:
    """Independent PCG64 stream for tensor ``name`` under ``seed``."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), zlib.crc32(name.encode())])))


def gaussian(shape, std: float, seed: int, name: str) -> np.ndarray:
    x = rng(seed, name).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def pertensor_pair(M: int, N: int, K: int, seed: int = 0):
    """A (M x K) and B (K x N), float32 N(0, 1), row-major."""
    return gaussian((M, K), 1.0, seed, "A"), gaussian((K, N), 1.0, seed, "B")


def outlier_channels(K: int, seed: int = 0, frac: float = 0.01) -> np.ndarray:
    """round(frac*K) distinct channel (K) indices, sorted."""
    n = int(round(frac * K))
    return np.sort(rng(seed, "outlier-channels").permutation(K)[:n])


def llm_linear(M: int, N: int, K: int, seed: int = 0, outlier_gain: float = 20.0):
    """Activations N(0,1) with 1% outlier channels x20 (same set for all M), weights N(0, 0.02)."""
    a = gaussian((M, K), 1.0, seed, "act-%d" % M)
    ch = outlier_channels(K, seed)
    a[:, ch] *= np.float32(outlier_gain)
    w = gaussian((K, N), 0.02, seed, "weight-%dx%d" % (K, N))
    return a, w


def tile_factors(rows: int, cols: int, seed: int, name: str, lo: float = -2.0, hi: float = 2.0,
                 tile: int = 32) -> np.ndarray:
    """One factor 10^U(lo, hi) per tile x tile tile: float32[rows/tile, cols/tile]."""
    u = rng(seed, name + "-tiles" + ("" if tile == 32 else "%d" % tile)).uniform(lo, hi,
                                                                              size=(rows // tile, cols // tile))
    return np.power(10.0, u).astype(np.float32)


def expand_tiles(f: np.ndarray, tile: int = 32) -> np.ndarray:
    return np.repeat(np.repeat(f, tile, axis=0), tile, axis=1)


def blockscaled_pair(M: int, N: int, K: int, seed: int = 0, tile: int = 32):
    """A, B N(0,1), each tile x tile tile (32 or 64) times its own log-uniform factor in [1e-2, 1e2]."""
    a, b = pertensor_pair(M, N, K, seed)
    a *= expand_tiles(tile_factors(M, K, seed, "A", tile=tile), tile)
    b *= expand_tiles(tile_factors(K, N, seed, "B", tile=tile), tile)
    return a, b


def zipf_counts(E: int, T: int, s: float = 1.2, seed: int = 0) -> np.ndarray:
    """Tokens per expert: each of T tokens picks expert e with p proportional to (e+1)^-s."""
    p = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    pick = rng(seed, "routing").choice(E, size=T, p=p)
    return np.bincount(pick, minlength=E).astype(np.int64)


def offsets_from_counts(counts) -> np.ndarray:
    off = np.zeros(len(counts) + 1, dtype=np.int32)
    off[1:] = np.cumsum(counts)
    return off


def moe(E: int = 8, T: int = 16384, K: int = 4096, N: int = 14336, seed: int = 0, s: float = 1.2):
    """(X T x K, W E x K x N, offsets int32[E+1]); rows of X grouped by expert."""
    counts = zipf_counts(E, T, s, seed)
    x = gaussian((T, K), 1.0, seed, "moe-x")
    w = np.empty((E, K, N), dtype=np.float32)
    for e in range(E):
        w[e] = gaussian((K, N), 0.02, seed, "moe-w%d" % e)
    return x, w, offsets_from_counts(counts)


def attention_qkv(heads: int = 32, seq_q: int = 4096, seq_kv: int = 4096, D: int = 128, seed: int = 0):
    return (gaussian((heads, seq_q, D), 1.0, seed, "Q"), gaussian((heads, seq_kv, D), 1.0, seed, "K"),
            gaussian((heads, seq_kv, D), 1.0, seed, "V"))
