"""Pins of the oracle's 2:4 weight sparsity ("FP8 GEMM in JAX with Triton for
Blackwell", opening section: sparsity support, about 2x at 50% weight
sparsity): magnitude pruning along K checked by its defining invariants and
constructed ties, and the compressed (values, 2-bit positions) form checked
by round trip and a hand-made example."""
import numpy as np

import oracle


def test_prune_invariants():
    rng = np.random.default_rng(1)
    w = rng.standard_normal((64, 48)).astype(np.float32)
    p = oracle.prune_2of4(w)
    for n in range(48):
        for g in range(16):
            grp, kept = w[4 * g:4 * g + 4, n], p[4 * g:4 * g + 4, n]
            nz = kept != 0
            assert nz.sum() == 2                                   # N(0,1) has no zeros
            assert np.array_equal(kept[nz], grp[nz])               # kept values unchanged
            assert np.abs(grp[nz]).min() >= np.abs(grp[~nz]).max()  # the two largest magnitudes
    assert np.array_equal(oracle.prune_2of4(p), p)                 # idempotent


def test_prune_ties_and_already_sparse_groups():
    w = np.array([[2, 1, 0, -3, 7],
                  [2, 0, 0, 3, 7],
                  [-2, 1, 0, 0, 7],
                  [2, 0, 0, 0, 7]], np.float32)
    p = oracle.prune_2of4(w)
    assert np.array_equal(p[:, 0], [2, 2, 0, 0])       # four equal magnitudes: the lowest two k
    assert np.array_equal(p[:, 1], [1, 0, 1, 0])       # equal pair kept, zeros dropped
    assert np.array_equal(p[:, 2], [0, 0, 0, 0])
    assert np.array_equal(p[:, 3], [-3, 3, 0, 0])      # already 2:4: unchanged
    assert np.array_equal(p[:, 4], [7, 7, 0, 0])


def decompress(vals, idx, K, N):
    q = np.zeros((K, N), np.uint8)
    for n in range(N):
        for kb in range(K // 32):
            word = int(idx[kb, n])
            for e in range(16):
                g = 8 * kb + e // 2
                pos = (word >> (2 * e)) & 3
                q[4 * g + pos, n] = vals[2 * g + e % 2, n]
    return q


def test_compress_round_trip_and_positions_ascending():
    rng = np.random.default_rng(2)
    w = oracle.prune_2of4(rng.standard_normal((96, 40)).astype(np.float32))
    w[8:12, 3] = 0.0                                    # a group with no nonzero entry
    w[12:16, 5] = [0, 0, 0, 1.5]                        # a group with one
    q, _, _ = oracle.quantize_pertensor(w)
    vals, idx = oracle.compress_2of4(q)
    assert vals.shape == (48, 40) and idx.shape == (3, 40)
    assert np.array_equal(decompress(vals, idx, 96, 40), q)
    for n in range(40):
        for kb in range(3):
            word = int(idx[kb, n])
            for gg in range(8):
                assert ((word >> (4 * gg)) & 3) < ((word >> (4 * gg + 2)) & 3)   # two distinct, ascending
    # the empty group keeps positions 0, 1; the one-entry group pairs its entry with position 0
    assert (int(idx[0, 3]) >> 8) & 0xF == (0 | 1 << 2)
    assert (int(idx[0, 5]) >> 12) & 0xF == (0 | 3 << 2)


def test_compress_hand_example():
    q = np.zeros((32, 1), np.uint8)
    q[1, 0], q[3, 0] = 0x38, 0x40          # group 0: positions 1, 3
    q[4, 0], q[6, 0] = 0xB8, 0x44          # group 1: positions 0, 2
    vals, idx = oracle.compress_2of4(q)
    assert list(vals[:4, 0]) == [0x38, 0x40, 0xB8, 0x44]
    assert int(idx[0, 0]) & 0xFF == (1 | 3 << 2 | 0 << 4 | 2 << 6)
    assert int(idx[0, 0]) & ~0xFF == sum(1 << (2 * (2 * g + 1)) for g in range(2, 8))   # empty groups: 0, 1
