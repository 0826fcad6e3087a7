"""GPU parity of the quantize kernels with the CPU oracle: codes, scales and
amax must be bit-exact.  Calls go through the C ABI (via the binding)."""
import numpy as np
import pytest
import torch

import oracle
import precision_dense_linear_amd as P
from precision_dense_linear_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def quantize_and_check(x: np.ndarray, what: str):
    q, s, a = P.fp8_quantize(gpu(x))
    torch.cuda.synchronize()
    rq, rs, ra = oracle.quantize_pertensor(x)
    assert a.item() == ra and s.item() == rs, (what, a.item(), ra, s.item(), rs)
    qh = q.cpu().numpy()
    bad = qh != rq
    assert not bad.any(), "%s: %d codes differ, first at %d (x=%r gpu=%#x oracle=%#x)" % (
        what, int(bad.sum()), int(np.argmax(bad)), x.flat[np.argmax(bad)], qh.flat[np.argmax(bad)], rq.flat[np.argmax(bad)])


@pytest.mark.parametrize("n", [1, 15, 16, 17, 4095, 65536 + 7])
def test_quantize_pertensor_ragged_lengths(n):
    x = W.gaussian((n,), 3.0, n, "q")
    quantize_and_check(x, "n=%d" % n)


def test_quantize_empty_and_zero():
    q, s, a = P.fp8_quantize(torch.empty(0, dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    assert a.item() == 0.0 and s.item() == 1.0
    x = np.zeros(1000, np.float32)
    x[3] = -0.0
    quantize_and_check(x, "zeros")
    q, _, _ = P.fp8_quantize(gpu(x))
    assert q.cpu().numpy()[3] == 0x80   # sign of zero kept


def test_quantize_ties_and_saturation():
    # every E4M3 midpoint and value, scaled so that amax = 448 (scale exactly 1)
    t = oracle.e4m3_table()
    mags = np.unique(np.abs(t[~np.isnan(t)]))
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    x = np.concatenate([mids, -mids, mags.astype(np.float32), np.nextafter(mids, np.float32(0)),
                        np.nextafter(mids, np.float32(1000)), [448.0, 2.0 ** -10, -(2.0 ** -10), 1e-40]]).astype(np.float32)
    quantize_and_check(x, "ties")
    # overflow beyond the format after division: amax element saturates exactly to 448
    y = np.array([1e6, -3e5, 1.0, 464.0 * 1e6 / 448.0], np.float32)
    quantize_and_check(y, "saturation")


@pytest.mark.parametrize("shape", [(256, 256), (1024, 1024), (8192, 8192)])
def test_quantize_pertensor_operands(shape):
    a, b = W.pertensor_pair(shape[0], shape[1], shape[0], seed=1)
    quantize_and_check(a, "A%s" % (shape,))


def test_quantize_llm_shapes():
    a, w = W.llm_linear(4096, 28672, 8192)
    quantize_and_check(a, "act 4096x8192 with outlier channels")
    quantize_and_check(w, "weight 8192x28672")


def test_convert_sweep_all_fp32_patterns():
    """Every binary32 pattern with |x| <= 448 at scale exactly 1 (amax 448 appended),
    and every 61st pattern above 448 with the chunk's own scale."""
    chunk = 1 << 26
    for c0 in range(0, 1 << 32, chunk):
        bits = torch.arange(c0, c0 + chunk, dtype=torch.int64, device=DEV)
        bits = torch.where(bits >= 1 << 31, bits - (1 << 32), bits).to(torch.int32)
        x = bits.view(torch.float32)
        small = x[(x.abs() <= 448.0)]
        if small.numel():
            xs = torch.cat([small, torch.tensor([448.0], device=DEV)])
            q, s, _ = P.fp8_quantize(xs)
            assert s.item() == 1.0
            xh = xs.cpu().numpy()
            ref = oracle.quantize_with_scale(xh, 1.0)
            qh = q.cpu().numpy()
            bad = qh != ref
            assert not bad.any(), (c0, xh[bad][:4], qh[bad][:4], ref[bad][:4])
        big = x[(x.abs() > 448.0) & torch.isfinite(x)][::61]
        if big.numel():
            quantize_and_check(big.cpu().numpy(), "patterns above 448 from %#x" % c0)
        print("sweep chunk %#010x done" % c0, flush=True)


def test_quantize_blocked_8192_tile_factors_full():
    a, b = W.blockscaled_pair(8192, 8192, 8192)
    for name, x in (("A", a), ("B", b)):
        q, ts = P.fp8_quantize_blocked(gpu(x))
        torch.cuda.synchronize()
        rq, rts = oracle.quantize_blocked(x)
        assert np.array_equal(ts.cpu().numpy(), rts), name
        assert np.array_equal(q.cpu().numpy(), rq), name


def test_quantize_blocked_zero_tile_and_small():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 96)).astype(np.float32)
    x[32:, 32:64] = 0.0
    q, ts = P.fp8_quantize_blocked(gpu(x))
    rq, rts = oracle.quantize_blocked(x)
    assert np.array_equal(ts.cpu().numpy(), rts) and rts[1, 1] == 1.0
    assert np.array_equal(q.cpu().numpy(), rq)


def check_grouped(x, off, what):
    q, s, a = P.fp8_quantize_grouped(gpu(x), gpu(off.astype(np.int32)))
    torch.cuda.synchronize()
    rq, rs, ra = oracle.quantize_grouped(x, off)
    assert np.array_equal(a.cpu().numpy(), ra), what
    assert np.array_equal(s.cpu().numpy(), rs), what
    lo, hi = int(off[0]), int(off[-1])
    assert np.array_equal(q.cpu().numpy()[lo:hi], rq[lo:hi]), what


def test_quantize_grouped_moe_activations_and_weights():
    x, w, off = W.moe()
    check_grouped(x, off, "MoE activations (Zipf groups)")
    E, K, N = w.shape
    check_grouped(w.reshape(E * K, N), np.arange(E + 1) * K, "stacked expert weights")


def test_quantize_grouped_edges():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((50, 8)) * np.arange(1, 51)[:, None]).astype(np.float32)
    check_grouped(x, np.array([0, 10, 10, 33, 50]), "empty group")
    check_grouped(x, np.array([5, 20, 45]), "rows outside the groups")
    check_grouped(x, np.array([0, 50]), "one group")


def test_quantize_pertensor_many_chunks_per_workgroup():
    # 4-float chunks of 512 float4s: a length whose chunk count (6145) exceeds
    # 2048, so workgroups own several chunks, with a partial last chunk and
    # 3 trailing floats outside the float4s
    n = (6144 * 512 + 100) * 4 + 3
    x = W.gaussian((n,), 2.0, 11, "q-chunks")
    x[n // 3] = -37.5   # the amax sits in a middle workgroup's range
    x[n // 3] *= 100.0
    quantize_and_check(x, "n=%d" % n)


def test_quantize_grouped_rows_across_workgroups():
    # 5000 rows: workgroups own runs of 3 rows (up to 2048 workgroups), so
    # groups start and end inside runs; ragged column count (9 float4s)
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((5000, 36)) * rng.uniform(0.1, 50.0, (5000, 1))).astype(np.float32)
    check_grouped(x, np.array([1, 2, 1000, 1000, 1001, 2999, 4998]), "ragged groups across workgroup runs")
    check_grouped(x, np.array([0, 5000]), "one group over every run")
