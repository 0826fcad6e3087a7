"""Benchmark of the scaled FP8 GEMM hot path on one MI355X.

One step = the whole per-tensor path on FP32 inputs already resident in HBM:
amax + scale + E4M3 quantization of A and of B, then the FP8 GEMM with FP32
accumulation and the fused scale/BF16 epilogue.  The default workload is the
M = N = K = 8192 GEMM with BF16 output (A, B drawn N(0, 1) from a seed).

Printed (rank 0, one JSON line):
  value       -- the metric: the FP8 GEMM kernel alone, 2*M*N*K / its average
                 launch time inside the timed steps, measured with HIP events
                 on the launch stream (TFLOP/s; default exact-product mode)
  pct_fp8_peak-- value as a percentage of the dense FP8 MFMA peak (5.0 PFLOP/s)
  ms_per_step -- the whole step (quantize A, quantize B, GEMM) per step;
                 step_tflops = 2*M*N*K / ms_per_step
  roofline    -- that GEMM kernel against its roofline: the dense FP8 MFMA
                 peak for every GEMM on FP8 operands (the default mode
                 multiplies on the BF16 matrix cores, whose peak is half of
                 it: frac_of_bf16_peak), or HBM for the memory-bound shapes,
                 whose launches are then timed back to back over rotating
                 copies of the operand codes that add up to more than twice
                 the 256 MB MALL (repeated launches on one B would be served
                 from the MALL, not HBM); kernels shorter than the host's
                 launch cost are replayed from a HIP graph
  sclk        -- the GPU clock sampled during the timed region, and the
                 GEMM's fraction of the MFMA peak at that clock
  vendor_same_box -- context only: hipBLASLt's FP8 and BF16 GEMMs (through
                 torch) on the same codes and shape, timed the same way
                 (BF16 with B as an N x K weight, and with row-major B)
  cpu_baseline-- the CPU oracle timed on a bounded sample of the same step
Other workloads (--workload) serve profiling of the other shape classes.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 MFMA (published; 256 CU x 8192 flop/clk x 2.4 GHz = 5033)
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense BF16 MFMA (published)
HBM_PEAK_GBPS = 8000.0     # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
CUS, FP8_FLOP_PER_CU_CLK, BF16_FLOP_PER_CU_CLK = 256, 8192, 4096


class SclkSampler:
    """Polls the current shader clock (the '*' line of pp_dpm_sclk in sysfs)
    from a background thread; mean_mhz() is None where the file is absent."""

    def __init__(self, period_s: float = 0.002):
        import glob
        import threading
        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        for p in self.paths:
            try:
                for line in open(p):
                    if line.rstrip().endswith("*"):
                        return float(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
            except (OSError, ValueError, IndexError):
                continue
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.paths:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.paths:
            self._thread.join()

    def mean_mhz(self):
        # samples at an idle level (under 500 MHz) are gaps between launches
        busy = [v for v in self.samples if v >= 500.0]
        return float(np.mean(busy)) if busy else None


# The sources the 8192^3 per-tensor GEMM kernel is compiled from: its
# committed byte counters stay valid while these are unchanged.
HEADLINE_SOURCES = ("device_utils.h", "gemm_common.h", "gemm_kernel.h", "gemm_dispatch.h", "launch.h", "gemm.hip")


def csrc_sha256(names=HEADLINE_SOURCES):
    import hashlib
    h = hashlib.sha256()
    for n in sorted(names):
        h.update(n.encode())
        h.update(open(os.path.join(ROOT, "precision_dense_linear_amd", "csrc", n), "rb").read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per GEMM launch from the committed rocprofv3 byte counters, if
    they were taken on the kernel's sources as they are now (else None)."""
    path = os.path.join(PROFILES, {"gemm8192": "gemm_kernel_8192x8192x8192_bf16.traffic.json"}.get(workload, "-"))
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    return rec["traffic_bytes"] if rec.get("csrc_sha256") == csrc_sha256() else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gemm8192",
                    choices=["gemm8192", "gemm1024", "gemm256", "llm16", "llm128", "llm4096", "blockscaled8192",
                             "moe", "mixed8192", "blockscaled8192_64", "blockscaled8192_e8m0", "sparse8192",
                             "sparse_llm4096", "attn4096", "attn4096_causal"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-vendor", action="store_true", help="skip timing the vendor GEMM library for comparison")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy twice (reference for the HBM byte counters)")
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="keep warming up at least this long so clocks have settled")
    ap.add_argument("--cpu-rows", type=int, default=4096, help="rows of A in the oracle's timed sample (about 10 s of CPU work at 8192^3)")
    return ap.parse_args()


class Workload:
    """Inputs resident on the GPU and one step of the hot path."""

    def __init__(self, name, dev):
        import torch
        import precision_dense_linear_amd as P
        from precision_dense_linear_amd import workloads as W
        self.P, self.torch, self.name = P, torch, name
        g = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        self.kind = "pertensor"
        self.out = torch.bfloat16
        self.b_e5m2 = False
        if name == "mixed8192":
            self.M = self.N = self.K = 8192
            a, b = W.pertensor_pair(8192, 8192, 8192, seed=0)
            self.out = torch.float16
            self.b_e5m2 = True
            self.desc = ("mixed-format per-tensor FP8 GEMM M=N=K=8192, FP16 out; A FP32 N(0,1) quantized to e4m3fn, "
                         "B FP32 N(0,1) quantized to e5m2, on device")
        elif name.startswith("gemm"):
            n = int(name[4:])
            self.M = self.N = self.K = n
            a, b = W.pertensor_pair(n, n, n, seed=0)
            self.desc = "per-tensor FP8 GEMM M=N=K=%d, BF16 out; A, B FP32 N(0,1) quantized to e4m3fn on device" % n
            if n == 256:
                self.out = torch.float32
                self.desc = self.desc.replace("BF16", "FP32")
        elif name.startswith("llm"):
            self.M = int(name[3:])
            self.N = 8192 if self.M == 16 else 28672
            self.K = 8192
            a, b = W.llm_linear(self.M, self.N, self.K)
            self.desc = ("LLM linear layer M=%d N=%d K=%d, per-tensor FP8, BF16 out; activations N(0,1) with 1%% "
                         "outlier channels x20, weights N(0,0.02)" % (self.M, self.N, self.K))
        elif name.startswith("sparse"):
            self.kind = "sparse"
            if name == "sparse8192":
                self.M = self.N = self.K = 8192
                a, b = W.pertensor_pair(8192, 8192, 8192, seed=0)
                self.desc = ("per-tensor FP8 GEMM M=N=K=8192 with B 2:4-pruned along K on the sparse matrix cores, BF16 "
                             "out; A, B FP32 N(0,1)")
            else:
                self.M, self.N, self.K = 4096, 28672, 8192
                a, b = W.llm_linear(self.M, self.N, self.K)
                self.desc = ("LLM linear layer M=4096 N=28672 K=8192 with the weights 2:4-pruned along K on the sparse "
                             "matrix cores, BF16 out; activations N(0,1) with 1% outlier channels x20, weights N(0,0.02)")
        elif name == "blockscaled8192_e8m0":
            self.kind = "block_e8"
            self.M = self.N = self.K = 8192
            a, b = W.blockscaled_pair(8192, 8192, 8192)
            self.desc = ("block-scaled FP8 GEMM M=N=K=8192 with power-of-two (E8M0) 32x32 tile scales applied by the "
                         "FP8 matrix cores, BF16 out; tile factors 10^U(-2,2)")
        elif name.startswith("attn"):
            self.kind = "attn"
            self.causal = name.endswith("causal")
            self.heads, S, D = 32, 4096, 128
            q, k, v = W.attention_qkv(self.heads, S, S, D)
            a, b = q, np.stack([k, v])
            self.M, self.N, self.K = S, D, S          # seq_q, head_dim, seq_kv
            self.desc = ("FP8 multi-head attention: 32 heads, seq_q = seq_kv = 4096, head_dim 128, %s, BF16 out; "
                         "Q, K, V FP32 N(0,1) quantized per tensor to e4m3fn on device"
                         % ("causal" if self.causal else "non-causal"))
        elif name.startswith("blockscaled8192"):
            self.kind = "block"
            self.block = 64 if name.endswith("_64") else 32
            self.M = self.N = self.K = 8192
            a, b = W.blockscaled_pair(8192, 8192, 8192, tile=self.block)
            self.desc = ("block-scaled (%dx%d tiles) FP8 GEMM M=N=K=8192, BF16 out; tile factors 10^U(-2,2)"
                         % (self.block, self.block))
        else:
            self.kind = "moe"
            x, w, off = W.moe()
            self.E, self.K, self.N = w.shape
            self.M = x.shape[0]
            a, b = x, w.reshape(self.E * self.K, self.N)
            self.off = g(off.astype(np.int32))
            self.woff = g((np.arange(self.E + 1) * self.K).astype(np.int32))
            self.desc = ("MoE grouped FP8 GEMM: 8 experts, 16384 tokens with Zipf(1.2) counts %s, K=4096, N=14336, "
                         "BF16 out" % list(np.diff(off)))
        self.a_host, self.b_host = a, b
        self.A, self.B = g(a), g(b)
        self.qa = torch.empty(a.shape, dtype=torch.uint8, device=dev)
        self.qb = torch.empty(b.shape, dtype=torch.uint8, device=dev)
        if self.kind == "sparse":
            self.qb = torch.empty((self.K // 2, self.N), dtype=torch.uint8, device=dev)
            self.qi = torch.empty((self.K // 32, self.N), dtype=torch.int32, device=dev)
        self.C = torch.empty((self.M, self.N), dtype=self.out, device=dev)
        self.ws = P.gemm_workspace(dev)  # split-K workspace (used by the few-tile shapes, M <= 64)
        if self.kind == "attn":
            self.C = torch.empty(a.shape, dtype=self.out, device=dev)
            self.sa, self.aa, self.sb, self.ab, self.sv, self.av = (torch.empty(1, device=dev) for _ in range(6))
        elif self.kind in ("pertensor", "sparse"):
            self.sa, self.aa = (torch.empty(1, device=dev) for _ in range(2))
            self.sb, self.ab = (torch.empty(1, device=dev) for _ in range(2))
        elif self.kind == "block_e8":
            pitch = lambda n: (n + 3) // 4 * 4
            self.sa = torch.empty((self.K // 32, pitch(self.M // 32)), dtype=torch.uint8, device=dev)
            self.sb = torch.empty((self.K // 32, pitch(self.N // 32)), dtype=torch.uint8, device=dev)
        elif self.kind == "block":
            self.sa = torch.empty((self.M // self.block, self.K // self.block), device=dev)
            self.sb = torch.empty((self.K // self.block, self.N // self.block), device=dev)
        else:
            self.sa, self.aa = (torch.empty(self.E, device=dev) for _ in range(2))
            self.sb, self.ab = (torch.empty(self.E, device=dev) for _ in range(2))
        self.flops = 2.0 * self.M * self.N * self.K
        if self.kind == "attn":    # both products over the visible (query, key) pairs
            pairs = self.M * (self.M + 1) / 2 if self.causal else float(self.M) * self.K
            self.flops = 4.0 * self.heads * pairs * self.N

    def quantize(self):
        P = self.P
        if self.kind == "attn":
            P.fp8_quantize(self.A, self.qa, self.sa, self.aa)
            P.fp8_quantize(self.B[0], self.qb[0], self.sb, self.ab)
            P.fp8_quantize(self.B[1], self.qb[1], self.sv, self.av)
        elif self.kind == "pertensor":
            P.fp8_quantize(self.A, self.qa, self.sa, self.aa)
            (P.fp8_quantize_e5m2 if self.b_e5m2 else P.fp8_quantize)(self.B, self.qb, self.sb, self.ab)
        elif self.kind == "sparse":
            P.fp8_quantize(self.A, self.qa, self.sa, self.aa)
            P.fp8_quantize_2of4(self.B, self.qb, self.qi, self.sb, self.ab)
        elif self.kind == "block_e8":
            P.fp8_quantize_blocked_e8m0(self.A, True, self.qa, self.sa)
            P.fp8_quantize_blocked_e8m0(self.B, False, self.qb, self.sb)
        elif self.kind == "block":
            qb = P.fp8_quantize_blocked64 if self.block == 64 else P.fp8_quantize_blocked
            qb(self.A, self.qa, self.sa)
            qb(self.B, self.qb, self.sb)
        else:
            P.fp8_quantize_grouped(self.A, self.off, self.qa, self.sa, self.aa)
            P.fp8_quantize_grouped(self.B, self.woff, self.qb, self.sb, self.ab)

    def gemm(self, fast=False, qa=None, qb=None):
        P = self.P
        qa = self.qa if qa is None else qa
        qb = self.qb if qb is None else qb
        if self.kind == "attn":
            P.fp8_attention(qa, qb[0], qb[1], self.sa, self.sb, self.sv, None, self.causal, self.out, O=self.C,
                            fast=fast)
        elif self.kind == "pertensor":
            P.fp8_gemm(qa, qb, self.sa, self.sb, self.out, C=self.C, fast=fast,
                       b_fmt="e5m2" if self.b_e5m2 else "e4m3", workspace=self.ws)
        elif self.kind == "sparse":
            P.fp8_gemm_sparse24(qa, qb, self.qi, self.sa, self.sb, self.out, C=self.C)
        elif self.kind == "block_e8":
            P.fp8_gemm_blockscaled_e8m0(qa, qb, self.sa, self.sb, self.out, C=self.C)
        elif self.kind == "block":
            P.fp8_gemm_blockscaled(qa, qb, self.sa, self.sb, self.out, C=self.C, block=self.block)
        else:
            P.fp8_grouped_gemm(qa, qb.view(self.E, self.K, self.N), self.off, self.sa, self.sb, self.out,
                               C=self.C, fast=fast)

    def step(self):
        self.quantize()
        self.gemm()

    def gemm_bytes(self):
        """Algorithmic HBM bytes of one GEMM launch: A and B codes once, C once."""
        osz = 4 if self.out == self.torch.float32 else 2
        if self.kind == "attn":    # Q, K, V codes once, O once
            return self.qa.numel() + self.qb.numel() + self.C.numel() * osz
        if self.kind == "moe":
            return self.M * self.K + self.E * self.K * self.N + self.M * self.N * osz
        t = getattr(self, "block", 32)
        extra = (self.M // t) * (self.K // t) * 4 + (self.K // t) * (self.N // t) * 4 if self.kind == "block" else 0
        if self.kind == "block_e8":
            extra = (self.M // 32) * (self.K // 32) + (self.K // 32) * (self.N // 32)
        if self.kind == "sparse":  # B: K/2 x N values + K/32 x N index words
            return self.M * self.K + (self.K // 2) * self.N + (self.K // 32) * self.N * 4 + self.M * self.N * osz
        return self.M * self.K + self.K * self.N + self.M * self.N * osz + extra


def cpu_baseline(w: Workload, rows: int):
    """The oracle on a bounded sample of the step: quantize B fully and `rows`
    rows of A, GEMM those rows; extrapolated to a full step."""
    import oracle
    M = w.M
    r = min(rows, M)
    sel = np.arange(r)
    t0 = time.perf_counter()
    if w.kind == "pertensor" and w.b_e5m2:
        qa, sa, _ = oracle.quantize_pertensor_fmt(w.a_host[:r], oracle.E4M3)
        tqa = time.perf_counter() - t0
        t0 = time.perf_counter()
        qb, sb, _ = oracle.quantize_pertensor_fmt(w.b_host, oracle.E5M2)
        tqb = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.gemm_rows_fmt(qa, qb, oracle.E4M3, oracle.E5M2, sa, sb, oracle.F16, rows=sel)
        tg = time.perf_counter() - t0
    elif w.kind == "pertensor":
        qa, sa, _ = oracle.quantize_pertensor(w.a_host[:r])
        tqa = time.perf_counter() - t0
        t0 = time.perf_counter()
        qb, sb, _ = oracle.quantize_pertensor(w.b_host)
        tqb = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.gemm_rows(qa, qb, sa, sb, oracle.BF16 if w.out != w.torch.float32 else oracle.F32, rows=sel)
        tg = time.perf_counter() - t0
    elif w.kind == "attn":
        from oracle import attention as OA
        hs = 4   # heads in the sample (of 32)
        qq, sq, _ = oracle.quantize_pertensor(w.a_host)
        qk, sk, _ = oracle.quantize_pertensor(w.b_host[0])
        qv, sv, _ = oracle.quantize_pertensor(w.b_host[1])
        tq = time.perf_counter() - t0
        t0 = time.perf_counter()
        OA.attention(qq[:hs], qk[:hs], qv[:hs], sq, sk, sv, 1.0 / np.sqrt(w.N), w.causal)
        tg = time.perf_counter() - t0
        t_step = tq + tg * w.heads / hs
        return {"value": round(w.flops / t_step / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
                "kind": "oracle",
                "sample": "quantize Q, K, V (%.2fs), float64 attention of %d of %d heads (%.2fs); scaled to one "
                          "full step = %.1fs" % (tq, hs, w.heads, tg, t_step)}
    else:
        return None
    t_step = tqa * M / r + tqb + tg * M / r
    return {"value": round(w.flops / t_step / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "quantize %d of %d rows of A (%.2fs) and all of B (%.2fs), exact %s GEMM of those %d rows "
                      "(%.2fs); scaled to one full step = %.1fs" % (r, M, tqa, tqb,
                                                                    "128-bit integer" if w.b_e5m2 else "FP64", r, tg,
                                                                    t_step)}


def vendor_reference(w: Workload):
    """Context, not part of the step: the vendor GEMM library (hipBLASLt, via
    torch) on the same shape and device, timed like the GEMM above -- its FP8
    GEMM on the same E4M3 codes (B handed over in the column-major layout it
    takes) and its BF16 GEMM on the codes widened to BF16, with B as an N x K
    weight (its fastest layout) and as the row-major K x N matrix."""
    torch = w.torch
    if w.kind == "attn":
        return vendor_attention(w)
    if w.kind != "pertensor" or w.b_e5m2 or w.out != torch.bfloat16:
        return None
    out = {"library": "hipBLASLt via torch._scaled_mm (FP8), torch.nn.functional.linear and torch.matmul (BF16)"}
    a8 = w.qa.view(torch.float8_e4m3fn)
    bt8 = w.qb.t().contiguous().view(torch.float8_e4m3fn)  # N x K, K contiguous
    sa, sb = w.sa.reshape(()), w.sb.reshape(())

    def timed(fn, n=20):
        for _ in range(3):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for s_, e_ in ev:
            s_.record()
            fn()
            e_.record()
        torch.cuda.synchronize()
        us = float(np.median([s_.elapsed_time(e_) for s_, e_ in ev])) * 1e3
        return {"median_us": round(us, 2), "tflops": round(w.flops / (us * 1e-6) / 1e12, 2)}

    try:
        out["fp8"] = timed(lambda: torch._scaled_mm(a8, bt8.t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16))
    except Exception as e:  # library without FP8 support on this device
        out["fp8"] = {"error": repr(e)[:200]}
    # BF16 in the layout that library is fastest with (B as an N x K weight,
    # nn.Linear's convention; a plain 2-D product), and with row-major B
    a16 = a8.to(torch.bfloat16)
    bt16 = bt8.to(torch.bfloat16)
    out["bf16"] = timed(lambda: torch.nn.functional.linear(a16, bt16))
    del bt16
    b16 = w.qb.view(torch.float8_e4m3fn).to(torch.bfloat16)
    out["bf16_b_row_major"] = timed(lambda: torch.matmul(a16, b16))
    del a16, b16, bt8
    return out


def vendor_attention(w: Workload):
    """Context, not part of the step: torch's scaled_dot_product_attention in
    BF16 (the ROCm fused attention kernels) on the same values, the codes
    widened to BF16 with the scales folded into Q and V, timed like the
    kernel above."""
    torch = w.torch
    q16 = (w.qa.view(torch.float8_e4m3fn).to(torch.float32) * (w.sa * w.sb)).to(torch.bfloat16)[None]
    k16 = w.qb[0].view(torch.float8_e4m3fn).to(torch.bfloat16)[None]
    v16 = (w.qb[1].view(torch.float8_e4m3fn).to(torch.float32) * w.sv).to(torch.bfloat16)[None]
    f = lambda: torch.nn.functional.scaled_dot_product_attention(q16, k16, v16, is_causal=w.causal,
                                                                  scale=1.0 / np.sqrt(w.N))
    try:
        for _ in range(3):
            f()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
        for s_, e_ in ev:
            s_.record()
            f()
            e_.record()
        torch.cuda.synchronize()
        us = float(np.median([s_.elapsed_time(e_) for s_, e_ in ev])) * 1e3
        return {"library": "torch.nn.functional.scaled_dot_product_attention (BF16)",
                "bf16": {"median_us": round(us, 2), "tflops": round(w.flops / (us * 1e-6) / 1e12, 2)}}
    except Exception as e:  # torch without a usable attention kernel here
        return {"library": "torch.nn.functional.scaled_dot_product_attention (BF16)", "error": repr(e)[:200]}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        x = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(2):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": x.numel() * 4, "bytes_written": y.numel() * 4}))
        return
    w = Workload(args.workload, dev)
    stream = torch.cuda.current_stream(dev)

    t_w = time.perf_counter()
    done = 0
    while done < args.warmup or time.perf_counter() - t_w < args.warmup_seconds:
        w.step()
        done += 1
        if done % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    # Timed region: K whole steps; GEMM launches bracketed by events on the
    # same stream to get the kernel's own average duration.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    with SclkSampler() as sclk:
        t0 = time.perf_counter()
        for i in range(args.steps):
            w.quantize()
            ev[i][0].record(stream)
            w.gemm()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    gemm_ms = [s.elapsed_time(e) for s, e in ev]

    # the native-FP8-accumulation GEMM (FP8_ACC_FAST; for attention, Q K^T on the FP8 matrix cores),
    # timed the same way, outside the timed region
    fast = None
    if w.kind not in ("block", "block_e8", "sparse"):
        for _ in range(3):
            w.gemm(fast=True)
        fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        for s_, e_ in fev:
            s_.record(stream)
            w.gemm(fast=True)
            e_.record(stream)
        torch.cuda.synchronize()
        fms = float(np.mean([s_.elapsed_time(e_) for s_, e_ in fev]))
        ft = w.flops / (fms * 1e-3) / 1e12
        fast = {"gemm_tflops": round(ft, 2), "pct_fp8_peak": round(100 * ft / FP8_PEAK_TFLOPS, 2),
                "avg_kernel_us": round(fms * 1e3, 2)}

    # quantize alone (for the GB/s figure), outside the timed region
    qev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    qev[0].record(stream)
    for _ in range(5):
        w.quantize()
    qev[1].record(stream)
    torch.cuda.synchronize()
    q_ms = qev[0].elapsed_time(qev[1]) / 5
    q_bytes = w.A.numel() * 5 + w.B.numel() * 5 + w.A.numel() * 4 + w.B.numel() * 4  # amax read; read + code write

    ms_step = elapsed * 1e3 / args.steps
    avg_gemm_ms = float(np.mean(gemm_ms))
    gemm_tflops = w.flops / (avg_gemm_ms * 1e-3) / 1e12
    mfma_bound = w.flops / w.gemm_bytes() > FP8_PEAK_TFLOPS / HBM_PEAK_GBPS * 1e3
    hbm_ms = None
    if not mfma_bound:
        # memory-bound shapes: back-to-back launches that rotate over enough
        # copies of the operand codes (> 2x the 256 MB MALL in all) that each
        # launch reads its operands from HBM, timed as one batch so that the
        # per-launch figure carries no event overhead
        per = w.qa.numel() + w.qb.numel()
        ncopy = int(min(256, max(4, -(-(640 << 20) // per))))
        cp = [(w.qa.clone(), w.qb.clone()) for _ in range(ncopy)]
        rounds = max(1, 40 // ncopy)
        for qa_, qb_ in cp:
            w.gemm(qa=qa_, qb=qb_)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(rounds):
            for qa_, qb_ in cp:
                w.gemm(qa=qa_, qb=qb_)
        e1.record(stream)
        torch.cuda.synchronize()
        hbm_ms = e0.elapsed_time(e1) / (rounds * ncopy)
        how = "back-to-back launches"
        if hbm_ms < 0.015:
            # Kernels this short are outrun by the host: ~10 us per call from
            # Python.  The rotation is then captured in a HIP graph and
            # replayed.  Longer kernels keep direct launches: graph replay
            # measured slower for them (M=128, N=28672: 74.7 against 65.8 us).
            cap = torch.cuda.Stream()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=cap):
                for qa_, qb_ in cp:
                    w.gemm(qa=qa_, qb=qb_)
            graph.replay()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(rounds):
                graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            hbm_ms = e0.elapsed_time(e1) / (rounds * ncopy)
            how = "back-to-back launches replayed from a HIP graph (host-launched: too short to keep the GPU busy)"
            del graph
        rotation = "%d %s rotating over %d copies of the A and B codes (%d MiB in all%s)" % (
            rounds * ncopy, how, ncopy, (ncopy * per) >> 20,
            ", > 2x the 256 MB MALL: operands from HBM" if ncopy * per > 512e6 else ": small enough to stay cached")
        del cp
    if mfma_bound and w.kind == "sparse":
        # half of the products are structurally zero: the matrix cores execute
        # M*N*K multiply-adds, priced against the dense FP8 rate (the sparse
        # instructions reach twice the dense rate in K, i.e. the same rate of
        # executed products)
        peak = FP8_PEAK_TFLOPS
        executed = gemm_tflops / 2
        roof = {"bound": "mfma", "achieved": round(executed, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(executed / peak, 4), "traffic": measured_traffic(args.workload),
                "peak_basis": "dense FP8 MFMA; achieved counts the executed (nonzero) products, 2*M*N*K/2; "
                              "gemm_tflops counts the dense-equivalent 2*M*N*K"}
    elif mfma_bound and w.kind == "block_e8":
        # power-of-two tile scales: the scaled FP8 matrix-core instructions
        peak = FP8_PEAK_TFLOPS
        roof = {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(gemm_tflops / peak, 4), "traffic": measured_traffic(args.workload),
                "peak_basis": "dense FP8 MFMA (the scaled FP8 instructions apply the E8M0 tile scales)"}
    elif mfma_bound:
        # FP8 operands: priced against the dense FP8 MFMA peak the metric
        # names; the default (exact-product) kernels multiply on the BF16
        # matrix cores, whose dense peak is half of it
        peak = FP8_PEAK_TFLOPS
        roof = {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(gemm_tflops / peak, 4), "traffic": measured_traffic(args.workload),
                "peak_basis": "dense FP8 MFMA (the metric's peak); the default mode widens the FP8 operands "
                              "exactly to BF16 so every product is exact, and runs on the BF16 matrix cores",
                "frac_of_bf16_peak": round(gemm_tflops / BF16_PEAK_TFLOPS, 4)}
    else:
        gbps = w.gemm_bytes() / (hbm_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(args.workload),
                "basis": rotation,
                "in_step_avg_kernel_us": round(avg_gemm_ms * 1e3, 2)}
    roof["kernel"] = {
        "pertensor": ("skinny_kernel (fp8_gemm with a workspace, M <= 16)" if getattr(w, "M", 1 << 30) <= 16
                      else "gemm_kernel (fp8_gemm)"),
        "block": ("gemm_kernel MODE_BLOCK64 (fp8_gemm_blockscaled, 64x64 tiles)" if getattr(w, "block", 32) == 64
                  else "gemm_kernel MODE_BLOCK (fp8_gemm_blockscaled)"),
        "block_e8": "gemm_kernel MODE_E8M0 (fp8_gemm_blockscaled_e8m0)",
        "sparse": "gemm_kernel MODE_SPARSE (fp8_gemm_sparse24)",
        "moe": "gemm_kernel (fp8_grouped_gemm)",
        "attn": "attention_kernel (fp8_attention)"}[w.kind]
    roof["avg_kernel_us"] = round((avg_gemm_ms if mfma_bound else hbm_ms) * 1e3, 2)
    vendor = None if args.no_vendor else vendor_reference(w)
    mhz = sclk.mean_mhz()
    sclk_out = None
    if mhz is not None:
        ghz = mhz / 1e3
        sclk_out = {"mean_mhz": round(mhz, 1), "samples": len(sclk.samples), "source": "pp_dpm_sclk, timed region",
                    "gemm_pct_bf16_peak_at_sclk": round(100 * gemm_tflops / (CUS * BF16_FLOP_PER_CU_CLK * ghz / 1e3), 2),
                    "gemm_pct_fp8_peak_at_sclk": round(100 * gemm_tflops / (CUS * FP8_FLOP_PER_CU_CLK * ghz / 1e3), 2)}

    out = {
        "metric": ("FP8 GEMM TFLOPS at M=N=K=8192 (BF16 out) + % of MI355X dense FP8 peak" if args.workload == "gemm8192"
                   else "%s TFLOPS, %s workload (kernel alone) + %% of MI355X dense FP8 peak"
                   % ("FP8 attention" if w.kind == "attn" else "FP8 GEMM", args.workload)),
        "value": round(gemm_tflops, 2),
        "unit": "TFLOP/s",
        "pct_fp8_peak": round(100 * gemm_tflops / FP8_PEAK_TFLOPS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 x fp8e5m2 (fp32 accumulate)" if w.b_e5m2 else "fp8e4m3 (fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": w.desc, "M": w.M, "N": w.N, "K": w.K,
                   "out": {torch.bfloat16: "bf16", torch.float16: "f16"}.get(w.out, "f32"),
                   "step": "quantize Q, K, V + attention" if w.kind == "attn" else "quantize A and B + GEMM",
                   "value": "%s kernel alone (average launch inside the timed steps)"
                            % ("attention" if w.kind == "attn" else "GEMM")},
        "step_tflops": round(w.flops / (ms_step * 1e-3) / 1e12, 2),
        "gemm_tflops": round(gemm_tflops, 2),
        "quantize_ms": round(q_ms, 4),
        "quantize_gbps": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
        "roofline": roof,
        "sclk": sclk_out,
        "fp8_acc_fast": fast,
        "vendor_same_box": vendor,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
