"""Benchmark of the a8w8 block-scale GEMM on one MI355X.

Default workload (the decode configuration the headline metric is quoted on):
M in {1, 2, 4, 8, 16}, N = 14336, K = 5120, fp8 e4m3 operands with 1x128 /
128x128 fp32 scales, bf16 out, and the weights rotated over >= 2 GiB of
distinct copies so that every call streams W from HBM (the 256 MB MALL cannot
hold them).  Each M has its own HIP graph of R calls, one per weight copy; one
step replays the graph of every M once, and value = microseconds per call
averaged over M (the pages quote each (M, N, K) row on its own).  The same
calls in one graph with M cycling call by call are reported beside it.

Before any number is printed the GPU output is checked against the fp64 CPU
oracle (first, middle and last weight copy, every M); a mismatch aborts the
run.  The JSON line also carries the roofline of the dominant kernel, a
prefill measurement (M >= 4096, fp8 TFLOP/s against the MFMA peak) and the
oracle's own time on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       [--decode-nk N:K] [--decode-ms 1,2,...]   (other decode shapes, e.g. 34816:5120)
       [--workload sweep]                         (the dense-M sweep report)
       [--no-mx]                                  (skip the MX-scaled and row-wise points)

The line also reports the MX-scaled variant (E8M0 scales per 1x32 activation
group and 32x32 weight block) at its page's tuned points, cold weights, and
the row-wise (per-token / per-channel) variant on the decode and prefill
shapes.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA, 5.0 PFLOP/s
ROTATE_BYTES = 2 * 1024 ** 3   # >= 2 GiB of distinct weight copies
METRIC = "µs/call + % HBM roofline (M≤16, cold W); fp8 TFLOP/s % MFMA peak (M≥4096)"


def algorithmic_bytes(M: int, N: int, K: int) -> int:
    """W, w_scale, A, a_scale and Y, each moved once."""
    KB, NB = K // 128, (N + 127) // 128
    return N * K + 4 * NB * KB + M * K + 4 * M * KB + 2 * M * N


def flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def recorded_traffic():
    """HBM bytes per launch of the decode kernel from the committed counter summary,
    or None when the kernel source changed since the counters were taken."""
    import hashlib
    import re
    prof = os.path.join(ROOT, "profiles", "skinny_rskinny_decode_qkv_N14336_K5120_traffic.md")
    src = os.path.join(ROOT, "fp8_block_scaled_a8w8_amd", "csrc", "a8w8_kernels.hip")
    try:
        text = open(prof).read()
        rec = json.loads(re.findall(r"```json\n(.*?)\n```", text, re.S)[-1])
        cur = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    except (OSError, IndexError, ValueError):
        return None
    return rec["traffic_bytes_per_launch"] if rec.get("kernel_source_sha256_16") == cur else None


def parity_gate(g, oracle, A, a_s, W_host, w_s, dA, da, dW, dw, Ms, what):
    """Compare GPU rows with the oracle; raise on mismatch (no perf without parity)."""
    import torch
    ref = oracle.gemm(A[:max(Ms)], a_s[:max(Ms)], W_host, w_s)
    worst = 0.0
    for M in Ms:
        y = g.gemm_a8w8_blockscale(dA[:M], da[:M], dW, dw)
        torch.cuda.synchronize()
        yh = y.float().cpu().numpy().astype(np.float64)
        r = ref[:M]
        rel = float(np.linalg.norm(yh - r) / np.linalg.norm(r))
        rms = float(np.sqrt(np.mean(r * r)))
        bad = np.abs(yh - r) > 2e-2 * rms
        if rel > 3e-3 or not np.all(np.isfinite(yh)):
            raise SystemExit(f"parity gate failed ({what}, M={M}): rel_l2={rel:.3e}")
        if bad.any():
            # allowed only where the GPU value is a bf16 neighbour of the exact result
            f, e = np.frexp(r[bad])
            lo = np.ldexp(np.floor(np.abs(f) * 256) / 256, e)
            hi = np.ldexp(np.ceil(np.abs(f) * 256) / 256, e)
            v = np.abs(yh[bad])
            if not np.all((v == lo) | (v == hi)):
                raise SystemExit(f"parity gate failed ({what}, M={M}): max-error rule")
        worst = max(worst, rel)
    return worst


_SIDE_STREAM = None


def time_graph(torch, calls, replays, warmup):
    """Capture `calls` (list of zero-arg callables) into one HIP graph on a side stream, after one
    eager pass of them there (warm-up); returns the graph after `warmup` replays."""
    global _SIDE_STREAM
    if _SIDE_STREAM is None:
        _SIDE_STREAM = torch.cuda.Stream()
    s = _SIDE_STREAM
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in calls:
            c()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        for c in calls:
            c()
    torch.cuda.synchronize()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    return graph


def timed_replays(torch, graph, n):
    """HIP events on the replay stream around n replays; returns ms per replay."""
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(n):
        graph.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / n


def read_ceiling_block(torch, dev, nbytes, R, replays, us_decode):
    """The part's streaming-read ceiling at the decode's byte count: a plain read kernel
    (fp8_block_scaled_a8w8_amd/csrc/read_ceiling.hip) over R rotated buffers of `nbytes`,
    timed like the GEMM (one HIP graph of R launches), best of a few grids."""
    import ctypes
    path = os.path.join(ROOT, "fp8_block_scaled_a8w8_amd", "libceilings.so")
    lib = ctypes.CDLL(path)
    fn = lib.a8w8_read_ceiling_launch
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    nbytes = nbytes // 16 * 16
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(R)]
    best = None
    for grid in (512, 1024, 2048, 4096):
        sink = torch.zeros(grid, dtype=torch.int32, device=dev)
        for unroll in (8, 16):
            def launch(b, grid=grid, unroll=unroll, sink=sink):
                rc = fn(b.data_ptr(), nbytes, sink.data_ptr(), grid, unroll, torch.cuda.current_stream().cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"read_ceiling launch failed ({rc})")
            graph = time_graph(torch, [(lambda b=b: launch(b)) for b in bufs], 0, 2)
            us = timed_replays(torch, graph, replays) * 1000.0 / R
            del graph
            if best is None or us < best[0]:
                best = (us, grid, unroll)
    del bufs
    us, grid, unroll = best
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"bytes": nbytes, "us": round(us, 3), "GB_s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "config": f"{grid} workgroups x 256 lanes, {unroll} 16-byte loads per lane in flight, {R} rotated buffers",
            "decode_frac_of_ceiling": round(us / us_decode, 4)}


def decode_shape_block(torch, g, inputgen, oracle, dev, N, K, Ms, replays, seed_w=11, with_fused=True):
    """One decode shape with cold weights (>= 2 GiB of rotated copies): parity gate on the first
    and last copy for every M (all 16 rows against the oracle), then, per M, one HIP graph of R
    calls timed with HIP events; returns per-M us/call and HBM fractions and their mean."""
    A, a_s = inputgen.make_activations(16, K, seed=seed_w + 1)
    W0, w_s = inputgen.make_weights(N, K, seed=seed_w)
    R = math.ceil(ROTATE_BYTES / (W0.nbytes + w_s.nbytes))
    dA, da, dw = (torch.from_numpy(x).to(dev) for x in (A, a_s, w_s))
    copies = [torch.from_numpy(W0 if r == 0 else inputgen.sign_flip_copy(W0, seed=2000 + r)).to(dev)
              for r in range(R)]
    worst = 0.0
    for r in (0, R - 1):
        Wr = W0 if r == 0 else inputgen.sign_flip_copy(W0, seed=2000 + r)
        worst = max(worst, parity_gate(g, oracle, A, a_s, Wr, w_s, dA, da, copies[r], dw, Ms,
                                       f"decode N={N} K={K} copy {r}"))
    per_m = {}
    for M in Ms:
        outM = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        gm = time_graph(torch, [(lambda r=r: g.gemm_a8w8_blockscale(dA[:M], da[:M], copies[r], dw, out=outM))
                                for r in range(R)], 0, 2)
        us = timed_replays(torch, gm, replays) * 1000.0 / R
        gbs = algorithmic_bytes(M, N, K) / (us * 1e-6) / 1e9
        per_m[str(M)] = {"us_per_call": round(us, 3), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                         "plan": g.gemm_a8w8_blockscale_plan(M, N, K)["name"]}
        del gm
    fused = fused_quant_block(torch, g, inputgen, dev, copies, dw, N, K, [m for m in (1, 2, 4, 8, 16) if m in Ms],
                              replays) if with_fused else {}
    del copies
    torch.cuda.empty_cache()
    us_mean = sum(v["us_per_call"] for v in per_m.values()) / len(per_m)
    bytes_mean = sum(algorithmic_bytes(M, N, K) for M in Ms) / len(Ms)
    return {"us_per_call_mean": round(us_mean, 3),
            "hbm_frac": round(bytes_mean / (us_mean * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_per_call_mean": round(bytes_mean), "weight_copies": R,
            "rotate_bytes": R * (W0.nbytes + w_s.nbytes), "parity_worst_rel_l2": round(worst, 6), "per_m": per_m,
            "fused_quantisation": fused}


def fused_quant_block(torch, g, inputgen, dev, copies, dw, N, K, Ms, replays):
    """Decode from bf16 activations: a8w8_quantize_1x128 then gemm_a8w8_blockscale (two kernels)
    against gemm_a8w8_blockscale_fused_quant (one), per M, each timed as one HIP graph of calls
    over the rotated weight copies.  Parity gate: the fused result equals the quantise-then-GEMM
    result with the fused plan's instance bit for bit (first and last copy, every M)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    try:
        g.gemm_a8w8_blockscale_fused_quant_plan(1, N, K, cu_count=cus)
    except g.A8W8Error:
        return {}
    X = inputgen.normal_bf16(16, K, 1.0, seed=77).to(torch.bfloat16).to(dev)
    R = len(copies)
    out = {}
    for M in Ms:
        Xm = X[:M]
        plan = g.gemm_a8w8_blockscale_fused_quant_plan(M, N, K, cu_count=cus)
        q, s = g.quantize_1x128(Xm)
        for r in (0, R - 1):
            y = g.gemm_a8w8_blockscale_fused_quant(Xm, copies[r], dw)
            two = g.gemm_a8w8_blockscale_run_variant(plan["variant"], q, s, copies[r], dw)
            if not torch.equal(y.view(torch.int16), two.view(torch.int16)):
                raise SystemExit(f"parity gate failed (fused quantisation N={N} K={K} M={M} copy {r})")
        outM = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        g2 = time_graph(torch, [(lambda r=r: (g.quantize_1x128(Xm, out=q, scale_out=s),
                                              g.gemm_a8w8_blockscale(q, s, copies[r], dw, out=outM)))
                                for r in range(R)], 0, 2)
        us2 = timed_replays(torch, g2, replays) * 1000.0 / R
        del g2
        g1 = time_graph(torch, [(lambda r=r: g.gemm_a8w8_blockscale_fused_quant(Xm, copies[r], dw, out=outM))
                                for r in range(R)], 0, 2)
        us1 = timed_replays(torch, g1, replays) * 1000.0 / R
        del g1
        out[str(M)] = {"fused_us_per_call": round(us1, 3), "quantize_then_gemm_us_per_call": round(us2, 3),
                       "fused_gain": round(us2 / us1 - 1.0, 4), "fused_plan": plan["name"],
                       "gemm_plan": g.gemm_a8w8_blockscale_plan(M, N, K)["name"]}
    return out


def mfma_ceiling_block(torch, dev, W_bytes_dev, replays):
    """The part's sustained fp8 MFMA rate (fp8_block_scaled_a8w8_amd/csrc/mfma_ceiling.hip): 8
    independent in-place MFMA chains per wave, two waves per SIMD, operands taken from real weight
    bytes; one HIP graph of 4 launches of about 2 ms each, timed with HIP events."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "fp8_block_scaled_a8w8_amd", "libceilings.so"))
    fn = lib.a8w8_mfma_ceiling_launch
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    fl = lib.a8w8_mfma_ceiling_flops
    fl.argtypes = [ctypes.c_int, ctypes.c_int]
    fl.restype = ctypes.c_double
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grid, iters = 2 * cus, 4000                    # 8 waves per CU
    nfrag = W_bytes_dev.numel() // 2048
    sink = torch.zeros(grid, dtype=torch.float32, device=dev)

    def launch():
        rc = fn(W_bytes_dev.data_ptr(), nfrag, sink.data_ptr(), grid, iters, torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"mfma_ceiling launch failed ({rc})")
    gr = time_graph(torch, [launch] * 4, 0, 1)
    ms = timed_replays(torch, gr, replays) / 4
    tf = fl(grid, iters) / (ms * 1e-3) / 1e12
    return {"TFLOP_s": round(tf, 1), "frac_of_peak": round(tf / FP8_PEAK_TFLOPS, 4),
            "ms_per_launch": round(ms, 4),
            "config": f"{grid} workgroups x 4 waves, {iters} rounds of 8 independent "
                      f"v_mfma_f32_16x16x128_f8f6f4 per wave, fp8 weight bytes as operands"}


def cu_capacity_block(torch, dev):
    """What one CU moves per clock through the data paths of the tile kernels
    (fp8_block_scaled_a8w8_amd/csrc/cu_capacity.hip): 16-byte LDS reads, 16-byte vector loads into
    registers and 16-byte direct-to-LDS copies, the last two from a 2 MB buffer (L2-resident) and a
    64 MB one (beyond L2, inside the 256 MB MALL).  One workgroup of 16 waves per CU; each times its
    own loop with the shader clock (s_memtime) and the 100 MHz real-time counter, so the figure is
    bytes per clock of the clock the part ran at, which is reported too.  Median over workgroups."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "fp8_block_scaled_a8w8_amd", "libceilings.so"))
    fn = lib.a8w8_cu_capacity_launch
    fn.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                   ctypes.c_void_p]
    fn.restype = ctypes.c_int
    nb = lib.a8w8_cu_capacity_bytes
    nb.argtypes = [ctypes.c_int]
    nb.restype = ctypes.c_double
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.zeros(2 * cus, dtype=torch.int64, device=dev)
    res = {}
    for name, which, size, iters in (("lds_read", 0, 0, 4000), ("vmem_load_L2", 1, 2 << 20, 1000),
                                     ("vmem_load_MALL", 1, 64 << 20, 1000), ("lds_dma_L2", 2, 2 << 20, 1000),
                                     ("lds_dma_MALL", 2, 64 << 20, 1000)):
        src = torch.full((max(size, 16),), 7, dtype=torch.uint8, device=dev)
        rows = []
        for _ in range(3):                      # the first launch warms the caches and the clock
            rc = fn(which, src.data_ptr(), size, out.data_ptr(), cus, iters, torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError(f"cu_capacity launch failed ({rc})")
            torch.cuda.synchronize()
            rows.append(out.view(cus, 2).cpu().numpy().astype(np.float64))
        cyc, ticks = rows[-1][:, 0], rows[-1][:, 1]
        bpc = nb(iters) / cyc
        res[name] = {"B_per_clk_per_CU": round(float(np.median(bpc)), 1),
                     "B_per_clk_per_CU_p10_p90": [round(float(np.percentile(bpc, 10)), 1),
                                                  round(float(np.percentile(bpc, 90)), 1)],
                     "GB_s_per_CU": round(float(np.median(nb(iters) / (ticks * 10.0))), 1),
                     "clock_GHz": round(float(np.median(cyc / (ticks * 10.0))), 3)}
        del src
    res["config"] = (f"{cus} workgroups x 16 waves (96 KB LDS each: one per CU), 8 16-byte operations per lane "
                     "per step, contiguous kilobyte per instruction")
    return res


def vendor_fp8_us(torch, a, w, reps=20):
    """Context, not part of this library: the vendor GEMM library's plain fp8 GEMM (per-tensor unit
    scales, no block scaling; torch._scaled_mm) on the same fp8 operand bytes, HIP events around
    `reps` back-to-back calls after three warm-up calls.  Returns us per call, or an error string."""
    try:
        one = torch.ones((), dtype=torch.float32, device=a.device)
        a8, w8 = a.view(torch.float8_e4m3fn), w.view(torch.float8_e4m3fn)
        for _ in range(3):
            torch._scaled_mm(a8, w8.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(reps):
            torch._scaled_mm(a8, w8.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1000.0 / reps
    except Exception as e:                      # reported, not fatal: this is context only
        return f"{type(e).__name__}: {str(e)[:160]}"


def quantize_bytes(M: int, K: int) -> int:
    """Algorithmic bytes of the activation quantisation: bf16 in, e4m3fn codes and fp32 scales out."""
    return 2 * M * K + M * K + 4 * M * (K // 128)


def quantize_block(torch, g, inputgen, oracle, dev, replays):
    """Per-1x128 activation quantisation at K = 5120, M in {16, 8192}: bit-exact parity gate
    against the oracle, then HIP-graph timing with the input rotated over distinct copies."""
    K = 5120
    out = {}
    for M in (16, 8192):
        x = inputgen.normal_bf16(M, K, 1.0, seed=50 + M)
        xb = x.to(torch.bfloat16).to(dev)
        q, s = g.quantize_1x128(xb)
        q_ref, s_ref = oracle.quantize_1x128(x.numpy())
        if not (np.array_equal(q.view(torch.uint8).cpu().numpy(), q_ref) and np.array_equal(s.cpu().numpy(), s_ref)):
            raise SystemExit(f"parity gate failed (quantize M={M})")
        R = min(256, max(2, math.ceil(ROTATE_BYTES / 2 / xb.numel() / 2)))   # >= 1 GiB of inputs when large
        xs = [xb] + [xb.clone() for _ in range(R - 1)]
        gr = time_graph(torch, [(lambda xr=xr: g.quantize_1x128(xr, out=q, scale_out=s)) for xr in xs], 0, 2)
        us = timed_replays(torch, gr, replays) * 1000.0 / R
        gbs = quantize_bytes(M, K) / (us * 1e-6) / 1e9
        out[f"M{M}_K{K}"] = {"us_per_call": round(us, 3), "GB_s": round(gbs, 1),
                             "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "input_copies": R}
        del gr, xs
    return out


# MX-scaled points: the page's tuned (b, M, N, K) microbenchmark points (gfx1250 BF16 and MX32
# tuned-rows page, ROCm/aiter #7247, Technical Details), plus its two other dense shapes at M = 768.
MX_POINTS = [(1, 48, 1792, 5120), (1, 768, 5120, 8192), (1, 768, 32768, 1280), (8, 16, 1024, 4096),
             (1, 768, 4608, 5120), (1, 768, 5120, 2304)]


def mx_bytes(b: int, M: int, N: int, K: int) -> int:
    """Algorithmic bytes of the MX GEMM: W, w_scale (E8M0 per 32x32), A, a_scale (E8M0 per 1x32), Y."""
    return b * (N * K + ((N + 31) // 32) * (K // 32) + M * K + M * (K // 32) + 2 * M * N)


def mx_block(torch, g, inputgen, oracle, dev, replays):
    """MX-scaled GEMM at the page's points: parity gate against the oracle on sampled rows (every
    batch), then cold-weight timing (weights rotated over >= 1 GiB of sign-flipped copies)."""
    out = {}
    for b, M, N, K in MX_POINTS:
        pa = [inputgen.make_mx_activations(M, K, seed=70 + i) for i in range(b)]
        pw = [inputgen.make_mx_weights(N, K, seed=80 + i) for i in range(b)]
        stack = (lambda xs: np.stack(xs)) if b > 1 else (lambda xs: xs[0])
        A, a_s = stack([x[0] for x in pa]), stack([x[1] for x in pa])
        W0, w_s = stack([x[0] for x in pw]), stack([x[1] for x in pw])
        dA, da, dw = (torch.from_numpy(x).to(dev) for x in (A, a_s, w_s))
        R = max(2, math.ceil(ROTATE_BYTES / 2 / (W0.nbytes + w_s.nbytes)))
        copies = [torch.from_numpy(W0).to(dev)] + \
            [torch.from_numpy(inputgen.sign_flip_copy(W0, seed=1000 + r)).to(dev) for r in range(1, R)]
        fn = g.batched_gemm_a8w8_mxscale if b > 1 else g.gemm_a8w8_mxscale
        ws = g.Workspace(b * (64 << 20))
        y = fn(dA, da, copies[-1], dw, workspace=ws)
        torch.cuda.synchronize()
        W_last = inputgen.sign_flip_copy(W0, seed=1000 + R - 1)
        rows = sorted({0, M // 2, M - 1})
        worst = 0.0
        for i in range(b):
            sl = (lambda x: x[i]) if b > 1 else (lambda x: x)
            ref = oracle.gemm_mx(sl(A), sl(a_s), sl(W_last), sl(w_s), rows=rows)
            yh = sl(y)[rows].float().cpu().numpy().astype(np.float64)
            rel = float(np.linalg.norm(yh - ref) / np.linalg.norm(ref))
            if rel > 3e-3 or not np.all(np.isfinite(yh)):
                raise SystemExit(f"parity gate failed (MX b={b} M={M} N={N} K={K}): rel_l2={rel:.3e}")
            worst = max(worst, rel)
        yo = torch.empty_like(y)
        gr = time_graph(torch, [(lambda r=r: fn(dA, da, copies[r], dw, out=yo, workspace=ws)) for r in range(R)], 0, 2)
        us = timed_replays(torch, gr, replays) * 1000.0 / R
        t_hbm = mx_bytes(b, M, N, K) / (HBM_PEAK_GBS * 1e9) * 1e6
        t_mfma = b * flops(M, N, K) / (FP8_PEAK_TFLOPS * 1e12) * 1e6
        plan = g.gemm_a8w8_ex_plan(M, N, K, scale_kind="mx", batch=b, workspace_bytes=ws.nbytes)
        out[f"b{b}_M{M}_N{N}_K{K}"] = {
            "us_per_call": round(us, 3), "bound": "hbm" if t_hbm >= t_mfma else "mfma",
            "frac": round(max(t_hbm, t_mfma) / us, 4),
            "GB_s": round(mx_bytes(b, M, N, K) / (us * 1e-6) / 1e9, 1),
            "TFLOP_s": round(b * flops(M, N, K) / (us * 1e-6) / 1e12, 1),
            "plan": plan["name"], "tuned": plan["fallback"] == 0, "weight_copies": R,
            "parity_rel_l2": round(worst, 6)}
        del gr, copies, ws
        torch.cuda.empty_cache()
    return out


def rowwise_bytes(M: int, N: int, K: int) -> int:
    """Algorithmic bytes of the row-wise GEMM: W, A, one fp32 scale per row of each, Y."""
    return N * K + 4 * N + M * K + 4 * M + 2 * M * N


def rowwise_block(torch, g, inputgen, oracle, dev, replays):
    """Row-wise (per-token / per-channel) GEMM: the decode qkv shape (M cycling 1..16, cold
    weights over >= 1 GiB) and one prefill point, each behind an oracle parity gate."""
    N, K, Ms = 14336, 5120, (1, 2, 4, 8, 16)
    A, a_s = inputgen.make_rowwise_activations(16, K, seed=90)
    W0, w_s = inputgen.make_rowwise_weights(N, K, seed=91)
    dA, da, dw = (torch.from_numpy(x).to(dev) for x in (A, a_s, w_s))
    R = max(len(Ms), math.ceil(ROTATE_BYTES / 2 / W0.nbytes) // len(Ms) * len(Ms))
    copies = [torch.from_numpy(W0).to(dev)] + \
        [torch.from_numpy(inputgen.sign_flip_copy(W0, seed=1000 + r)).to(dev) for r in range(1, R)]
    ref = oracle.gemm_rowwise(A, a_s, W0, w_s)
    for M in Ms:
        yh = g.gemm_a8w8_rowwise(dA[:M], da[:M], copies[0], dw).float().cpu().numpy().astype(np.float64)
        rel = float(np.linalg.norm(yh - ref[:M]) / np.linalg.norm(ref[:M]))
        if rel > 3e-3 or not np.all(np.isfinite(yh)):
            raise SystemExit(f"parity gate failed (row-wise M={M}): rel_l2={rel:.3e}")
    outs = [torch.empty((Ms[r % len(Ms)], N), dtype=torch.bfloat16, device=dev) for r in range(R)]
    gr = time_graph(torch, [(lambda r=r: g.gemm_a8w8_rowwise(dA[:Ms[r % len(Ms)]], da[:Ms[r % len(Ms)]],
                                                             copies[r], dw, out=outs[r])) for r in range(R)], 0, 2)
    us = timed_replays(torch, gr, replays) * 1000.0 / R
    bytes_mean = sum(rowwise_bytes(Ms[r % len(Ms)], N, K) for r in range(R)) / R
    out = {"decode": {"us_per_call": round(us, 3), "workload": f"M in {{1,2,4,8,16}}, N={N}, K={K}, cold W "
                      f"({R} copies)", "hbm_frac": round(bytes_mean / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}}
    del gr, copies, outs
    Mp = 8192
    Ap, ap_ = inputgen.make_rowwise_activations(Mp, K, seed=92)
    dAp, dap = torch.from_numpy(Ap).to(dev), torch.from_numpy(ap_).to(dev)
    dW0 = torch.from_numpy(W0).to(dev)
    y = g.gemm_a8w8_rowwise(dAp, dap, dW0, dw)
    rows = [0, 4095, 8191]
    yh = y[rows].float().cpu().numpy().astype(np.float64)
    rp = oracle.gemm_rowwise(Ap, ap_, W0, w_s, rows=rows)
    rel = float(np.linalg.norm(yh - rp) / np.linalg.norm(rp))
    if rel > 3e-3:
        raise SystemExit(f"parity gate failed (row-wise prefill): rel_l2={rel:.3e}")
    gp = time_graph(torch, [lambda: g.gemm_a8w8_rowwise(dAp, dap, dW0, dw, out=y)] * 4, 0, 2)
    ms = timed_replays(torch, gp, 10) / 4
    tf = flops(Mp, N, K) / (ms * 1e-3) / 1e12
    out[f"prefill_M{Mp}_N{N}_K{K}"] = {"us_per_call": round(ms * 1000, 2), "TFLOP_s": round(tf, 1),
                                        "mfma_frac": round(tf / FP8_PEAK_TFLOPS, 4)}
    del gp
    return out


PREFILL_POINTS = [(M, N) for N in (14336, 16384) for M in (512, 2048, 6016, 8192)]
DECODE_SHAPES = {"out_proj": (5120, 6144), "gate_up": (34816, 5120)}


def check_rows(y_rows, ref, what):
    """The parity bar on sampled rows: rel-L2 <= 3e-3 and the max-error rule (|err| <= 2e-2 rms(ref),
    or the GPU value is one of the two bf16 neighbours of the exact result)."""
    rel = float(np.linalg.norm(y_rows - ref) / np.linalg.norm(ref))
    rms = float(np.sqrt(np.mean(ref * ref)))
    if rel > 3e-3 or not np.all(np.isfinite(y_rows)):
        raise SystemExit(f"parity gate failed ({what}): rel_l2={rel:.3e}")
    bad = np.abs(y_rows - ref) > 2e-2 * rms
    if bad.any():
        f, e = np.frexp(ref[bad])
        lo = np.ldexp(np.floor(np.abs(f) * 256) / 256, e)
        hi = np.ldexp(np.ceil(np.abs(f) * 256) / 256, e)
        v = np.abs(y_rows[bad])
        if not np.all((v == lo) | (v == hi)):
            raise SystemExit(f"parity gate failed ({what}): max-error rule")
    return rel


def prefill_block(torch, g, inputgen, oracle, dev, points):
    """Prefill points (K = 5120): per point a parity gate on sampled rows (first, middle, last and the
    rows on both sides of three tile boundaries of the plan), then a HIP graph of 4 calls replayed
    10 times; TFLOP/s and fraction of the 5 PF fp8 peak."""
    Kp = 5120
    Mmax = max(M for M, _ in points)
    A8, a8 = inputgen.make_activations(Mmax, Kp, seed=0)
    dA8, da8 = torch.from_numpy(A8).to(dev), torch.from_numpy(a8).to(dev)
    out_res = {}
    for Np in sorted({N for _, N in points}):
        Wp, wp = inputgen.make_weights(Np, Kp, seed=1)
        dWp, dwp = torch.from_numpy(Wp).to(dev), torch.from_numpy(wp).to(dev)
        for Mp in [M for M, N in points if N == Np]:
            plan = g.gemm_a8w8_blockscale_plan(Mp, Np, Kp)
            bm = plan["bm"]
            rows = sorted({0, Mp // 2, Mp - 1} | {b + d for b in (bm, (Mp // bm // 2) * bm, (Mp // bm - 1) * bm)
                                                  for d in (-1, 0) if 0 <= b + d < Mp})
            out = torch.empty((Mp, Np), dtype=torch.bfloat16, device=dev)
            g.gemm_a8w8_blockscale(dA8[:Mp], da8[:Mp], dWp, dwp, out=out)
            torch.cuda.synchronize()
            yh = out[rows].float().cpu().numpy().astype(np.float64)
            rel = check_rows(yh, oracle.gemm(A8[:Mp], a8[:Mp], Wp, wp, rows=rows), f"prefill M={Mp} N={Np}")
            gp = time_graph(torch, [lambda: g.gemm_a8w8_blockscale(dA8[:Mp], da8[:Mp], dWp, dwp, out=out)] * 4, 0, 2)
            ms = timed_replays(torch, gp, 10) / 4
            tf = flops(Mp, Np, Kp) / (ms * 1e-3) / 1e12
            out_res[f"M{Mp}_N{Np}_K{Kp}"] = {"us_per_call": round(ms * 1000, 2), "TFLOP_s": round(tf, 1),
                                             "mfma_frac": round(tf / FP8_PEAK_TFLOPS, 4), "plan": plan["name"],
                                             "parity_rows": len(rows), "parity_rel_l2": round(rel, 6)}
            # context: the vendor library's unscaled fp8 GEMM on the same operand bytes, right after
            vus = vendor_fp8_us(torch, dA8[:Mp], dWp)
            out_res[f"M{Mp}_N{Np}_K{Kp}"]["vendor_unscaled_fp8_context"] = (
                {"us_per_call": round(vus, 2), "TFLOP_s": round(flops(Mp, Np, Kp) / (vus * 1e-6) / 1e12, 1)}
                if isinstance(vus, float) else {"error": vus})
            log(f"prefill M={Mp} N={Np}: {out_res[f'M{Mp}_N{Np}_K{Kp}']}")
            del gp, out
        del dWp
    return out_res


def cpu_baseline_block(inputgen, oracle, A, a_s, W0, w_s, Ms, N, K, seconds):
    """The oracle as it stands, on the host cores: the decode workload (full outputs, ~`seconds`),
    the tiny configuration (full, median of 3) and the prefill configuration M = 8192, N = 14336
    on a bounded sample of rows (the time per row scaled to all 8192 rows: every row of Y costs the
    same N x K products)."""
    n_calls, t_cpu = 0, 0.0
    while t_cpu < seconds:
        M = Ms[n_calls % len(Ms)]
        t = time.time()
        oracle.gemm(A[:M], a_s[:M], W0, w_s)
        t_cpu += time.time() - t
        n_calls += 1
    At, at = inputgen.make_activations(4, 1024, seed=0)
    Wt, wt = inputgen.make_weights(512, 1024, seed=1)
    tiny = []
    for _ in range(3):
        t = time.time()
        oracle.gemm(At, at, Wt, wt)
        tiny.append(time.time() - t)
    Ap, ap_ = inputgen.make_activations(64, 5120, seed=0)
    Wp, wp = inputgen.make_weights(14336, 5120, seed=1)
    t = time.time()
    oracle.gemm(Ap, ap_, Wp, wp)
    per_row = (time.time() - t) / 64
    return {"value": round(t_cpu / n_calls * 1e6, 1), "unit": "µs/call", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"{n_calls} calls of the decode workload (M cycling {','.join(map(str, Ms))}; N={N}, K={K}; "
                      f"fp64, full output) on the host cores",
            "host_cpu_count": os.cpu_count(), "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS"),
            "threads_used": oracle.threads(),
            "tiny_M4_N512_K1024_us": round(float(np.median(tiny)) * 1e6, 1),
            "prefill_M8192_N14336_K5120_us": round(per_row * 8192 * 1e6, 1),
            "prefill_sample": "64 rows of the M = 8192, N = 14336, K = 5120 prefill (full N), time per row x 8192"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-decode-shapes", action="store_true",
                    help="skip the out_proj (5120:6144) and gate_up (34816:5120) decode shapes")
    ap.add_argument("--prefill-points", default=None,
                    help="with --workload prefill: M:N[,M:N...] (K = 5120) to run, one after another")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--workload", choices=["decode", "sweep", "prefill"], default="decode",
                    help="decode: the headline decode workload and every other leg (default); sweep: the "
                         "dense-M sweep report; prefill: only the prefill points (for per-point profiles)")
    ap.add_argument("--sweep-out", default=None, help="where the sweep writes its per-point table (markdown)")
    ap.add_argument("--decode-nk", default="14336:5120",
                    help="N:K of the decode workload (default: the qkv shape 14336:5120)")
    ap.add_argument("--decode-ms", default="1,2,4,8,16", help="M values the decode workload cycles through")
    ap.add_argument("--no-mx", action="store_true", help="skip the MX-scaled and row-wise points")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip the bf16-activation legs (quantise then GEMM, and the fused entry)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after the run, copy 256 MiB device-to-device three times (traffic calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU; the build runs on exactly one "
                          "MI355X and has no multi-GPU path (--gpus must be 1)"}))
        raise SystemExit(2)

    import torch
    import fp8_block_scaled_a8w8_amd as g
    import inputgen
    import oracle

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = "cuda:0"
    props = torch.cuda.get_device_properties(0)
    if not props.gcnArchName.startswith("gfx950"):
        raise SystemExit(f"bench.py targets gfx950, found {props.gcnArchName}")

    if args.workload == "sweep":
        return sweep(args, torch, g, inputgen, oracle)
    if args.workload == "prefill":
        pts = PREFILL_POINTS if not args.prefill_points else \
            [tuple(int(x) for x in p.split(":")) for p in args.prefill_points.split(",")]
        res = prefill_block(torch, g, inputgen, oracle, dev, pts)
        if args.calib_copy:
            calib_copy(torch)
        print(json.dumps({"metric": "prefill fp8 TFLOP/s", "points": res}), flush=True)
        return None

    # ------------------------------------------------------------ decode, cold W
    N, K = (int(x) for x in args.decode_nk.split(":"))
    Ms = [int(x) for x in args.decode_ms.split(",")]
    if K % 128 or not Ms or min(Ms) < 1 or max(Ms) > 16:
        raise SystemExit("decode workload: K must be a multiple of 128 and every M in 1..16")
    qkv = (N, K, Ms) == (14336, 5120, [1, 2, 4, 8, 16])
    t = time.time()
    A, a_s = inputgen.make_activations(16, K, seed=0)
    W0, w_s = inputgen.make_weights(N, K, seed=1)
    w_bytes = W0.nbytes + w_s.nbytes
    R = math.ceil(ROTATE_BYTES / w_bytes)
    R = int(math.ceil(R / len(Ms)) * len(Ms))           # every M gets the same number of calls
    dA = torch.from_numpy(A).to(dev)
    da = torch.from_numpy(a_s).to(dev)
    dw = torch.from_numpy(w_s).to(dev)
    copies = []
    for r in range(R):
        Wr = W0 if r == 0 else inputgen.sign_flip_copy(W0, seed=1000 + r)
        copies.append(torch.from_numpy(Wr).to(dev))
    log(f"decode inputs: N={N} K={K} {R} weight copies ({R * w_bytes / 2**30:.2f} GiB) in {time.time() - t:.1f}s")

    gate = 0.0
    for r in (0, R // 2, R - 1):
        Wr = W0 if r == 0 else inputgen.sign_flip_copy(W0, seed=1000 + r)
        gate = max(gate, parity_gate(g, oracle, A, a_s, Wr, w_s, dA, da, copies[r], dw, Ms, f"copy {r}"))
    log(f"parity gate passed: worst rel_l2 {gate:.3e}")

    # One HIP graph per M, each of R calls over the R rotated weight copies (the pages time
    # each (M, N, K) row on its own); one step replays the graphs of every M once, so a step
    # is len(Ms) * R calls and the value is the mean over M of the per-call time.
    graphs = {}
    for M in Ms:
        outM = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        graphs[M] = time_graph(torch, [(lambda r=r, M=M, outM=outM: g.gemm_a8w8_blockscale(
            dA[:M], da[:M], copies[r], dw, out=outM)) for r in range(R)], 0, args.warmup)
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.time()
    ev0.record(stream)
    for _ in range(args.steps):
        for M in Ms:
            graphs[M].replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.time() - t_wall
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    us_per_call = ms_per_step * 1000.0 / (R * len(Ms))
    bytes_mean = sum(algorithmic_bytes(M, N, K) for M in Ms) / len(Ms)
    achieved = bytes_mean / (us_per_call * 1e-6) / 1e9

    # per-M breakdown: each M's graph on its own
    per_m = {}
    for M in Ms:
        ms = timed_replays(torch, graphs[M], max(5, args.steps // 5))
        us = ms * 1000.0 / R
        gbs = algorithmic_bytes(M, N, K) / (us * 1e-6) / 1e9
        per_m[str(M)] = {"us_per_call": round(us, 3), "GB_s": round(gbs, 1),
                         "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                         "plan": g.gemm_a8w8_blockscale_plan(M, N, K)["name"]}
    del graphs
    log("per-M:", json.dumps(per_m))

    # The same calls in one graph with M cycling call by call (a different kernel instance may
    # follow each call): reported beside the per-M value, not as it.
    outs = [torch.empty((Ms[r % len(Ms)], N), dtype=torch.bfloat16, device=dev) for r in range(R)]
    gmix = time_graph(torch, [(lambda r=r: g.gemm_a8w8_blockscale(dA[:Ms[r % len(Ms)]], da[:Ms[r % len(Ms)]],
                                                                  copies[r], dw, out=outs[r])) for r in range(R)],
                      0, 2)
    us_mixed = timed_replays(torch, gmix, max(5, args.steps // 5)) * 1000.0 / R
    del gmix
    mixed = {"us_per_call": round(us_mixed, 3),
             "note": f"one graph of {R} calls with M cycling {','.join(map(str, Ms))} call by call"}
    log("mixed-M graph:", json.dumps(mixed))

    # the part's streaming-read ceiling at the same bytes per call
    ceiling = read_ceiling_block(torch, dev, round(bytes_mean), R, max(5, args.steps // 10), us_per_call)
    log("read ceiling:", json.dumps(ceiling))

    # the same workload with the weights prepacked offline (a8w8_prepack_weights)
    pcopies = [g.prepack_weights(c) for c in copies]
    for r in (0, R - 1):            # bitwise the same as the row-major run of the packed plan's instance
        for M in Ms:
            y_row = g.gemm_a8w8_blockscale_run_variant(g.gemm_a8w8_ex_plan(M, N, K, packed=True)["variant"],
                                                       dA[:M], da[:M], copies[r], dw)
            y_pk = g.gemm_a8w8_blockscale_packed(dA[:M], da[:M], pcopies[r], dw, N)
            if not torch.equal(y_row.view(torch.int16), y_pk.view(torch.int16)):
                raise SystemExit(f"parity gate failed (packed weights, copy {r}, M={M})")

    per_m_pk = {}
    for M in Ms:
        outM = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        gm = time_graph(torch, [(lambda r=r: g.gemm_a8w8_blockscale_packed(dA[:M], da[:M], pcopies[r], dw, N,
                                                                            out=outM)) for r in range(R)], 0, 2)
        us = timed_replays(torch, gm, max(5, args.steps // 5)) * 1000.0 / R
        per_m_pk[str(M)] = {"us_per_call": round(us, 3),
                            "hbm_frac": round(algorithmic_bytes(M, N, K) / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        del gm
    us_pk = sum(v["us_per_call"] for v in per_m_pk.values()) / len(per_m_pk)
    packed = {"us_per_call": round(us_pk, 3),
              "hbm_frac": round(bytes_mean / (us_pk * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
              "per_m": per_m_pk,
              "plans": {str(M): g.gemm_a8w8_ex_plan(M, N, K, packed=True)["name"] for M in Ms},
              "note": "same workload, weights prepacked offline into the kernels' fragment order, plans from "
                      "the packed decode table; outputs bitwise equal to the row-major run of the same instance"}
    del pcopies
    log("prepacked:", json.dumps(packed))

    # the same workload from bf16 activations: quantise then GEMM, against the fused entry
    fused = {} if args.no_fused else fused_quant_block(torch, g, inputgen, dev, copies, dw, N, K, Ms,
                                                       max(5, args.steps // 5))
    log("fused quantisation:", json.dumps(fused))

    # ------------------------------------------------------------ prefill (compute-bound)
    prefill = {} if args.no_prefill else prefill_block(torch, g, inputgen, oracle, dev, PREFILL_POINTS)
    log("prefill:", json.dumps(prefill))

    # ------------------------------------------------------------ other decode shapes (out_proj, gate_up)
    decode_shapes = {}
    if not args.no_decode_shapes:
        for name, (Nd, Kd) in DECODE_SHAPES.items():
            decode_shapes[f"{name}_N{Nd}_K{Kd}"] = decode_shape_block(torch, g, inputgen, oracle, dev, Nd, Kd,
                                                                     list(range(1, 17)), max(5, args.steps // 5),
                                                                     with_fused=not args.no_fused)
            log(f"decode {name}:", json.dumps(decode_shapes[f"{name}_N{Nd}_K{Kd}"]))

    # ------------------------------------------------------------ sustained MFMA ceiling
    mfma_ceiling = mfma_ceiling_block(torch, dev, copies[0], 5)
    log("mfma ceiling:", json.dumps(mfma_ceiling))
    if prefill:
        for v in prefill.values():
            v["frac_of_mfma_ceiling"] = round(v["TFLOP_s"] / mfma_ceiling["TFLOP_s"], 4)

    # ------------------------------------------------------------ per-CU data-path capacities
    capacity = cu_capacity_block(torch, dev)
    log("cu capacity:", json.dumps(capacity))

    # ------------------------------------------------------------ activation quantisation
    quant = quantize_block(torch, g, inputgen, oracle, dev, max(5, args.steps // 10))
    log("quantize:", json.dumps(quant))

    # ------------------------------------------------------------ MX-scaled variant
    mx = {} if args.no_mx else mx_block(torch, g, inputgen, oracle, dev, max(5, args.steps // 10))
    log("mx:", json.dumps(mx))

    # ------------------------------------------------------------ row-wise (per-token) variant
    rowwise = {} if args.no_mx else rowwise_block(torch, g, inputgen, oracle, dev, max(5, args.steps // 10))
    log("rowwise:", json.dumps(rowwise))

    # ------------------------------------------------------------ CPU baseline (the oracle)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_block(inputgen, oracle, A, a_s, W0, w_s, Ms, N, K, args.cpu_seconds)
        log("cpu baseline:", json.dumps(cpu))

    res = {
        "metric": METRIC,
        "value": round(us_per_call, 3),
        "unit": "µs/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 x fp8e4m3 -> fp32 accumulate -> bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, 1x128 / 128x128 fp32 scales)",
        "config": {"workload": f"decode{' qkv-like' if qkv else ''}: M in {{{','.join(map(str, Ms))}}}, "
                               f"N={N}, K={K}, cold weights "
                               f"rotated over {R} copies ({R * w_bytes / 2**30:.2f} GiB); one step = one "
                               f"HIP-graph replay of {R} calls for each M; value = mean over M of us/call",
                   "calls_per_step": R * len(Ms), "rotate_bytes": R * w_bytes,
                   "table_hash": f"0x{g.gemm_a8w8_table_hash():016x}"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic() if qkv else None,
                     "kernel": "M<=16 weight-streaming kernels: "
                               + ", ".join(sorted({v["plan"] for v in per_m.values()})),
                     "bytes_per_launch": round(bytes_mean)},
        "per_m": per_m,
        "mixed_m_graph": mixed,
        "read_ceiling": ceiling,
        "prepacked_weights": packed,
        "fused_quantisation": fused,
        "prefill": prefill,
        "decode_shapes": decode_shapes,
        "mfma_ceiling": mfma_ceiling,
        "cu_capacity": capacity,
        "quantize": quant,
        "mx": mx,
        "rowwise": rowwise,
        "parity": {"worst_rel_l2": round(gate, 6)},
        "wall_s_timed": round(wall, 3),
        "cpu_baseline": cpu,
    }
    if args.calib_copy:
        calib_copy(torch)
    print(json.dumps(res), flush=True)


def calib_copy(torch):
    """A plain device copy of known size (reads and writes 256 MiB), for counter calibration."""
    n = 256 * 2**20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"calibration copy: 3 x {n} bytes read and written")


SWEEP_NK = [(5120, 6144), (14336, 5120), (16384, 5120), (34816, 5120), (256, 6144), (32, 6144)]


def sweep(args, torch, g, inputgen, oracle):
    """Dense arbitrary-M sweep: 256 seeded M in 1..8192 for each (N, K)."""
    dev = "cuda:0"
    Ms = inputgen.random_m_values(256, seed=2)
    rng = np.random.default_rng(6)
    points = []
    fallbacks = 0
    worst_ratio = 0.0
    worst_rel = 0.0
    t_start = time.time()
    for (N, K) in SWEEP_NK:
        A, a_s = inputgen.make_activations(8192, K, seed=0)
        W0, w_s = inputgen.make_weights(N, K, seed=1)
        dA = torch.from_numpy(A).to(dev)
        da = torch.from_numpy(a_s).to(dev)
        dw = torch.from_numpy(w_s).to(dev)
        R = max(2, math.ceil(2**30 / (W0.nbytes + w_s.nbytes)))
        copies = [torch.from_numpy(W0).to(dev)] + \
            [torch.from_numpy(inputgen.sign_flip_copy(W0, seed=1000 + r)).to(dev) for r in range(1, R)]
        picked = []
        ws = g.Workspace((128 << 20) + (1 << 20))
        for M in Ms:
            plan = g.gemm_a8w8_ex_plan(M, N, K, workspace_bytes=ws.nbytes)
            fallbacks += plan["fallback"]
            worst_ratio = max(worst_ratio, plan["key_m"] / M)
            # long calls need no rotation to be cold: cap the graph at ~20 ms of work
            fl = flops(M, N, K)
            est_us = max(algorithmic_bytes(M, N, K) / 6e3, fl / 2e9)
            Rp = max(2, min(R, int(20000 / max(est_us, 1.0))))
            out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            gr = time_graph(torch, [(lambda r=r: g.gemm_a8w8_blockscale(dA[:M], da[:M], copies[r], dw, out=out,
                                                                        workspace=ws))
                                    for r in range(Rp)], 0, 1)
            reps = max(2, int(5000 / (est_us * Rp)))
            us = timed_replays(torch, gr, reps) * 1000.0 / Rp
            del gr
            # the graph's last call used a rotated copy: recompute with copy 0 for the parity check
            g.gemm_a8w8_blockscale(dA[:M], da[:M], copies[0], dw, out=out, workspace=ws)
            rows = sorted({M - 1, int(rng.integers(0, M))})
            picked.append((M, rows, out[rows].float().cpu().numpy().astype(np.float64)))
            by = algorithmic_bytes(M, N, K)
            t_hbm = by / (HBM_PEAK_GBS * 1e3)          # us
            t_mfma = fl / (FP8_PEAK_TFLOPS * 1e6)      # us
            bound = "hbm" if t_hbm >= t_mfma else "mfma"
            frac = max(t_hbm, t_mfma) / us
            points.append({"N": N, "K": K, "M": M, "us": round(us, 3), "bound": bound,
                           "frac": round(frac, 4), "plan": plan["name"], "key_m": plan["key_m"],
                           "fallback": plan["fallback"]})
        union = sorted({r for _, rows, _ in picked for r in rows})
        ref = oracle.gemm(A, a_s, W0, w_s, rows=union)
        pos = {r: i for i, r in enumerate(union)}
        ys = np.concatenate([v for _, _, v in picked])
        refs = np.concatenate([ref[[pos[r] for r in rows]] for _, rows, _ in picked])
        rel = float(np.linalg.norm(ys - refs) / np.linalg.norm(refs))
        worst_rel = max(worst_rel, rel)
        if rel > 3e-3:
            raise SystemExit(f"parity gate failed (sweep N={N} K={K}): rel_l2={rel:.3e}")
        log(f"sweep N={N} K={K}: {len(Ms)} points, parity rel_l2 {rel:.3e}, "
            f"median {np.median([p['frac'] for p in points if p['N'] == N]):.3f} of roofline")
        del copies, dA
        torch.cuda.empty_cache()
    fr = np.array([p["frac"] for p in points])
    summary = {
        "metric": "dense-M sweep: fraction of the binding roofline per call (median over points)",
        "value": round(float(np.median(fr)), 4), "unit": "fraction of roofline", "n_gpus": 1,
        "higher_is_better": True, "data": "synthetic", "dtype": "fp8e4m3 x fp8e4m3 -> fp32 accumulate -> bf16",
        "config": {"workload": "256 M values uniform in 1..8192 (seed 2) x (N,K) in " + str(SWEEP_NK),
                   "table_hash": f"0x{g.gemm_a8w8_table_hash():016x}"},
        "points": len(points), "fallbacks": fallbacks, "max_key_over_m": round(worst_ratio, 4),
        "frac_p10": round(float(np.percentile(fr, 10)), 4), "frac_p90": round(float(np.percentile(fr, 90)), 4),
        "parity_worst_rel_l2": round(worst_rel, 6), "seconds": round(time.time() - t_start, 1),
    }
    if args.sweep_out:
        with open(args.sweep_out, "w") as f:
            f.write("# Dense-M sweep on one MI355X\n\n")
            f.write("Command: `python bench.py --workload sweep --sweep-out <file>`\n\n")
            f.write("```\n" + json.dumps(summary) + "\n```\n\n")
            for (N, K) in SWEEP_NK:
                sub = [p for p in points if p["N"] == N and p["K"] == K]
                f.write(f"## N={N}, K={K}\n\n| M | key M | plan | µs/call | bound | % of roofline |\n"
                        "|---:|---:|---|---:|---|---:|\n")
                for p in sorted(sub, key=lambda p: p["M"]):
                    f.write(f"| {p['M']} | {p['key_m']} | {p['plan']} | {p['us']} | {p['bound']} | "
                            f"{100 * p['frac']:.1f} |\n")
                f.write("\n")
    print(json.dumps(summary), flush=True)


if __name__ == "__main__":
    main()
