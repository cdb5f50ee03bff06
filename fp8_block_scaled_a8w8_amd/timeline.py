"""Per-wave timelines of the row-range skinny (decode) kernel: where a call's time goes.

Loads the timeline build of the library (``python -m fp8_block_scaled_a8w8_amd.build --timeline``),
whose row-range kernel stamps the 100 MHz real-time counter at five points of every wave (entry,
first pass issued, last data consumed, after the reduction barrier, after its store) into the
call's workspace.  For each decode shape it captures one HIP graph of R calls over >= 2 GiB of
rotated weight copies (cold weights, as the benchmark), replays it, reads the stamps of the
graph's last call, and prints per-workgroup phase percentiles beside the graph's time per call:
the difference between the two is the time a call spends outside its waves (dispatch, the
kernel-boundary fences).  Two reference rows follow: the graph time per call of a near-empty
kernel (256 workgroups reading 4 KB each: the floor a graph node costs) and of the streaming-read
ceiling kernel at qkv's byte count.

    python -m fp8_block_scaled_a8w8_amd.timeline [--reps 3]
"""
from __future__ import annotations

import argparse
import ctypes
import math
import os

import numpy as np
import torch

import inputgen
from fp8_block_scaled_a8w8_amd import SCALE_KINDS, GemmDesc, gemm_a8w8_ex_plan, variants
from fp8_block_scaled_a8w8_amd.build import CEILINGS_LIB, TIMELINE_LIB

SHAPES = [(5120, 6144, 1, "rskinny_t2_d3_w16_g1"), (5120, 6144, 16, "rskinny_t2_d3_w16_g1"),
          (14336, 5120, 1, "rskinny_t4_d5_w8_g1"), (14336, 5120, 8, "rskinny_t4_d5_w8_g1"),
          (14336, 5120, 16, "rskinny_t4_d5_w8_g1")]
COUNTER_BYTES = 65536
TICK_US = 0.01                      # s_memrealtime: 100 MHz


def _lib():
    if not os.path.exists(TIMELINE_LIB):
        raise SystemExit(f"{TIMELINE_LIB} is missing: python -m fp8_block_scaled_a8w8_amd.build --timeline")
    L = ctypes.CDLL(TIMELINE_LIB)
    L.gemm_a8w8_ex.restype = ctypes.c_int
    L.gemm_a8w8_ex.argtypes = [ctypes.POINTER(GemmDesc), ctypes.c_void_p]
    L.gemm_a8w8_workspace_init.restype = ctypes.c_int
    L.gemm_a8w8_workspace_init.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    return L


def phases(rec: np.ndarray, groups: int, waves: int) -> dict:
    """Per-workgroup phase times (us from the first wave's entry) from the stamp records."""
    t = rec[: groups * waves * 6].reshape(groups, waves, 6).astype(np.int64)
    rel = (t[:, :, :5] - t[:, :, 0].min()) * TICK_US
    start, issued, data = rel[:, :, 0].min(1), rel[:, :, 1].max(1), rel[:, :, 2].max(1)
    barrier, end = rel[:, :, 3].max(1), rel[:, :, 4].max(1)
    return {"span": float(end.max()), "start": start, "issued": issued, "data": data, "barrier": barrier,
            "end": end, "tail": end - data}


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=3)
    args = ap.parse_args()
    L = _lib()
    dev = "cuda:0"
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    by_name = {v["name"]: v for v in variants()}
    ws_bytes = 8 << 20
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    assert L.gemm_a8w8_workspace_init(ws.data_ptr(), ws_bytes, torch.cuda.current_stream().cuda_stream) == 0
    print("| shape | M | instance | graph µs/call | span µs | outside waves µs | start p90 | issued p50 | "
          "data p50 / max | tail p50 | end p0 / p50 / max |")
    print("|---|---:|---|---:|---:|---:|---:|---:|---:|---:|---:|")
    for N, K, M, name in SHAPES:
        v = by_name[name]
        groups = int(gemm_a8w8_ex_plan(M, N, K, variant=v["variant"], cu_count=cus)["grid"])
        W0, w_s = inputgen.make_weights(N, K, seed=1)
        R = math.ceil(2 * 2**30 / W0.nbytes)
        copies = [torch.from_numpy(W0 if r == 0 else inputgen.sign_flip_copy(W0, seed=100 + r)).to(dev)
                  for r in range(R)]
        A, a_s = inputgen.make_activations(M, K, seed=3)
        dA, da, dw = (torch.from_numpy(x).to(dev) for x in (A, a_s, w_s))
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        descs = [GemmDesc(dA.data_ptr(), da.data_ptr(), c.data_ptr(), dw.data_ptr(), out.data_ptr(), 1, M, N, K,
                          SCALE_KINDS["block"], 0, v["variant"], 0, ws.data_ptr(), ws_bytes) for c in copies]
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())

        def calls():
            for d in descs:
                rc = L.gemm_a8w8_ex(ctypes.byref(d), s.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"gemm_a8w8_ex failed ({rc})")
        with torch.cuda.stream(s):
            calls()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            calls()
        torch.cuda.synchronize()
        for _ in range(args.reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1000.0 / R
        rec = ws[COUNTER_BYTES:].view(torch.int64).cpu().numpy()
        ph = phases(rec, groups, v["waves"])
        p = np.percentile
        print(f"| {N}×{K} | {M} | {name} | {us:.2f} | {ph['span']:.2f} | {us - ph['span']:.2f} | "
              f"{p(ph['start'], 90):.2f} | {p(ph['issued'], 50):.2f} | {p(ph['data'], 50):.2f} / "
              f"{ph['data'].max():.2f} | {p(ph['tail'], 50):.2f} | {ph['end'].min():.2f} / "
              f"{p(ph['end'], 50):.2f} / {ph['end'].max():.2f} |", flush=True)
        del graph, copies
        torch.cuda.empty_cache()
    floor_and_read(dev, args.reps)


def _graph_us(dev, launch, R, reps):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for r in range(R):
            launch(r, s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        for r in range(R):
            launch(r, s)
    torch.cuda.synchronize()
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000.0 / R


def floor_and_read(dev, reps):
    C = ctypes.CDLL(CEILINGS_LIB)
    C.a8w8_read_ceiling_launch.restype = ctypes.c_int
    C.a8w8_read_ceiling_launch.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_void_p]
    sink = torch.zeros(8192, dtype=torch.int32, device=dev)
    small = torch.ones(256 * 4096, dtype=torch.uint8, device=dev)

    def tiny(r, s):
        assert C.a8w8_read_ceiling_launch(small.data_ptr(), small.numel(), sink.data_ptr(), 256, 16,
                                          s.cuda_stream) == 0
    us = _graph_us(dev, tiny, 64, reps)
    print(f"| graph floor: near-empty kernel | - | read_kernel, 256 WGs x 4 KB | {us:.2f} | | | | | | | |")
    nbytes = 14336 * 5120
    R = math.ceil(2 * 2**30 / nbytes)
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(R)]

    def read(r, s):
        assert C.a8w8_read_ceiling_launch(bufs[r].data_ptr(), nbytes, sink.data_ptr(), 4096, 8,
                                          s.cuda_stream) == 0
    us = _graph_us(dev, read, R, reps)
    print(f"| read ceiling at 14336×5120 bytes | - | read_kernel, 4096 WGs | {us:.2f} | | | | | | | |")


if __name__ == "__main__":
    main()
