#!/usr/bin/env python3
"""Throughput of the block-scaled quantizer hot path on one MI355X.

One step = one pass of the whole path over the layer-step workload (the one workload that
runs every stage): MXFP8 dual (rowwise 1x32 + columnwise 32x1) quantization of BF16
activations A[65536,2048] and weights W[2048,6144], per-token NVFP4 quantization of the
524288 routed rows X[524288,2048] grouped by 128 experts (Zipf(1.1) load skew), then the
BF16 dequantization of all six outputs -- eight kernel launches on one stream, inputs
resident in HBM.

Metric: algorithmic HBM bytes (every input byte read once, every output byte written once)
per second.  The dominant kernel (NVFP4 grouped quantize, 2.75 GB per launch) is also
timed on its own with HIP events on its stream, to report its fraction of the HBM
roofline; the CPU oracle is timed on a bounded sample of the same step.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--profile-pass]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "quantize/dequantize HBM GB/s (bytes read+written) and % of MI355X HBM peak"
HBM_PEAK_GBS = 8000.0                      # MI355X HBM3E, AMD public specification

WORKLOAD = ("layer-step stream: MXFP8 dual quant of A[65536,2048] and W[2048,6144] BF16, "
            "per-token NVFP4 grouped quant of X[524288,2048] (65536 tokens x top-8 of 128 "
            "experts, Zipf(1.1)), BF16 dequant of all outputs")


def mx_both_bytes(M, K):        # read BF16, write two E4M3 copies + two E8M0 scale arrays
    return 2 * M * K + 2 * (M * K + M * K // 32)


def mx_dq_bytes(M, K):          # read E4M3 + E8M0, write BF16
    return M * K + M * K // 32 + 2 * M * K


def nv_bytes(R, K):             # BF16 <-> packed E2M1 + E4M3 per 16 + FP32 per row
    return 2 * R * K + R * K // 2 + R * K // 16 + 4 * R


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample", type=int, default=1,
                   help="the CPU baseline runs 1/N of the step's rows")
    p.add_argument("--profile-pass", action="store_true",
                   help="short run for hardware-counter passes: one 1 GiB device copy (the "
                        "counter calibration kernel), then the steps")
    return p.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the quantizer path is row-local and this build runs "
              "on a single MI355X (see DESIGN.md for how it would shard); --gpus %d is not "
              "supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import block_scaled_precision_mxfp8_amd as bsq
    import workloads

    if not os.path.exists(bsq.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    bsq.lib()

    dev = torch.device("cuda:0")
    t_gen = time.time()
    cfg = workloads.config5()
    a_np, w_np, tok, off = cfg["a"], cfg["w"], cfg["token_idx"], cfg["offsets"]

    def dev_bf16(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    A, W = dev_bf16(a_np), dev_bf16(w_np)
    tok_d = torch.from_numpy(tok).to(dev)
    X = A.index_select(0, tok_d)
    offsets = torch.from_numpy(off).to(dev)
    (MA, KA), (MW, KW), (RX, KX) = A.shape, W.shape, X.shape
    gen_s = time.time() - t_gen

    # outputs, allocated once (the library never allocates)
    u8, bf = torch.uint8, torch.bfloat16
    a_out = (torch.empty(MA, KA, dtype=u8, device=dev), torch.empty(MA, KA // 32, dtype=u8, device=dev),
             torch.empty(KA, MA, dtype=u8, device=dev), torch.empty(KA, MA // 32, dtype=u8, device=dev))
    w_out = (torch.empty(MW, KW, dtype=u8, device=dev), torch.empty(MW, KW // 32, dtype=u8, device=dev),
             torch.empty(KW, MW, dtype=u8, device=dev), torch.empty(KW, MW // 32, dtype=u8, device=dev))
    xq = torch.empty(RX, KX // 2, dtype=u8, device=dev)
    xsb = torch.empty(RX, KX // 16, dtype=u8, device=dev)
    xst = torch.empty(RX, dtype=torch.float32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    ya = (torch.empty(MA, KA, dtype=bf, device=dev), torch.empty(KA, MA, dtype=bf, device=dev))
    yw = (torch.empty(MW, KW, dtype=bf, device=dev), torch.empty(KW, MW, dtype=bf, device=dev))
    yx = torch.empty(RX, KX, dtype=bf, device=dev)

    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(max(args.steps, 1))]

    def step(i=None):
        bsq.mx_quantize_mxfp8(A, "both", *a_out, stream=stream)
        bsq.mx_quantize_mxfp8(W, "both", *w_out, stream=stream)
        if i is not None:
            ev[i][0].record(stream)
        bsq.nv_quantize_nvfp4_per_token_grouped(X, offsets, xq, xsb, xst, status, stream=stream)
        if i is not None:
            ev[i][1].record(stream)
        bsq.mx_dequantize(a_out[0], a_out[1], ya[0], stream=stream)
        bsq.mx_dequantize(a_out[2], a_out[3], ya[1], stream=stream)
        bsq.mx_dequantize(w_out[0], w_out[1], yw[0], stream=stream)
        bsq.mx_dequantize(w_out[2], w_out[3], yw[1], stream=stream)
        bsq.nv_dequantize(xq, xsb, xst, yx, stream=stream)

    if args.profile_pass:
        src = torch.empty(1 << 29, dtype=torch.int16, device=dev).fill_(1)   # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if int(status.item()) != bsq.BSQ_OK:
        raise RuntimeError("expert offsets rejected by the device check")

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    bytes_step = (mx_both_bytes(MA, KA) + mx_both_bytes(MW, KW) + nv_bytes(RX, KX)
                  + 2 * mx_dq_bytes(MA, KA) + 2 * mx_dq_bytes(MW, KW) + nv_bytes(RX, KX))
    elems_step = 2 * MA * KA + 2 * MW * KW + RX * KX + 2 * MA * KA + 2 * MW * KW + RX * KX
    ms_step = elapsed * 1e3 / max(args.steps, 1)
    gbs = bytes_step * args.steps / elapsed / 1e9

    nv_ms = [s.elapsed_time(e) for s, e in ev[:args.steps]]
    nv_avg_s = float(np.mean(nv_ms)) / 1e3 if nv_ms else float("nan")
    nv_launch_bytes = nv_bytes(RX, KX)
    nv_gbs = nv_launch_bytes / nv_avg_s / 1e9

    out = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "bytes_per_step": bytes_step,
                   "elements_per_step": elems_step, "parallelism": "single GPU",
                   "launches_per_step": 8},
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "elements_per_s": round(elems_step * args.steps / elapsed, 1),
        "roofline": {"bound": "hbm", "kernel": "nv_quant_rows_kernel<4> (grouped, 524288x2048)",
                     "achieved": round(nv_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(nv_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": nv_launch_bytes,
                     "avg_launch_us": round(nv_avg_s * 1e6, 2)},
        "cpu_baseline": None,
        "setup_s": round(gen_s, 1),
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(a_np, w_np, tok, args.cpu_sample)

    print(json.dumps(out), flush=True)


def cpu_baseline(a_np, w_np, tok, frac):
    """The CPU oracle (as it stands, OpenMP over rows) on 1/frac of the step's rows: the
    first M/frac rows of A (both copies), the first rows of W, the first R/frac routed
    rows, and the dequantization of all of those outputs."""
    import oracle

    MA = (a_np.shape[0] // frac) // 32 * 32
    MW = max(32, (w_np.shape[0] // frac) // 32 * 32)
    RX = tok.size // frac
    a_s = np.ascontiguousarray(a_np[:MA])
    w_s = np.ascontiguousarray(w_np[:MW])
    x_s = a_np[tok[:RX]]
    oracle.lib()
    t0 = time.perf_counter()
    for m in (a_s, w_s):
        qr, sr = oracle.mx_quantize_rowwise(m)
        qc, sc = oracle.mx_quantize_colwise(m)
        oracle.mx_dequantize(qr, sr)
        oracle.mx_dequantize(qc, sc)
    q, sb, st = oracle.nv_quantize_per_token(x_s)
    oracle.nv_dequantize(q, sb, st)
    dt = time.perf_counter() - t0
    KA, KW, KX = a_s.shape[1], w_s.shape[1], x_s.shape[1]
    b = (mx_both_bytes(MA, KA) + mx_both_bytes(MW, KW) + 2 * nv_bytes(RX, KX)
         + 2 * mx_dq_bytes(MA, KA) + 2 * mx_dq_bytes(MW, KW))
    return {"value": round(b / dt / 1e9, 3), "unit": "GB/s", "cores": oracle.max_threads(),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": "1/%d of the step: A[:%d] and W[:%d] MXFP8 dual + dequant of both copies, "
                      "%d routed rows NVFP4 + dequant" % (frac, MA, MW, RX)}


if __name__ == "__main__":
    main()
