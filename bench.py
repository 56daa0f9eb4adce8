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
                       [--profile-pass] [--all-configs] [--profile-op OP] [--hbm-ceiling]
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


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "nv_quant_grouped_524288x2048_traffic.json")


def measured_traffic():
    """HBM bytes per launch of the dominant kernel, from the committed FETCH_SIZE/WRITE_SIZE
    counter passes (scaled by the 1 GiB copy calibration), or None when the kernel's sources
    have changed since the counters were taken."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_RECORD))
        h = hashlib.sha256()
        for p in rec["kernel_sources"]:
            with open(os.path.join(ROOT, p), "rb") as fh:
                h.update(fh.read())
    except (OSError, KeyError, ValueError):
        return None
    return rec["traffic_bytes_per_launch"] if h.hexdigest() == rec["kernel_sources_sha256"] else None


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample", type=int, default=1,
                   help="the CPU baseline runs 1/N of the step's rows")
    p.add_argument("--cpu-reps", type=int, default=2,
                   help="times the CPU baseline's sample is run inside its timed region "
                        "(about 10 s of CPU work on a 16-core share at the defaults)")
    p.add_argument("--all-configs", action="store_true",
                   help="instead of the step: time every kernel of the five workloads on its own "
                        "(512 MiB cache flush before each launch) and print one JSON line per op")
    p.add_argument("--profile-pass", action="store_true",
                   help="short run for hardware-counter passes: one 1 GiB device copy (the "
                        "counter calibration kernel), then the steps")
    p.add_argument("--hbm-ceiling", action="store_true",
                   help="instead of the step: time the byte-moving probes of tests/probes "
                        "(read, write and copy; memory-only copies of the access patterns of the "
                        "NVFP4 quantizer and dequantizer, the quantize-then-scatter and the MXFP8 "
                        "dual quantizer) next to the kernels themselves, one JSON line each")
    p.add_argument("--profile-op", choices=sorted(PROFILE_OPS),
                   help="counter pass of one extended op: one 1 GiB device copy, then the op "
                        "twice on random inputs of the benchmark's shapes")
    return p.parse_args()


PROFILE_OPS = ("per_group_quant", "per_group_dequant", "tile16_quant", "tile16_dequant",
               "scatter", "grouped_dual", "grouped_colwise", "workload2", "workload4")


def profile_op(torch, bsq, workloads, dev, op):
    """One op, twice, after a 1 GiB copy, for rocprofv3 counter passes: the ops of workload
    2 (MXFP8 dual quant of 8192 x 2048 and both dequants) and of workload 4 (per-row NVFP4
    and rowwise MXFP8 of the stacked gate_up and down weights, with their dequants), the
    per-expert-scale and 16x16-tile NVFP4 export of the stacked gate_up weights (196608 x
    2048, 128 groups), quantize-then-scatter of 65536 tokens to 8 routed rows each, and
    grouped MXFP8 of 524288 x 2048 rows over 128 experts with Zipf(1.1) top-8 routing."""
    torch.manual_seed(0)
    u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
    src = torch.empty(1 << 29, dtype=torch.int16, device=dev).fill_(1)
    dst = torch.empty_like(src)
    if op == "workload2":
        # MXFP8 dual quant of the 8192 x 2048 activations, dequant of both copies
        x = torch.from_numpy(workloads.config2()["x"].view(np.int16)).view(bf).to(dev)
        M, K = x.shape
        out = (torch.empty(M, K, dtype=u8, device=dev), torch.empty(M, K // 32, dtype=u8, device=dev),
               torch.empty(K, M, dtype=u8, device=dev), torch.empty(K, M // 32, dtype=u8, device=dev))
        yr, yc = torch.empty(M, K, dtype=bf, device=dev), torch.empty(K, M, dtype=bf, device=dev)

        def fn():
            bsq.mx_quantize_mxfp8(x, "both", *out)
            bsq.mx_dequantize(out[0], out[1], yr)
            bsq.mx_dequantize(out[2], out[3], yc)
    elif op == "workload4":
        # per-row NVFP4 and rowwise MXFP8 of the stacked expert weights, and their dequant
        ws = [(torch.randn(M, K, device=dev) * 0.02).to(bf) for M, K in ((196608, 2048), (262144, 768))]
        bufs = []
        for w in ws:
            M, K = w.shape
            bufs.append(((torch.empty(M, K // 2, dtype=u8, device=dev), torch.empty(M, K // 16, dtype=u8, device=dev),
                          torch.empty(M, dtype=f32, device=dev)),
                         (torch.empty(M, K, dtype=u8, device=dev), torch.empty(M, K // 32, dtype=u8, device=dev)),
                         torch.empty(M, K, dtype=bf, device=dev)))

        def fn():
            for w, (nv_out, mx_out, y) in zip(ws, bufs):
                bsq.nv_quantize_nvfp4_per_token(w, *nv_out)
                bsq.nv_dequantize(*nv_out, y)
                bsq.mx_quantize_mxfp8(w, "rowwise", *mx_out)
                bsq.mx_dequantize(*mx_out, y)
    elif op.startswith(("per_group", "tile16")):
        M, K, rows = 196608, 2048, 1536
        w = (torch.randn(M, K, device=dev) * 0.02).to(bf)
        off = torch.arange(0, M + 1, rows, dtype=torch.int64, device=dev)
        q, y = torch.empty(M, K // 2, dtype=u8, device=dev), torch.empty(M, K, dtype=bf, device=dev)
        sb, sb2 = torch.empty(M, K // 16, dtype=u8, device=dev), torch.empty(M // 16, K // 16, dtype=u8, device=dev)
        sg, st = torch.empty(M // rows, dtype=f32, device=dev), torch.zeros(1, dtype=torch.int32, device=dev)
        if op == "per_group_dequant":
            bsq.nv_quantize_nvfp4_per_group(w, off, q, sb, sg, st)
        if op == "tile16_dequant":
            bsq.nv_quantize_nvfp4_2d(w, off, q, sb2, sg, st)
        fn = {"per_group_quant": lambda: bsq.nv_quantize_nvfp4_per_group(w, off, q, sb, sg, st),
              "per_group_dequant": lambda: bsq.nv_dequantize_per_group(q, sb, sg, off, y),
              "tile16_quant": lambda: bsq.nv_quantize_nvfp4_2d(w, off, q, sb2, sg, st),
              "tile16_dequant": lambda: bsq.nv_dequantize_2d(q, sb2, sg, off, y)}[op]
    elif op == "scatter":
        T, K, k = 65536, 2048, 8
        h = (torch.randn(T, K, device=dev) * 2).to(bf)
        rows_of = torch.randperm(T * k, device=dev).reshape(T, k)
        N = T * k
        out = (torch.empty(N, K // 2, dtype=u8, device=dev), torch.empty(N, K // 16, dtype=u8, device=dev),
               torch.empty(N, dtype=f32, device=dev), torch.zeros(1, dtype=torch.int32, device=dev))
        fn = lambda: bsq.nv_quantize_nvfp4_per_token_scatter(h, rows_of, N, *out)
    else:
        M, K = 524288, 2048
        x = (torch.randn(M, K, device=dev) * 2).to(bf)
        _, off_np = workloads.zipf_routing(np.random.default_rng(4), 65536, 128, 8)
        off = torch.from_numpy(off_np).to(dev)
        s_ld = bsq.mx_group_scale_entries(M, off.numel() - 1)
        out = (torch.empty(M, K, dtype=u8, device=dev), torch.empty(M, K // 32, dtype=u8, device=dev),
               torch.empty(K, M, dtype=u8, device=dev), torch.empty(K, s_ld, dtype=u8, device=dev),
               torch.zeros(1, dtype=torch.int32, device=dev))
        if op == "grouped_dual":
            fn = lambda: bsq.mx_quantize_mxfp8_grouped(x, off, "both", s_ld, *out)
        else:
            fn = lambda: bsq.mx_quantize_mxfp8_grouped(x, off, "colwise", s_ld, None, None, *out[2:])
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    print(json.dumps({"profile_op": op}), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the quantizer path is row-local, so it would shard by "
              "rows (each GPU quantizing its own rows and experts, with no communication) and is "
              "measured on a single MI355X; --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import block_scaled_precision_mxfp8_amd as bsq
    import workloads

    if not os.path.exists(bsq.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    bsq.lib()

    dev = torch.device("cuda:0")
    if args.all_configs:
        return all_configs(torch, bsq, workloads, dev)
    if args.profile_op:
        return profile_op(torch, bsq, workloads, dev, args.profile_op)
    if args.hbm_ceiling:
        return hbm_ceiling(torch, bsq, dev)
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
        "dtype": "bf16",
        "arithmetic": "bf16 in; binary32 IEEE scale and NVFP4 products, integer BF16-magnitude "
                      "maxima and E8M0 codes; out E4M3/E8M0/E2M1 codes, f32 token scales, bf16 dequant",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "bytes_per_step": bytes_step,
                   "elements_per_step": elems_step, "parallelism": "single GPU",
                   "launches_per_step": 8},
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "elements_per_s": round(elems_step * args.steps / elapsed, 1),
        "roofline": {"bound": "hbm", "kernel": "nv_quant_rows_kernel<4> (grouped, 524288x2048)",
                     "achieved": round(nv_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(nv_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "bytes_per_launch": nv_launch_bytes,
                     "avg_launch_us": round(nv_avg_s * 1e6, 2)},
        "cpu_baseline": None,
        "setup_s": round(gen_s, 1),
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(a_np, w_np, tok, args.cpu_sample, args.cpu_reps)

    print(json.dumps(out), flush=True)


def hbm_ceiling(torch, bsq, dev, reps=21):
    """What moving the bytes costs on this device, without arithmetic: a 2 GiB read, 2 GiB
    writes and 2 GiB -> 2 GiB copies (one 16-byte piece per lane, non-temporal loads; stores
    non-temporal or ordinary), and the per-token NVFP4 quantizer's own access pattern on
    524288 rows of 2048 BF16, timed beside the quantizer on the same rows, the dequantizer's
    pattern beside the dequantizer on the quantizer's outputs, and the quantize-then-scatter's
    pattern beside it (65536 tokens to the 524288 Zipf-routed rows); a 256 MiB copy
    and the MXFP8 dual quantizer's access pattern beside that quantizer on the layer step's
    65536 x 2048 activations, and a 24 MiB copy with the same pattern and quantizer on its
    2048 x 6144 weights (each copy reads and writes about as much).  Each launch
    follows a read of a 512 MiB buffer; "alone" is the median of HIP events around the
    launch, "with next read" times the launch together with the next 512 MiB read and
    subtracts that read's own time, which counts write-backs a launch leaves for later."""
    import ctypes
    sys.path.insert(0, os.path.join(ROOT, "tests", "probes"))
    import build_probe
    if not os.path.exists(build_probe.HBM_LIB):
        build_probe.build()
    hp = ctypes.CDLL(build_probe.HBM_LIB)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    flush = torch.ones(1 << 26, dtype=torch.int64, device=dev)
    n16 = 1 << 27                                         # 2 GiB in 16-byte pieces
    x = torch.empty(n16 * 8, dtype=torch.int16, device=dev)
    for c in range(8):                                    # finite BF16 bit patterns
        part = x[c * n16:(c + 1) * n16]
        part.copy_(torch.randint(0, 0x7F80, (n16,), dtype=torch.int32, device=dev).to(torch.int16))
    y = torch.empty_like(x)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    R, K = 524288, 2048
    q = torch.empty(R, K // 2, dtype=torch.uint8, device=dev)
    sb = torch.empty(R, K // 16, dtype=torch.uint8, device=dev)
    st = torch.empty(R, dtype=torch.float32, device=dev)
    xb = x.view(torch.bfloat16).view(R, K)
    yb = y.view(torch.bfloat16).view(R, K)
    T = 65536                                             # tokens routed to 8 of 128 experts (Zipf 1.1)
    import workloads
    tok, _ = workloads.zipf_routing(np.random.default_rng(4), T, 128, 8)
    dst = torch.from_numpy(workloads.scatter_rows(tok, T, 8)).to(dev)
    scb = 2 * T * K + R * (K // 2 + K // 16 + 4) + 8 * T * 8
    MA = 65536                                            # the layer step's activations
    a = xb[:MA]
    a_out = (torch.empty(MA, K, dtype=torch.uint8, device=dev), torch.empty(MA, K // 32, dtype=torch.uint8, device=dev),
             torch.empty(K, MA, dtype=torch.uint8, device=dev), torch.empty(K, MA // 32, dtype=torch.uint8, device=dev))
    MW, KW = 2048, 6144                                   # the layer step's weights
    w = x.view(torch.bfloat16)[:MW * KW].view(MW, KW)
    w_out = (torch.empty(MW, KW, dtype=torch.uint8, device=dev), torch.empty(MW, KW // 32, dtype=torch.uint8, device=dev),
             torch.empty(KW, MW, dtype=torch.uint8, device=dev), torch.empty(KW, MW // 32, dtype=torch.uint8, device=dev))
    P = lambda t: ctypes.c_void_p(t.data_ptr())

    def timed(fn, follow):
        ts = []
        for _ in range(reps):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            if follow:
                flush.sum()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return float(np.median(ts))

    def ok(rc):
        if rc != 0:
            raise RuntimeError("probe launch failed: %d" % rc)

    gi = 2 * n16 * 16
    nvb = nv_bytes(R, K)
    probes = [
        ("read 2 GiB", gi // 2, lambda: ok(hp.hbm_probe_read(P(x), ctypes.c_int64(n16), P(sink), sp))),
        ("write 2 GiB, non-temporal", gi // 2, lambda: ok(hp.hbm_probe_write(P(y), ctypes.c_int64(n16), 1, sp))),
        ("write 2 GiB, ordinary", gi // 2, lambda: ok(hp.hbm_probe_write(P(y), ctypes.c_int64(n16), 0, sp))),
        ("copy 2 GiB, non-temporal stores", gi, lambda: ok(hp.hbm_probe_copy(P(x), P(y), ctypes.c_int64(n16), 1, sp))),
        ("copy 2 GiB, ordinary stores", gi, lambda: ok(hp.hbm_probe_copy(P(x), P(y), ctypes.c_int64(n16), 0, sp))),
        ("NVFP4 quantizer access pattern, 524288x2048, no arithmetic", nvb,
         lambda: ok(hp.hbm_probe_nv_pattern(P(x), ctypes.c_int64(R), P(q), P(sb), P(st), sp))),
        ("NVFP4 per-token quantizer (nv_quant_rows_kernel), 524288x2048", nvb,
         lambda: bsq.nv_quantize_nvfp4_per_token(xb, q, sb, st, stream=stream)),
        ("NVFP4 dequantizer access pattern, 524288x2048, no arithmetic", nvb,
         lambda: ok(hp.hbm_probe_nv_dequant_pattern(P(q), P(sb), P(st), ctypes.c_int64(R), ctypes.c_int64(K),
                                                    P(y), sp))),
        ("NVFP4 per-token dequantizer (nv_dequant_kernel), 524288x2048", nvb,
         lambda: bsq.nv_dequantize(q, sb, st, yb, stream=stream)),
        ("quantize-then-scatter access pattern, 65536 tokens x 2048 -> 524288 rows, no arithmetic", scb,
         lambda: ok(hp.hbm_probe_scatter_pattern(P(x), ctypes.c_int64(T), P(dst), 8, ctypes.c_int64(R),
                                                 P(q), P(sb), P(st), sp))),
        ("NVFP4 quantize-then-scatter (nv_quant_scatter_kernel), 65536 tokens x 2048 -> 524288 rows", scb,
         lambda: ok(bsq.lib().nv_quantize_nvfp4_per_token_scatter(x.data_ptr(), T, K, dst.data_ptr(), 8, R,
                                                                  q.data_ptr(), sb.data_ptr(), st.data_ptr(),
                                                                  None, stream.cuda_stream))),
        ("copy 256 MiB, non-temporal stores", 2 * (gi // 16),
         lambda: ok(hp.hbm_probe_copy(P(x), P(y), ctypes.c_int64(n16 // 8), 1, sp))),
        ("MXFP8 dual quantizer access pattern, 65536x2048, no arithmetic", mx_both_bytes(MA, K),
         lambda: ok(hp.hbm_probe_mx_dual_pattern(P(a), ctypes.c_int64(MA), ctypes.c_int64(K), *map(P, a_out), sp))),
        ("MXFP8 dual quantizer (mx_quant_tile_kernel), 65536x2048", mx_both_bytes(MA, K),
         lambda: bsq.mx_quantize_mxfp8(a, "both", *a_out, stream=stream)),
        ("copy 24 MiB, non-temporal stores", 4 * MW * KW,
         lambda: ok(hp.hbm_probe_copy(P(x), P(y), ctypes.c_int64(2 * MW * KW // 16), 1, sp))),
        ("MXFP8 dual quantizer access pattern, 2048x6144, no arithmetic", mx_both_bytes(MW, KW),
         lambda: ok(hp.hbm_probe_mx_dual_pattern(P(w), ctypes.c_int64(MW), ctypes.c_int64(KW), *map(P, w_out), sp))),
        ("MXFP8 dual quantizer (mx_quant_tile_kernel), 2048x6144", mx_both_bytes(MW, KW),
         lambda: bsq.mx_quantize_mxfp8(w, "both", *w_out, stream=stream)),
    ]
    for _, _, fn in probes:                               # warm-up and launch checks
        fn()
    torch.cuda.synchronize()
    t_read = timed(lambda: None, True)
    for name, nbytes, fn in probes:
        alone = timed(fn, False)
        follow = timed(fn, True) - t_read
        print(json.dumps({"probe": name, "bytes": nbytes, "alone_us": round(alone, 1),
                          "with_next_read_us": round(follow, 1), "GB_s": round(nbytes / alone / 1e3, 1),
                          "pct_hbm_peak": round(nbytes / alone / 1e3 / HBM_PEAK_GBS * 100, 1)}), flush=True)


def all_configs(torch, bsq, workloads, dev, reps=21):
    """Median time of each op of each workload.  Before each launch a 512 MiB buffer is read
    (a reduction, so the caches are left holding clean lines of that buffer): no input of
    the timed op is served from the 256 MiB Infinity Cache or the L2, and no dirty lines of
    the flush are written back while the op runs."""
    flush = torch.ones(1 << 26, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()

    def bf(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    def timed(fn):
        ts = []
        for i in range(reps):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return float(np.median(ts))

    def report(cfg, op, shape, nbytes, elems, fn):
        us = timed(fn)
        print(json.dumps({"config": cfg, "op": op, "shape": shape, "bytes": nbytes, "median_us": round(us, 2),
                          "GB_s": round(nbytes / us / 1e3, 1), "pct_hbm_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS * 100, 1),
                          "elems_per_s": round(elems / us * 1e6, 1)}), flush=True)

    def mx_row(x):
        M, K = x.shape
        out = (torch.empty(M, K, dtype=torch.uint8, device=dev), torch.empty(M, K // 32, dtype=torch.uint8, device=dev))
        return out, lambda: bsq.mx_quantize_mxfp8(x, "rowwise", out[0], out[1], stream=stream)

    def mx_both(x):
        M, K = x.shape
        u8 = torch.uint8
        out = (torch.empty(M, K, dtype=u8, device=dev), torch.empty(M, K // 32, dtype=u8, device=dev),
               torch.empty(K, M, dtype=u8, device=dev), torch.empty(K, M // 32, dtype=u8, device=dev))
        return out, lambda: bsq.mx_quantize_mxfp8(x, "both", *out, stream=stream)

    def mx_dq(q, s):
        y = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        return y, lambda: bsq.mx_dequantize(q, s, y, stream=stream)

    def nv(x, off=None):
        R, K = x.shape
        out = (torch.empty(R, K // 2, dtype=torch.uint8, device=dev), torch.empty(R, K // 16, dtype=torch.uint8, device=dev),
               torch.empty(R, dtype=torch.float32, device=dev))
        if off is None:
            return out, lambda: bsq.nv_quantize_nvfp4_per_token(x, *out, stream=stream)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        return out, lambda: bsq.nv_quantize_nvfp4_per_token_grouped(x, off, *out, status, stream=stream)

    def nv_dq(q, sb, st):
        y = torch.empty(q.shape[0], 2 * q.shape[1], dtype=torch.bfloat16, device=dev)
        return y, lambda: bsq.nv_dequantize(q, sb, st, y, stream=stream)

    def run(cfg, name, x, kind, off=None):
        M, K = x.shape
        shape = "%dx%d" % (M, K)
        if kind == "mx_row":
            out, fn = mx_row(x)
            report(cfg, "mxfp8 rowwise quant " + name, shape, mx_both_bytes(M, K) - (M * K + M * K // 32), M * K, fn)
            fn()
            y, fn = mx_dq(out[0], out[1])
            report(cfg, "mxfp8 dequant " + name, shape, mx_dq_bytes(M, K), M * K, fn)
        elif kind == "mx_both":
            out, fn = mx_both(x)
            report(cfg, "mxfp8 dual quant " + name, shape, mx_both_bytes(M, K), M * K, fn)
            fn()
            y, fn = mx_dq(out[0], out[1])
            report(cfg, "mxfp8 dequant rowwise copy " + name, shape, mx_dq_bytes(M, K), M * K, fn)
            y, fn = mx_dq(out[2], out[3])
            report(cfg, "mxfp8 dequant columnwise copy " + name, "%dx%d" % (K, M), mx_dq_bytes(K, M), M * K, fn)
        else:
            out, fn = nv(x, off)
            report(cfg, "nvfp4 per-token quant%s %s" % (" grouped" if off is not None else "", name), shape,
                   nv_bytes(M, K), M * K, fn)
            fn()
            y, fn = nv_dq(*out)
            report(cfg, "nvfp4 dequant " + name, shape, nv_bytes(M, K), M * K, fn)
        torch.cuda.synchronize()

    run(1, "x", bf(workloads.config1()["x"]), "mx_row")
    run(2, "x", bf(workloads.config2()["x"]), "mx_both")
    c3 = workloads.config3(materialize=False)
    h = bf(c3["h"])
    run(3, "routed rows", h.index_select(0, torch.from_numpy(c3["token_idx"]).to(dev)), "nv",
        torch.from_numpy(c3["offsets"]).to(dev))
    del h
    c4 = workloads.config4()
    for key, rows in (("gate_up", 1536), ("down", 2048)):
        w = bf(c4[key])
        run(4, key, w, "nv")
        run(4, key, w, "mx_row")
        # standard NVFP4 export with one FP32 scale per expert tensor (gate and up share it):
        # two passes over the weights, so x is read twice
        M, K = w.shape
        G = M // rows
        off = torch.arange(0, M + 1, rows, dtype=torch.int64, device=dev)
        g_out = (torch.empty(M, K // 2, dtype=torch.uint8, device=dev), torch.empty(M, K // 16, dtype=torch.uint8, device=dev),
                 torch.empty(G, dtype=torch.float32, device=dev), torch.zeros(1, dtype=torch.int32, device=dev))
        report(4, "nvfp4 per-expert-scale quant (two passes) " + key, "%dx%d" % (M, K),
               4 * M * K + M * K // 2 + M * K // 16 + 4 * G, M * K,
               lambda: bsq.nv_quantize_nvfp4_per_group(w, off, *g_out, stream=stream))
        y = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
        report(4, "nvfp4 per-expert-scale dequant " + key, "%dx%d" % (M, K),
               2 * M * K + M * K // 2 + M * K // 16 + 4 * G, M * K,
               lambda: bsq.nv_dequantize_per_group(g_out[0], g_out[1], g_out[2], off, y, stream=stream))
        # the same export with 16x16 tiles (two-dimensional block scaling)
        t_out = (g_out[0], torch.empty(M // 16, K // 16, dtype=torch.uint8, device=dev), g_out[2], g_out[3])
        report(4, "nvfp4 16x16-tile quant (two passes) " + key, "%dx%d" % (M, K),
               4 * M * K + M * K // 2 + M * K // 256 + 4 * G, M * K,
               lambda: bsq.nv_quantize_nvfp4_2d(w, off, *t_out, stream=stream))
        report(4, "nvfp4 16x16-tile dequant " + key, "%dx%d" % (M, K),
               2 * M * K + M * K // 2 + M * K // 256 + 4 * G, M * K,
               lambda: bsq.nv_dequantize_2d(t_out[0], t_out[1], t_out[2], off, y, stream=stream))
        torch.cuda.synchronize()
        del w, g_out, t_out, y
    del c4
    c5 = workloads.config5()
    a, w = bf(c5["a"]), bf(c5["w"])
    run(5, "activations", a, "mx_both")
    run(5, "weights", w, "mx_both")
    x = a.index_select(0, torch.from_numpy(c5["token_idx"]).to(dev))
    off = torch.from_numpy(c5["offsets"]).to(dev)
    run(5, "routed rows", x, "nv", off)
    K = x.shape[1]
    # the same routed rows produced from the 65536 tokens without gathering them: each token
    # quantized once and written to its 8 routed rows (reads A once instead of X)
    T = a.shape[0]
    dst = torch.from_numpy(workloads.scatter_rows(c5["token_idx"], T, 8)).to(dev)
    s_out = (torch.empty(x.shape[0], K // 2, dtype=torch.uint8, device=dev), torch.empty(x.shape[0], K // 16, dtype=torch.uint8, device=dev),
             torch.empty(x.shape[0], dtype=torch.float32, device=dev), torch.zeros(1, dtype=torch.int32, device=dev))
    report(5, "nvfp4 quantize-then-scatter routed rows (from 65536 tokens)", "%dx%d" % tuple(x.shape),
           2 * T * K + x.shape[0] * (K // 2 + K // 16 + 4) + 8 * dst.numel(), x.numel(),
           lambda: bsq.nv_quantize_nvfp4_per_token_scatter(a, dst, x.shape[0], *s_out, stream=stream))
    del s_out
    # the same routed rows as the MoE weight-gradient operand: MXFP8 with 32x1 blocks
    # confined to each expert's rows (partial last blocks), rowwise copy fused or not
    M, K = x.shape
    nb = int(((np.diff(c5["offsets"]) + 31) // 32).sum())
    s_ld = bsq.mx_group_scale_entries(M, off.numel() - 1)
    u8 = torch.uint8
    g_out = (torch.empty(M, K, dtype=u8, device=dev), torch.empty(M, K // 32, dtype=u8, device=dev),
             torch.empty(K, M, dtype=u8, device=dev), torch.empty(K, s_ld, dtype=u8, device=dev),
             torch.zeros(1, dtype=torch.int32, device=dev))
    col_bytes = 2 * M * K + M * K + K * nb
    report(5, "mxfp8 grouped dual quant routed rows", "%dx%d" % (M, K), col_bytes + M * K + M * K // 32, M * K,
           lambda: bsq.mx_quantize_mxfp8_grouped(x, off, "both", s_ld, *g_out, stream=stream))
    report(5, "mxfp8 grouped columnwise quant routed rows", "%dx%d" % (M, K), col_bytes, M * K,
           lambda: bsq.mx_quantize_mxfp8_grouped(x, off, "colwise", s_ld, None, None, *g_out[2:], stream=stream))
    torch.cuda.synchronize()


def _oracle_step_sample(oracle, a_np, w_np, tok, frac, reps):
    """Time the CPU oracle (as it stands, OpenMP over rows) on 1/frac of the step's rows,
    reps times over: the first M/frac rows of A (both copies), the first rows of W, the first
    R/frac routed rows, and the dequantization of all of those outputs."""
    MA = (a_np.shape[0] // frac) // 32 * 32
    MW = max(32, (w_np.shape[0] // frac) // 32 * 32)
    RX = tok.size // frac
    a_s = np.ascontiguousarray(a_np[:MA])
    w_s = np.ascontiguousarray(w_np[:MW])
    x_s = a_np[tok[:RX]]
    t0 = time.perf_counter()
    for _ in range(reps):
        for m in (a_s, w_s):
            qr, sr = oracle.mx_quantize_rowwise(m)
            qc, sc = oracle.mx_quantize_colwise(m)
            oracle.mx_dequantize(qr, sr)
            oracle.mx_dequantize(qc, sc)
        q, sb, st = oracle.nv_quantize_per_token(x_s)
        oracle.nv_dequantize(q, sb, st)
    dt = time.perf_counter() - t0
    KA, KW, KX = a_s.shape[1], w_s.shape[1], x_s.shape[1]
    b = reps * (mx_both_bytes(MA, KA) + mx_both_bytes(MW, KW) + 2 * nv_bytes(RX, KX)
                + 2 * mx_dq_bytes(MA, KA) + 2 * mx_dq_bytes(MW, KW))
    sample = ("%d x 1/%d of the step: A[:%d] and W[:%d] MXFP8 dual + dequant of both copies, "
              "%d routed rows NVFP4 + dequant" % (reps, frac, MA, MW, RX))
    return round(b / dt / 1e9, 3), round(dt, 2), sample


def cpu_baseline(a_np, w_np, tok, frac, reps):
    """The CPU oracle on a bounded sample of the step, with all host threads, and once more
    on a 32x smaller sample with one thread."""
    import oracle

    oracle.lib()
    cores = oracle.max_threads()
    gbs, secs, sample = _oracle_step_sample(oracle, a_np, w_np, tok, frac, reps)
    oracle.set_threads(1)
    try:
        gbs1, secs1, sample1 = _oracle_step_sample(oracle, a_np, w_np, tok, frac * 32, 1)
    finally:
        oracle.set_threads(cores)
    return {"value": gbs, "unit": "GB/s", "cores": cores, "kind": "oracle", "seconds": secs,
            "sample": sample,
            "single_thread": {"value": gbs1, "unit": "GB/s", "cores": 1, "seconds": secs1,
                              "sample": sample1}}


if __name__ == "__main__":
    main()
