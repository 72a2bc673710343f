#!/usr/bin/env python3
"""Benchmark of the rotated-and-centred W4A4 quantised linear on one MI355X.

One step = one hq_quant_linear call (activation kernel + integer-exact GEMM
with the dequant epilogue; E2M3 / FP6 MFMA for 4-bit codes, the same layer on
the int8 MFMA engine is reported alongside) over one synthetic batch already
resident in HBM. Inputs
rotate through enough distinct X/Y buffers (> 512 MB) that a step's
activations are not served from the 256 MB Infinity Cache left over from the
previous visit. Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dit_fc1]
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Hadamard-quantized linear tokens/s + effective TOPS (% int8 MFMA/HBM roofline)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA (5.0 POP/s)
FP6_PEAK_TOPS = 10100.0        # MI355X dense fp6 / fp4 MFMA (10.1 PFLOP/s)
# Non-packed fp32 VALU lane operations per second: 256 CUs x 4 SIMDs x 16
# lanes x 2.4 GHz (a wave64 instruction issues over 4 cycles); the 157.3
# TFLOP/s vector figure counts packed fp32 fma, which this build does not emit.
VALU_F32_LANE_OPS = 256 * 4 * 16 * 2.4e9


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dit_fc1")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="measure the headline workload only, on both engines (no group-wise, "
                         "weight-only Hadamard or centring objects), e.g. for clean profiles")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--write-traffic", metavar="DIR",
                    help="host only: turn the FETCH_SIZE / WRITE_SIZE counter runs in DIR "
                         "(rocprofv3 -o fetch / -o write, csv) into the committed traffic record "
                         "of the dit_fc1 GEMM, then exit")
    return ap.parse_args()


def cpu_baseline(w, x, weight, bias, sigma, l1, l2, target_s):
    """Time the CPU oracle's online half (transform, centre, quantise, integer GEMM,
    dequantise) on a bounded prefix of the workload's tokens; weight prep excluded."""
    from oracle import hq_oracle as O
    import threadpoolctl
    sig = np.ones(w.d_in) if sigma is None else sigma.astype(np.float64)
    prep = O.prepare_weights(weight, sig, w.block, w.w_bits)
    rows = min(w.T, 256)
    t0 = time.perf_counter()
    O.quant_linear(x[:rows], prep, bias, sig, block=w.block, a_bits=w.a_bits,
                   center=int(w.center), l1=l1, l2=l2, out_dtype=w.out_dtype)
    dt = time.perf_counter() - t0
    if dt < target_s and rows < w.T:
        rows = int(min(w.T, max(rows, rows * target_s / max(dt, 1e-3))))
        t0 = time.perf_counter()
        O.quant_linear(x[:rows], prep, bias, sig, block=w.block, a_bits=w.a_bits,
                       center=int(w.center), l1=l1, l2=l2, out_dtype=w.out_dtype)
        dt = time.perf_counter() - t0
    info = threadpoolctl.threadpool_info()
    cores = max([i.get("num_threads", 1) for i in info] + [1])
    return {"value": rows / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {rows} of {w.T} tokens of {w.name}, float64 NumPy oracle "
                      f"(online half, prepared weights reused), {dt:.2f} s"}


def measure(hq, torch, desc, w, Xs, Ys, S, W, B, L1, L2, steps, warmup, dev):
    """Times `steps` quant_linear calls after `warmup`, then each of the two
    kernels alone (stage entry points, captured back to back in a HIP graph
    so the per-kernel time carries no host launch gaps)."""
    nbuf = len(Xs)
    tdt = Xs[0].dtype
    prep = hq.prepare(desc, W, B, S, L1, L2)
    ws = torch.empty(hq.workspace_bytes(desc, w.T), dtype=torch.uint8, device=dev)
    codes = torch.empty(hq.code_bytes(desc, w.T), dtype=torch.uint8, device=dev)
    s_x = torch.empty(desc.sx_shape(w.T), dtype=torch.float32, device=dev)
    mu = torch.empty(w.T, dtype=torch.float32, device=dev)
    U = torch.empty(w.T, w.rank, dtype=torch.float32, device=dev) if w.rank else None

    def step(i):
        hq.quant_linear(desc, prep, Xs[i % nbuf], out=Ys[i % nbuf], workspace=ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(steps):
        step(warmup + i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / steps

    # Per-kernel durations on the stream the kernels run on.
    n = min(steps, 20)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g1, g2 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        hq.act_quantize(desc, prep, Xs[0], out=(codes, s_x, mu, U))      # warm
        hq.gemm_dequant(desc, prep, codes, s_x, mu, U, out=Ys[0])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g1):
        for i in range(n):
            hq.act_quantize(desc, prep, Xs[i % nbuf], out=(codes, s_x, mu, U))
    with torch.cuda.graph(g2):
        for i in range(n):
            hq.gemm_dequant(desc, prep, codes, s_x, mu, U, out=Ys[i % nbuf])
    times = []
    for g in (g1, g2):
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / n)
    del g1, g2
    return {"ms": ms, "wall": wall, "k1": times[0], "k2": times[1], "prep": prep}


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary of this kernel and
    workload (profiles/<kernel>_<workload>_traffic.json), or None when there is
    none or the kernel sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel.replace('_dequant', '')}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec["sources_sha256"] or rec["kernel"] != kernel:
        return None
    return int(round(rec["traffic_bytes_per_launch"]))


TRAFFIC_SOURCES = ["hadamard_rotated_bit_amd/csrc/hq_gemm6_kernel.h",
                   "hadamard_rotated_bit_amd/csrc/hq_gemm_kernel.h",
                   "hadamard_rotated_bit_amd/csrc/hq_gemm6.hip",
                   "hadamard_rotated_bit_amd/csrc/hq_device.h",
                   "hadamard_rotated_bit_amd/csrc/hq_gemm_types.h"]
COPY_BYTES = 18874368   # one clone of dit_fc1's X (8192 x 1152 bf16): the plain copy kernel


def write_traffic(d):
    """Per-dispatch FETCH_SIZE and WRITE_SIZE (KiB) of the FP6 GEMM from two
    counter runs of this benchmark, each scaled by what the counter reads for
    the run's plain copy kernel of known size, into
    profiles/gemm_f6_dit_fc1_traffic.json with the hash of the GEMM sources."""
    import csv
    import hashlib
    from collections import defaultdict

    def per_kernel(f, counter):
        acc = defaultdict(list)
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return acc

    def pick(acc, key):
        v = [x for k in acc if key in k for x in acc[k]]
        if not v:
            raise SystemExit(f"no dispatch of {key} in the counter files")
        return sum(v) / len(v), len(v)

    fe = per_kernel(os.path.join(d, "fetch_counter_collection.csv"), "FETCH_SIZE")
    wr = per_kernel(os.path.join(d, "write_counter_collection.csv"), "WRITE_SIZE")
    cf, _ = pick(fe, "__amd_rocclr_copyBuffer")
    cw, _ = pick(wr, "__amd_rocclr_copyBuffer")
    fs, ws = COPY_BYTES / 1024 / cf, COPY_BYTES / 1024 / cw
    print(f"copy kernel: FETCH_SIZE {cf:.1f} KiB, WRITE_SIZE {cw:.1f} KiB -> scales {fs:.4f}, {ws:.4f}")
    for key in ["gemm_f6_persist", "gemm_i8_kernel", "row_fast_kernel"]:
        f, n = pick(fe, key)
        w, n2 = pick(wr, key)
        print(f"| `{key}` | {f:.1f} | {w:.1f} | {f * fs * 1024 / 1e6:.1f} MB | "
              f"{w * ws * 1024 / 1e6:.1f} MB | {(f * fs + w * ws) * 1024 / 1e6:.1f} MB | {n}, {n2} dispatches")
    f, _ = pick(fe, "gemm_f6_persist")
    w, _ = pick(wr, "gemm_f6_persist")
    h = hashlib.sha256()
    for src in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, src), "rb") as fh:
            h.update(fh.read())
    rec = {"kernel": "gemm_f6_dequant", "workload": "dit_fc1", "sources": TRAFFIC_SOURCES,
           "sources_sha256": h.hexdigest(), "fetch_kib_per_dispatch": f,
           "write_kib_per_dispatch": w,
           "copy_kernel": {"bytes": COPY_BYTES, "fetch_kib": cf, "write_kib": cw,
                           "fetch_scale": fs, "write_scale": ws},
           "traffic_bytes_per_launch": (f * fs + w * ws) * 1024}
    with open(os.path.join(ROOT, "profiles", "gemm_f6_dit_fc1_traffic.json"), "w") as fh:
        json.dump(rec, fh, indent=1)
    print(f"traffic per launch: {rec['traffic_bytes_per_launch'] / 1e6:.1f} MB")


def kernel_report(hq, desc, w, r):
    in_b = 2 if w.dtype == "bf16" else 4
    fp6 = hq.code_format(desc) == hq.HQ_CODES_E2M3
    # read X, write codes, s_x, mu, U
    k1_bytes = w.T * (w.d_in * in_b + 8 + 4 * w.rank) + hq.code_bytes(desc, w.T)
    k2_ops = 2.0 * w.T * w.d_in * w.d_out                          # code multiply-adds x 2
    peak = FP6_PEAK_TOPS if fp6 else INT8_PEAK_TOPS
    k1_gbs = k1_bytes / (r["k1"] * 1e-3) / 1e9
    k2_tops = k2_ops / (r["k2"] * 1e-3) / 1e12
    return fp6, peak, k1_gbs, k2_tops, k2_ops


def centring_modes(hq, torch, WL, steps, warmup, dev):
    """square4k (channels with different means) under per-token and per-channel
    centring: time per quant_linear call and the output SQNR against the
    float32 layer X W + b (HaTQ Sec. IV-A Eq. (10))."""
    w = WL.WORKLOADS["square4k"]
    x = WL.gen_x(w)
    X0 = torch.from_numpy(x).to(dev).to(torch.bfloat16)
    W = torch.from_numpy(WL.gen_weight(w)).to(dev).to(torch.bfloat16)
    B = torch.from_numpy(WL.gen_bias(w)).to(dev)
    nbuf = max(2, math.ceil(512e6 / (X0.numel() * 2)))
    Xs = [X0] + [X0.clone() for _ in range(nbuf - 1)]
    Y = torch.empty(w.T, w.d_out, dtype=torch.bfloat16, device=dev)
    ref = torch.addmm(B, X0.float(), W.float().t())
    out = {"workload": "square4k", "tokens": w.T, "d_in": w.d_in, "d_out": w.d_out,
           "block": w.block, "bits": "W4A4", "io_dtype": "bf16"}
    for mode, key in ((hq.HQ_CENTER_TOKEN, "per_token"), (hq.HQ_CENTER_CHANNEL, "per_channel")):
        desc = hq.Desc(w.d_in, w.d_out, w.block, w.a_bits, w.w_bits, mode, False, 0,
                       hq.BF16, hq.BF16, hq.BF16)
        prep = hq.prepare(desc, W, B)
        ws = torch.empty(hq.workspace_bytes(desc, w.T), dtype=torch.uint8, device=dev)
        for i in range(warmup):
            hq.quant_linear(desc, prep, Xs[i % nbuf], out=Y, workspace=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            hq.quant_linear(desc, prep, Xs[(warmup + i) % nbuf], out=Y, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        hq.quant_linear(desc, prep, X0, out=Y, workspace=ws)
        err = (Y.float() - ref).pow(2).sum().item()
        sqnr = 10.0 * math.log10(ref.pow(2).sum().item() / max(err, 1e-300))
        out[key] = {"value": round(w.T / (ms * 1e-3), 1), "unit": "tokens/s",
                    "ms_per_step": round(ms, 5), "sqnr_db": round(sqnr, 2)}
    return out


def group_wise(hq, torch, WL, steps, warmup, dev):
    """flux_g64 (group-wise scales, 64-point blocks, rank 32): time per call and
    per kernel, and the output SQNR against the float32 layer
    X W + b + (X L1) L2 with group-wise and with per-row scales on the same
    rotation. The group GEMM rescales every 64-channel partial product on the
    VALU (one multiply and one fma per output element and group); its floor is
    that work at the chip's non-packed fp32 rate."""
    w = WL.WORKLOADS["flux_g64"]
    x = WL.gen_x(w)
    l1, l2 = WL.gen_lowrank(w)
    X0 = torch.from_numpy(x).to(dev).to(torch.bfloat16)
    W = torch.from_numpy(WL.gen_weight(w)).to(dev).to(torch.bfloat16)
    B = torch.from_numpy(WL.gen_bias(w)).to(dev)
    L1 = torch.from_numpy(l1).to(dev).to(torch.bfloat16)
    L2 = torch.from_numpy(l2).to(dev).to(torch.bfloat16)
    nbuf = max(2, math.ceil(512e6 / (X0.numel() * 2)))
    Xs = [X0] + [X0.clone() for _ in range(nbuf - 1)]
    Ys = [torch.empty(w.T, w.d_out, dtype=torch.bfloat16, device=dev) for _ in range(nbuf)]
    desc = hq.Desc(w.d_in, w.d_out, w.block, w.a_bits, w.w_bits, int(w.center), False, w.rank,
                   hq.BF16, hq.BF16, hq.BF16, group=w.group)
    r = measure(hq, torch, desc, w, Xs, Ys, None, W, B, L1, L2, steps, warmup, dev)
    del Xs, Ys
    ops = 2.0 * w.T * w.d_in * w.d_out
    valu_lane_ops = 2.0 * w.T * w.d_out * (w.d_in // w.group)
    valu_floor_ms = valu_lane_ops / VALU_F32_LANE_OPS * 1e3
    ref = torch.addmm(B, X0.float(), W.float().t()) + (X0.float() @ L1.float()) @ L2.float()
    sq = {}
    for key, g in (("group64", w.group), ("per_row", 0)):
        d = dataclasses.replace(desc, group=g)
        Y = hq.quant_linear(d, r["prep"] if g else hq.prepare(d, W, B, None, L1, L2), X0)
        err = (Y.float() - ref).pow(2).sum().item()
        sq[key] = round(10.0 * math.log10(ref.pow(2).sum().item() / max(err, 1e-300)), 2)
        del Y
    return {"workload": w.name, "tokens": w.T, "d_in": w.d_in, "d_out": w.d_out,
            "block": w.block, "group": w.group, "rank": w.rank, "bits": "W4A4",
            "io_dtype": "bf16", "value": round(w.T / (r["ms"] * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(r["ms"], 5), "row_transform_ms": round(r["k1"], 5),
            "gemm_ms": round(r["k2"], 5), "gemm_TOPS": round(ops / (r["k2"] * 1e-3) / 1e12, 2),
            "gemm_mfma_frac": round(ops / (r["k2"] * 1e-3) / 1e12 / FP6_PEAK_TOPS, 4),
            "gemm_valu_floor_ms": round(valu_floor_ms, 5),
            "gemm_valu_frac": round(valu_floor_ms / r["k2"], 4),
            "sqnr_db": sq}


def integer_layer(hq, torch, WL, steps, warmup, dev, side):
    """lic_wh as an integer-only layer with integer requantisation (int8
    codes in, int8 codes out): the weight-only Hadamard layer (H_256 on the
    output channels, output in the original basis) or the double-Hadamard
    layer (input in the H_256 basis of the previous DH layer, output moved to
    the next one's H_256 basis). Time per call (int8 GEMM into int32, then the
    requantisation) and the output SQNR of the int8 codes against the float32
    layer in the same basis. The input codes are the workload's X (rotated for
    DH) on a per-tensor grid (synthetic input)."""
    w = WL.WORKLOADS["lic_wh"]
    X = torch.from_numpy(WL.gen_x(w)).to(dev)
    W = torch.from_numpy(WL.gen_weight(w)).to(dev)
    B = torch.from_numpy(WL.gen_bias(w)).to(dev)
    ref = torch.addmm(B, X, W.t())
    wh = side == hq.HQ_INT_WH
    if not wh:
        # orthonormal Sylvester H_256: the DH input and output bases
        H = torch.ones(1, 1, dtype=torch.float64)
        while H.shape[0] < w.block:
            H = torch.cat([torch.cat([H, H], 1), torch.cat([H, -H], 1)], 0)
        H = (H / math.sqrt(w.block)).to(dev)
        def rot(a):
            return (a.double().reshape(a.shape[0], -1, w.block) @ H).reshape(a.shape).float()
        X, ref = rot(X), rot(ref)
    s_x = float(X.abs().max().item() / 127.0)
    s_y = float(ref.abs().max().item() / 127.0)
    X0 = torch.clamp(torch.round(X / s_x), -127, 127).to(torch.int8)
    desc = hq.IntDesc(w.d_in, w.d_out, w.block, hq.F32, side, 1 if wh else w.block)
    prep = hq.int_prepare(desc, W, B, s_x, s_y)
    nbuf = max(2, math.ceil(512e6 / X0.numel()))
    Xs = [X0] + [X0.clone() for _ in range(nbuf - 1)]
    Ys = [torch.empty(w.T, w.d_out, dtype=torch.int8, device=dev) for _ in range(nbuf)]
    ws = torch.empty(hq.int_workspace_bytes(desc, w.T), dtype=torch.uint8, device=dev)
    for i in range(warmup):
        hq.int_linear(desc, prep, Xs[i % nbuf], out=Ys[i % nbuf], workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        hq.int_linear(desc, prep, Xs[(warmup + i) % nbuf], out=Ys[(warmup + i) % nbuf],
                      workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    y = Ys[(warmup + steps - 1) % nbuf].float() * s_y
    sq = 10.0 * math.log10(ref.pow(2).sum().item() / max((y - ref).pow(2).sum().item(), 1e-300))
    del Xs, Ys
    # bytes that must move: int8 codes in and out, weight codes, constants
    algo = w.T * (w.d_in + w.d_out) + w.d_out * (w.d_in + 12)
    return {"workload": w.name, "layer": "WH" if wh else "DH-to-DH", "tokens": w.T,
            "d_in": w.d_in, "d_out": w.d_out, "block": w.block, "bits": "W8A8 int8 -> int8",
            "value": round(w.T / (ms * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(ms, 5), "algorithmic_GBs": round(algo / (ms * 1e-3) / 1e9, 1),
            "sqnr_db": round(sq, 2)}


def main():
    args = parse()
    if args.write_traffic:
        write_traffic(args.write_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): this build runs on a "
              "single GPU; across GPUs the layer would shard by tokens with no communication",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import hadamard_rotated_bit_amd as hq
    from hadamard_rotated_bit_amd import workloads as WL

    w = WL.WORKLOADS[args.workload]
    dt = hq.BF16 if w.dtype == "bf16" else hq.F32
    desc = hq.Desc(w.d_in, w.d_out, w.block, w.a_bits, w.w_bits, int(w.center),
                   w.alpha is not None, w.rank, dt, dt, dt)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")

    x = WL.gen_x(w)
    weight, bias = WL.gen_weight(w), WL.gen_bias(w)
    l1, l2 = WL.gen_lowrank(w)
    X0 = torch.from_numpy(x).to(dev).to(tdt)
    W = torch.from_numpy(weight).to(dev).to(tdt)
    B = torch.from_numpy(bias).to(dev)
    L1 = None if l1 is None else torch.from_numpy(l1).to(dev).to(tdt)
    L2 = None if l2 is None else torch.from_numpy(l2).to(dev).to(tdt)
    S = None
    if w.alpha is not None:          # offline calibration on the workload's own tokens
        S = hq.sigma(desc, hq.channel_absmax(desc, X0), W, w.alpha)

    xbytes = X0.numel() * X0.element_size()
    nbuf = max(2, math.ceil(512e6 / xbytes))
    Xs = [X0] + [X0.clone() for _ in range(nbuf - 1)]
    Ys = [torch.empty(w.T, w.d_out, dtype=tdt, device=dev) for _ in range(nbuf)]

    r = measure(hq, torch, desc, w, Xs, Ys, S, W, B, L1, L2, args.steps, args.warmup, dev)
    fp6, peak, k1_gbs, k2_tops, k2_ops = kernel_report(hq, desc, w, r)
    ms = r["ms"]
    tokens_s = w.T / (ms * 1e-3)
    eff_tops = k2_ops / (ms * 1e-3) / 1e12
    if r["k2"] >= r["k1"]:
        kname = "gemm_f6_dequant" if fp6 else "gemm_i8_dequant"
        roof = {"kernel": kname, "bound": "mfma",
                "achieved": round(k2_tops, 2), "peak": peak, "unit": "TFLOP/s",
                "ops": ("e2m3" if fp6 else "int8") + " multiply-add x2",
                "frac": round(k2_tops / peak, 4), "traffic": measured_traffic(kname, w.name),
                "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE)"}
    else:
        roof = {"kernel": "row_transform", "bound": "hbm", "achieved": round(k1_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(k1_gbs / HBM_PEAK_GBS, 4),
                "traffic": None}
    out = {
        "metric": METRIC, "value": round(tokens_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "e2m3" if fp6 else "int8",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.T, "d_in": w.d_in, "d_out": w.d_out,
                   "block": w.block, "bits": f"W{w.w_bits}A{w.a_bits}", "center": int(w.center),
                   "smooth_alpha": w.alpha, "rank": w.rank, "io_dtype": w.dtype,
                   "gemm": "e2m3 fp6 mfma" if fp6 else "int8 mfma"},
        "effective_tops": round(eff_tops, 2),
        "roofline": roof,
        "kernels": {
            "row_transform_ms": round(r["k1"], 5), "row_transform_GBs": round(k1_gbs, 1),
            "row_transform_hbm_frac": round(k1_gbs / HBM_PEAK_GBS, 4),
            "gemm_ms": round(r["k2"], 5), "gemm_TOPS": round(k2_tops, 2),
            "gemm_mfma_frac": round(k2_tops / peak, 4),
        },
        "wall_s_timed": round(r["wall"], 4),
    }
    if fp6:
        # the same layer on the int8 engine (int4 codes in int8 lanes, int32
        # accumulation): identical accumulators, measured against the int8 peak
        d8 = dataclasses.replace(desc, gemm=hq.HQ_GEMM_I8)
        r8 = measure(hq, torch, d8, w, Xs, Ys, S, W, B, L1, L2, args.steps, args.warmup, dev)
        _, p8, g8, t8, _ = kernel_report(hq, d8, w, r8)
        out["int8_engine"] = {
            "value": round(w.T / (r8["ms"] * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(r8["ms"], 5), "row_transform_ms": round(r8["k1"], 5),
            "row_transform_GBs": round(g8, 1), "gemm_ms": round(r8["k2"], 5),
            "gemm_TOPS": round(t8, 2), "gemm_mfma_frac": round(t8 / p8, 4), "peak": p8}
    del Xs, Ys
    if not args.no_extras:
        out["group_wise"] = group_wise(hq, torch, WL, min(args.steps, 20), min(args.warmup, 5),
                                       dev)
        out["integer_layers"] = [
            integer_layer(hq, torch, WL, min(args.steps, 20), min(args.warmup, 5), dev, side)
            for side in (hq.HQ_INT_WH, hq.HQ_INT_DH)]
        out["centring_modes"] = centring_modes(hq, torch, WL, min(args.steps, 20),
                                               min(args.warmup, 5), dev)
    if not args.no_cpu_baseline:
        sig = None if S is None else S.cpu().numpy()
        out["cpu_baseline"] = cpu_baseline(w, x, weight, bias, sig, l1, l2, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
