#!/usr/bin/env python3
"""Benchmark of the rotated-and-centred low-bit linear layer on one MI355X.

One step = one hq_quant_linear call (the activation kernel, then the
integer-exact GEMM with the dequant epilogue; E2M3 / FP6 MFMA for 4-bit
codes, int8 MFMA for 8-bit codes) over one synthetic batch already resident
in HBM. The headline is the FLUX-scale joint-attention projection (4608 x
3072 -> 12288 bf16, three 1024-point blocks, per-token centring, W4A4 with
the rank-32 branch); the other workloads (the toy layer, the DiT MLP fc1,
the square 4096 projection with centring on and off, the learned-image-coding
double-Hadamard W8A8 layer) get one object each in the same JSON line.

Inputs rotate through enough distinct X / Y buffers (> 512 MB) that a step's
activations are not served from the 256 MB Infinity Cache left over from the
previous visit. Each workload first makes untimed calls for SPIN_UP_S seconds
(the GPU leaves the idle clock state host-side data generation leaves it in),
then W warmup steps, then the K timed steps. Per-kernel times come from HIP
events recorded after each stage inside a run of steps (the two stage entry
points called in turn, as quant_linear issues them, on the stream the events
are recorded on; median over the steps). The same stages launched back to
back in a replayed HIP graph (median of five replays) are reported beside
them as `graph_ms`: a run of GEMMs with no activation stage between them
holds the chip at a higher power and a lower clock than the step does. Where
the two in-step stage times add up to more than 1.06x the step (launch-bound
layers, whose GPU then waits for the host between the stages), the graph
times take their place (`stage_timing`: "graph" instead of "steps").
Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload flux_proj]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
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
SPIN_UP_S = 0.2                # untimed calls before each workload's timings (s)
GRAPH_REPS = 5                 # timed replays per stage graph (median taken)
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA (5.0 POP/s)
FP6_PEAK_TOPS = 10100.0        # MI355X dense fp6 / fp4 MFMA (10.1 PFLOP/s)
# Non-packed fp32 VALU lane operations per second: 256 CUs x 4 SIMDs x 16
# lanes x 2.4 GHz (a wave64 instruction issues over 4 cycles); the 157.3
# TFLOP/s vector figure counts packed fp32 fma, which this build does not emit.
VALU_F32_LANE_OPS = 256 * 4 * 16 * 2.4e9
CONFIG_ORDER = ["tiny", "dit_fc1", "square4k", "lic_dh", "flux_proj"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="flux_proj")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="measure the headline workload only (both engines), e.g. for clean "
                         "profiles: no other configs, group-wise, integer-layer or centring objects")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--write-traffic", metavar="DIR",
                    help="host only: turn the FETCH_SIZE / WRITE_SIZE counter runs in DIR "
                         "(rocprofv3 -o fetch / -o write, csv) of the --workload run into the "
                         "committed traffic record of its GEMM, then exit")
    return ap.parse_args()


def host_cores() -> int:
    return len(os.sched_getaffinity(0))


def sha256_arrays(**arrays) -> dict:
    out = {}
    for k, a in arrays.items():
        if a is not None:
            out[k] = hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
    return out


def cpu_baseline(w, x, weight, bias, sigma, l1, l2, Y_gpu, target_s):
    """The C++ CPU oracle's online half (transform, centre, quantise, integer
    GEMM, dequantise; weight preparation done once beforehand and not timed)
    on a bounded prefix of the workload's tokens, std::thread over tokens on
    every host core. The same rows of the GPU output are compared with the
    oracle's (relative Frobenius error) as the run's parity statistic."""
    from oracle import cpp as C
    cores = host_cores()
    sig = np.ones(w.d_in) if sigma is None else sigma.astype(np.float64)
    t0 = time.perf_counter()
    prep = C.prepare_weights(weight, sig, w.block, w.w_bits, threads=cores)
    prep_s = time.perf_counter() - t0

    def run(n):
        t0 = time.perf_counter()
        r = C.quant_linear(x[:n], prep, bias, sig, block=w.block, a_bits=w.a_bits,
                           center=int(w.center), l1=l1, l2=l2, out_dtype=w.out_dtype,
                           want_acc=False, threads=cores)
        return r, time.perf_counter() - t0

    rows = min(w.T, 256)
    r, dt = run(rows)
    if dt < target_s and rows < w.T:
        rows = int(min(w.T, max(rows, rows * target_s / max(dt, 1e-3))))
        r, dt = run(rows)
    y = Y_gpu[:rows].float().cpu().numpy().astype(np.float64)
    ref = r["y_out"]
    err = float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))
    # one thread on the two small workloads (the tiny layer and the
    # learned-image-coding 1x1 convolution), a prefix of up to 2048 tokens
    from oracle import hq_oracle as O
    from hadamard_rotated_bit_amd import workloads as WL
    single = {}
    for name in ("tiny", "lic_dh"):
        wc = WL.WORKLOADS[name]
        xc, wt, bc = WL.gen_x(wc), WL.gen_weight(wc), WL.gen_bias(wc)
        sg = (O.smoothing_scales(xc, wt, wc.alpha) if wc.alpha is not None
              else np.ones(wc.d_in))
        pc = C.prepare_weights(wt, sg, wc.block, wc.w_bits, threads=1)
        n = min(wc.T, 2048)
        t0 = time.perf_counter()
        C.quant_linear(xc[:n], pc, bc, sg, block=wc.block, a_bits=wc.a_bits,
                       center=int(wc.center), out_dtype=wc.out_dtype, want_acc=False, threads=1)
        single[name] = {"value": n / (time.perf_counter() - t0), "unit": "tokens/s",
                        "cores": 1, "sample": f"first {n} of {wc.T} tokens"}
    return {"value": rows / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle-c++",
            "single_thread": single,
            "sample": f"first {rows} of {w.T} tokens of {w.name}, float64 C++17 oracle "
                      f"(online half, std::thread on {cores} host cores, prepared weights "
                      f"reused), {dt:.2f} s; weight preparation {prep_s:.2f} s, not timed",
            "parity_rel_fro_vs_gpu": err, "parity_rows": rows}


def spin_up(torch, fn, nbuf, seconds=SPIN_UP_S):
    """Untimed calls of fn for at least `seconds` of wall time, so that the
    GPU leaves its idle clock state (data generation on the host keeps it
    idle before each workload) before anything is timed."""
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        fn(i % nbuf)
        i += 1
    torch.cuda.synchronize()


def timed_steps(torch, fn, nbuf, steps, warmup):
    for i in range(warmup):
        fn(i % nbuf)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        fn((warmup + i) % nbuf)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, time.perf_counter() - t0


def step_percentiles(torch, fn, nbuf, steps, start):
    """p10 / p50 / p90 of `steps` individually event-timed calls fn(i) issued
    back to back (ms), after the bracketed run."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        fn((start + i) % nbuf)
        ev[i + 1].record()
    torch.cuda.synchronize()
    d = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    pick = lambda q: round(d[int(round(q * (len(d) - 1)))], 5)
    return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9)}


def staged_steps(torch, step, act, gemm, nbuf, steps, start, queued=10):
    """Per-stage times inside a run of steps: act(i) then gemm(i) for `steps`
    consecutive i, a HIP event recorded after each call on the stream both
    run on; the median over the steps of each stage's time (ms). `queued`
    plain steps go first, unsynchronised, so that the host is ahead of the
    GPU when the first event is recorded."""
    for i in range(queued):
        step((start + i) % nbuf)
    start += queued
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps + 1)]
    ev[0].record()
    for i in range(steps):
        act((start + i) % nbuf)
        ev[2 * i + 1].record()
        gemm((start + i) % nbuf)
        ev[2 * i + 2].record()
    torch.cuda.synchronize()
    k1 = sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps))
    k2 = sorted(ev[2 * i + 1].elapsed_time(ev[2 * i + 2]) for i in range(steps))
    return k1[steps // 2], k2[steps // 2]


def graph_time(torch, fn, n, reps=GRAPH_REPS):
    """Time of fn(i), i < n, captured back to back in one HIP graph and
    replayed on the current stream, timed with HIP events on that stream:
    the median over `reps` timed replays (after one untimed replay) of the
    replay time divided by n."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for k in range(reps):
        g.replay()
        ev[k + 1].record()
    torch.cuda.synchronize()
    del g
    t = sorted(ev[k].elapsed_time(ev[k + 1]) for k in range(reps))
    return t[reps // 2] / n


class Layer:
    """One workload on the GPU: inputs, the prepared blob, rotating buffers."""

    def __init__(self, hq, torch, WL, w, dev, gemm=None, center=None):
        self.w = w
        dt = hq.BF16 if w.dtype == "bf16" else hq.F32
        self.tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.x = WL.gen_x(w)
        self.weight, self.bias = WL.gen_weight(w), WL.gen_bias(w)
        self.l1, self.l2 = WL.gen_lowrank(w)
        self.X0 = torch.from_numpy(self.x).to(dev).to(self.tdt)
        self.W = torch.from_numpy(self.weight).to(dev).to(self.tdt)
        self.B = torch.from_numpy(self.bias).to(dev)
        self.L1 = None if self.l1 is None else torch.from_numpy(self.l1).to(dev).to(self.tdt)
        self.L2 = None if self.l2 is None else torch.from_numpy(self.l2).to(dev).to(self.tdt)
        self.desc = hq.Desc(w.d_in, w.d_out, w.block, w.a_bits, w.w_bits,
                            int(w.center if center is None else center), w.alpha is not None,
                            w.rank, dt, dt, dt, hq.HQ_GEMM_AUTO if gemm is None else gemm)
        self.S = None
        if w.alpha is not None:   # offline calibration on the workload's own tokens
            self.S = hq.sigma(self.desc, hq.channel_absmax(self.desc, self.X0), self.W, w.alpha)
        xbytes = self.X0.numel() * self.X0.element_size()
        self.nbuf = max(2, math.ceil(512e6 / xbytes))
        self.Xs = [self.X0] + [self.X0.clone() for _ in range(self.nbuf - 1)]
        self.Ys = [torch.empty(w.T, w.d_out, dtype=self.tdt, device=dev)
                   for _ in range(self.nbuf)]
        self.dev = dev

    def sha(self):
        return sha256_arrays(x=self.x, weight=self.weight, bias=self.bias, l1=self.l1, l2=self.l2)

    def free(self):
        del self.Xs, self.Ys


def measure(hq, torch, L, desc, steps, warmup):
    """Times `steps` quant_linear calls after `warmup` (the step), then the
    two stages inside a run of steps and each stage alone as a replayed
    graph: the activation stage as quant_linear runs it (hq_act_quantize_ws)
    and the GEMM + epilogue (hq_gemm_dequant)."""
    w, dev = L.w, L.dev
    prep = hq.prepare(desc, L.W, L.B, L.S, L.L1, L.L2)
    ws = torch.empty(hq.workspace_bytes(desc, w.T), dtype=torch.uint8, device=dev)
    codes = torch.empty(hq.code_bytes(desc, w.T), dtype=torch.uint8, device=dev)
    s_x = torch.empty(desc.sx_shape(w.T), dtype=torch.float32, device=dev)
    mu = torch.empty(w.T, dtype=torch.float32, device=dev)
    U = torch.empty(w.T, w.rank, dtype=torch.float32, device=dev) if w.rank else None
    nbuf = L.nbuf

    def step(i):
        hq.quant_linear(desc, prep, L.Xs[i], out=L.Ys[i], workspace=ws)

    spin_up(torch, step, nbuf)
    ms, wall = timed_steps(torch, step, nbuf, steps, warmup)
    pct = step_percentiles(torch, step, nbuf, steps, warmup + steps)
    n = max(1, min(steps, 20))
    if int(desc.center) == hq.HQ_CENTER_CHANNEL:
        # per-channel centring: the statistics stage (column means and the
        # corrected bias) is timed with the activation stage
        mean, bias_eff = hq.channel_center(desc, prep, L.Xs[0], workspace=ws)

        def act(i):
            hq.channel_center_into(desc, prep, L.Xs[i % nbuf], mean, bias_eff, ws)
            hq.act_quantize(desc, prep, L.Xs[i % nbuf], out=(codes, s_x, mu, U), mean=mean,
                            workspace=ws)

        def gemm(i):
            hq.gemm_dequant(desc, prep, codes, s_x, bias_eff, U, out=L.Ys[i % nbuf])
    else:
        def act(i):
            hq.act_quantize(desc, prep, L.Xs[i % nbuf], out=(codes, s_x, mu, U), workspace=ws)

        def gemm(i):
            hq.gemm_dequant(desc, prep, codes, s_x, mu, U, out=L.Ys[i % nbuf])
    k1, k2 = staged_steps(torch, step, act, gemm, nbuf, max(steps, 20), warmup + 2 * steps)
    k1g, k2g = graph_time(torch, act, n), graph_time(torch, gemm, n)
    timing = "steps"
    if k1 + k2 > 1.06 * ms:
        # launch-bound layer: the events between the stages keep the GPU
        # waiting for the host, so the in-step split is not the kernels' time
        k1, k2, timing = k1g, k2g, "graph"
    return {"ms": ms, "wall": wall, "k1": k1, "k2": k2, "k1_graph": k1g, "k2_graph": k2g,
            "timing": timing, "prep": prep, "pct": pct}


def kernel_figures(hq, desc, w, r):
    """Algorithmic work of each kernel and the rates it reached.

    K1 (activation stage) bytes per call: read X, write the codes in the
    descriptor's format, s_x and mu (4 B per token each) and U (4 r B per
    token), read 1/sigma and (rank > 0) the two bf16 halves of L1 once; the
    4-bit minimum (0.5 B per code) is reported beside it. K2 (GEMM +
    epilogue) ops = 2 T d_in d_out code multiply-adds; bytes = both code
    matrices, the per-row and per-column vectors, U and L2 (rank > 0) and Y."""
    in_b = 2 if w.dtype == "bf16" else 4
    out_b = in_b
    fp6 = hq.code_format(desc) == hq.HQ_CODES_E2M3
    code_b = hq.code_bytes(desc, w.T)
    k1_bytes = (w.T * (w.d_in * in_b + 8 + 4 * w.rank) + code_b + 4 * w.d_in
                + 4 * w.rank * w.d_in)
    k1_min = w.T * (w.d_in * in_b + 8 + 4 * w.rank) + w.T * w.d_in * w.a_bits // 8
    k2_ops = 2.0 * w.T * w.d_in * w.d_out
    k2_bytes = (code_b + hq.code_bytes(desc, w.d_out) + 8 * w.T + 12 * w.d_out
                + 4 * w.rank * w.T + 4 * w.rank * w.d_out + out_b * w.T * w.d_out)
    peak = FP6_PEAK_TOPS if fp6 else INT8_PEAK_TOPS
    k1_gbs = k1_bytes / (r["k1"] * 1e-3) / 1e9
    k2_tops = k2_ops / (r["k2"] * 1e-3) / 1e12
    k2_gbs = k2_bytes / (r["k2"] * 1e-3) / 1e9
    return {
        "engine": "e2m3 fp6 mfma" if fp6 else "int8 mfma",
        "value": round(w.T / (r["ms"] * 1e-3), 1), "unit": "tokens/s",
        "ms_per_step": round(r["ms"], 5),
        "ms_per_step_percentiles": r["pct"],
        "stage_timing": r["timing"],
        "effective_TOPS_step": round(k2_ops / (r["ms"] * 1e-3) / 1e12, 2),
        "k1": {"ms": round(r["k1"], 5), "graph_ms": round(r["k1_graph"], 5),
               "bytes": int(k1_bytes), "GBs": round(k1_gbs, 1),
               "hbm_frac": round(k1_gbs / HBM_PEAK_GBS, 4),
               "bytes_4bit_min": int(k1_min),
               "hbm_frac_4bit_min": round(k1_min / (r["k1"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "k2": {"ms": round(r["k2"], 5), "graph_ms": round(r["k2_graph"], 5),
               "ops": k2_ops, "TOPS": round(k2_tops, 2),
               "peak_TOPS": peak, "mfma_frac": round(k2_tops / peak, 4),
               "bytes": int(k2_bytes), "GBs": round(k2_gbs, 1),
               "hbm_frac": round(k2_gbs / HBM_PEAK_GBS, 4)},
    }


def diagnostics(hq, torch, L, desc, prep):
    """Not gates: output SQNR (HaTQ Sec. IV-A Eq. (10)) of the method and of
    the same quantiser without any transform (sigma = 1, no rotation, no
    centring) against the unquantised layer in float32, and the excess
    kurtosis (Eq. (9)) of X and of X~ over all entries."""
    w = L.w
    X = L.X0
    ref = torch.addmm(L.B, X.float(), L.W.float().t())
    if L.L1 is not None:
        xs = X.float() if L.S is None else X.float() / L.S
        ref = ref + (xs @ L.L1.float()) @ L.L2.float()

    def sqnr(Y):
        e = (Y.float() - ref).pow(2).sum().item()
        return round(10.0 * math.log10(ref.pow(2).sum().item() / max(e, 1e-300)), 2)

    Y = hq.quant_linear(desc, prep, X)
    # the same quantiser on X W + b alone: no smoothing, no rotation, no
    # centring and no low-rank branch (its reference leaves the branch out)
    plain = dataclasses.replace(desc, block=1, smooth=False, center=hq.HQ_CENTER_NONE, rank=0)
    pp = hq.prepare(plain, L.W, L.B)
    Y0 = hq.quant_linear(plain, pp, X)
    ref0 = torch.addmm(L.B, X.float(), L.W.float().t())
    e0 = (Y0.float() - ref0).pow(2).sum().item()
    sq = {"method": sqnr(Y),
          "no_transform": round(10.0 * math.log10(ref0.pow(2).sum().item() / max(e0, 1e-300)), 2)}
    del pp, Y0, ref0

    def kurt(v):
        v = v.double().flatten()
        d = v - v.mean()
        return round((d.pow(4).mean() / d.pow(2).mean().pow(2) - 3.0).item(), 3)

    xt, _ = hq.act_transform(desc, prep, X)
    k = {"x": kurt(X.float()), "x_tilde": kurt(xt)}
    del xt
    return Y, sq, k


def config_object(hq, torch, WL, name, steps, warmup, dev, both_engines=True):
    """Every figure for one workload; returns (object, Layer, measurement)."""
    w = WL.WORKLOADS[name]
    L = Layer(hq, torch, WL, w, dev)
    r = measure(hq, torch, L, L.desc, steps, warmup)
    obj = {"workload": w.name, "tokens": w.T, "d_in": w.d_in, "d_out": w.d_out,
           "block": w.block, "bits": f"W{w.w_bits}A{w.a_bits}", "center": int(w.center),
           "smooth_alpha": w.alpha, "rank": w.rank, "io_dtype": w.dtype}
    obj.update(kernel_figures(hq, L.desc, w, r))
    Y, obj["sqnr_db"], obj["kurtosis"] = diagnostics(hq, torch, L, L.desc, r["prep"])
    obj["input_sha256"] = L.sha()
    if both_engines and hq.code_format(L.desc) == hq.HQ_CODES_E2M3:
        # the same layer on the int8 engine (int4 codes in int8 lanes, int32
        # accumulation): identical accumulators, measured against the int8 peak
        d8 = dataclasses.replace(L.desc, gemm=hq.HQ_GEMM_I8)
        r8 = measure(hq, torch, L, d8, steps, warmup)
        obj["int8_engine"] = kernel_figures(hq, d8, w, r8)
        del r8
    return obj, L, r, Y


def centring_off(hq, torch, L, r_on, steps, warmup):
    """The square projection run again with centring off (HadaNorm's centring
    is the difference), and the centring overhead per kernel and per step."""
    d0 = dataclasses.replace(L.desc, center=hq.HQ_CENTER_NONE)
    r0 = measure(hq, torch, L, d0, steps, warmup)
    obj = kernel_figures(hq, d0, L.w, r0)
    Y, obj["sqnr_db"], obj["kurtosis"] = diagnostics(hq, torch, L, d0, r0["prep"])
    del Y
    over = {"k1_ms": round(r_on["k1"] - r0["k1"], 5), "k2_ms": round(r_on["k2"] - r0["k2"], 5),
            "step_ms": round(r_on["ms"] - r0["ms"], 5)}
    return obj, over


def centring_modes(hq, torch, L, steps, warmup):
    """square4k under per-channel centring (mu one vector over channels, b~
    one corrected bias): time per call and output SQNR."""
    d2 = dataclasses.replace(L.desc, center=hq.HQ_CENTER_CHANNEL)
    r2 = measure(hq, torch, L, d2, steps, warmup)
    Y, sq, k = diagnostics(hq, torch, L, d2, r2["prep"])
    del Y
    return {"value": round(L.w.T / (r2["ms"] * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(r2["ms"], 5), "sqnr_db": sq}


def group_wise(hq, torch, WL, steps, warmup, dev):
    """flux_g64 (group-wise scales, 64-point blocks, rank 32): time per call and
    per kernel, and the output SQNR with group-wise and with per-row scales on
    the same rotation. The group GEMM rescales every 64-channel partial product
    on the VALU (one multiply and one fma per output element and group); its
    floor is that work at the chip's non-packed fp32 rate."""
    w = WL.WORKLOADS["flux_g64"]
    L = Layer(hq, torch, WL, w, dev)
    desc = dataclasses.replace(L.desc, group=w.group)
    r = measure(hq, torch, L, desc, steps, warmup)
    ops = 2.0 * w.T * w.d_in * w.d_out
    valu_floor_ms = 2.0 * w.T * w.d_out * (w.d_in // w.group) / VALU_F32_LANE_OPS * 1e3
    sq = {}
    _, sq["group64"], _ = diagnostics(hq, torch, L, desc, r["prep"])
    d0 = dataclasses.replace(desc, group=0)
    _, sq["per_row"], _ = diagnostics(hq, torch, L, d0, hq.prepare(d0, L.W, L.B, None, L.L1, L.L2))
    L.free()
    return {"workload": w.name, "tokens": w.T, "d_in": w.d_in, "d_out": w.d_out,
            "block": w.block, "group": w.group, "rank": w.rank, "bits": "W4A4",
            "io_dtype": "bf16", "value": round(w.T / (r["ms"] * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(r["ms"], 5), "row_transform_ms": round(r["k1"], 5),
            "gemm_ms": round(r["k2"], 5), "gemm_TOPS": round(ops / (r["k2"] * 1e-3) / 1e12, 2),
            "gemm_mfma_frac": round(ops / (r["k2"] * 1e-3) / 1e12 / FP6_PEAK_TOPS, 4),
            "gemm_valu_floor_ms": round(valu_floor_ms, 5),
            "gemm_valu_frac": round(valu_floor_ms / r["k2"], 4),
            "sqnr_db": {k: v["method"] for k, v in sq.items()}}


def integer_layer(hq, torch, WL, steps, warmup, dev, side, gelu=False):
    """lic_wh as an integer-only layer with integer requantisation (int8
    codes in, int8 codes out): the weight-only Hadamard layer (H_256 on the
    output channels, output in the original basis), the double-Hadamard
    layer (input in the H_256 basis of the previous DH layer, output moved to
    the next one's H_256 basis), or (gelu) a WH layer followed by GELU and
    handing over to a DH layer (H_out before the activation, the integer
    GELU table on its own int8 grids, the next layer's H_256 after it). Time
    per call and the output SQNR of the int8 codes against the float32 layer
    (and activation) in the same basis. The input codes are the workload's X
    (rotated for DH) on a per-tensor grid (synthetic input)."""
    w = WL.WORKLOADS["lic_wh"]
    X = torch.from_numpy(WL.gen_x(w)).to(dev)
    W = torch.from_numpy(WL.gen_weight(w)).to(dev)
    B = torch.from_numpy(WL.gen_bias(w)).to(dev)
    ref = torch.addmm(B, X, W.t())
    wh = side == hq.HQ_INT_WH
    # orthonormal Sylvester H_256: the DH input and output bases
    H = torch.ones(1, 1, dtype=torch.float64)
    while H.shape[0] < w.block:
        H = torch.cat([torch.cat([H, H], 1), torch.cat([H, -H], 1)], 0)
    H = (H / math.sqrt(w.block)).to(dev)

    def rot(a):
        return (a.double().reshape(a.shape[0], -1, w.block) @ H).reshape(a.shape).float()
    if not wh:
        X, ref = rot(X), rot(ref)
    s_z = s_u = 0.0
    if gelu:
        act = torch.nn.functional.gelu(ref.double())
        s_z = float(ref.abs().max().item() / 127.0)
        s_u = float(act.abs().max().item() / 127.0)
        ref = rot(act)
    s_x = float(X.abs().max().item() / 127.0)
    s_y = float(ref.abs().max().item() / 127.0)
    X0 = torch.clamp(torch.round(X / s_x), -127, 127).to(torch.int8)
    desc = hq.IntDesc(w.d_in, w.d_out, w.block, hq.F32, side, 1 if wh else w.block,
                      hq.HQ_INT_ACT_GELU if gelu else hq.HQ_INT_ACT_NONE, w.block if gelu else 1)
    prep = hq.int_prepare(desc, W, B, s_x, s_y, s_z, s_u)
    nbuf = max(2, math.ceil(512e6 / X0.numel()))
    Xs = [X0] + [X0.clone() for _ in range(nbuf - 1)]
    Ys = [torch.empty(w.T, w.d_out, dtype=torch.int8, device=dev) for _ in range(nbuf)]
    ws = torch.empty(hq.int_workspace_bytes(desc, w.T), dtype=torch.uint8, device=dev)
    spin_up(torch, lambda i: hq.int_linear(desc, prep, Xs[i], out=Ys[i], workspace=ws), nbuf)
    ms, _ = timed_steps(torch, lambda i: hq.int_linear(desc, prep, Xs[i], out=Ys[i], workspace=ws),
                        nbuf, steps, warmup)
    y = Ys[(warmup + steps - 1) % nbuf].float() * s_y
    sq = 10.0 * math.log10(ref.pow(2).sum().item() / max((y - ref).pow(2).sum().item(), 1e-300))
    del Xs, Ys
    # bytes that must move: int8 codes in and out, weight codes, constants
    algo = w.T * (w.d_in + w.d_out) + w.d_out * (w.d_in + 12)
    return {"workload": w.name,
            "layer": "WH-to-DH with GELU" if gelu else ("WH" if wh else "DH-to-DH"), "tokens": w.T,
            "d_in": w.d_in, "d_out": w.d_out, "block": w.block, "bits": "W8A8 int8 -> int8",
            "value": round(w.T / (ms * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(ms, 5), "algorithmic_GBs": round(algo / (ms * 1e-3) / 1e9, 1),
            "sqnr_db": round(sq, 2)}


# ---- traffic records (rocprofv3 FETCH_SIZE / WRITE_SIZE) -------------------

GEMM_SOURCES = ["hadamard_rotated_bit_amd/csrc/hq_gemm6_kernel.h",
                "hadamard_rotated_bit_amd/csrc/hq_gemm_kernel.h",
                "hadamard_rotated_bit_amd/csrc/hq_gemm6.hip",
                "hadamard_rotated_bit_amd/csrc/hq_gemm.hip",
                "hadamard_rotated_bit_amd/csrc/hq_device.h",
                "hadamard_rotated_bit_amd/csrc/hq_gemm_types.h"]


def sources_sha(srcs) -> str:
    h = hashlib.sha256()
    for src in srcs:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter record of this kernel
    and workload (profiles/<kernel>_<workload>_traffic.json), or None when
    there is none or the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel") != kernel or sources_sha(rec["sources"]) != rec["sources_sha256"]:
        return None
    return int(round(rec["traffic_bytes_per_launch"]))


def write_traffic(d, workload):
    """Per-dispatch FETCH_SIZE and WRITE_SIZE (KiB) of the GEMM from two counter
    runs of this benchmark on `workload`, each scaled by what the counter reads
    for the run's plain copy kernel of known size (a clone of X), into
    profiles/gemm_f6_dequant_<workload>_traffic.json with the hash of the GEMM sources."""
    import csv
    from collections import defaultdict
    from hadamard_rotated_bit_amd import workloads as WL
    w = WL.WORKLOADS[workload]
    copy_bytes = w.T * w.d_in * (2 if w.dtype == "bf16" else 4)

    def per_kernel(f, counter):
        # copy dispatches are told apart by grid size: the clones of X are the
        # largest; the runtime's other, small copies use the same kernel name
        acc, grids = defaultdict(list), defaultdict(set)
        rows = []
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    rows.append(r)
                    grids[r["Kernel_Name"]].add(int(r["Grid_Size"]))
        for r in rows:
            k = r["Kernel_Name"]
            if "copyBuffer" in k and int(r["Grid_Size"]) != max(grids[k]):
                continue
            acc[k].append(float(r["Counter_Value"]))
        return acc

    def pick(acc, key):
        # the instance with the most dispatches among those whose name holds
        # `key` (the timed kernel; the diagnostics launch other instances a
        # few times)
        names = [k for k in acc if key in k]
        if not names:
            raise SystemExit(f"no dispatch of {key} in the counter files")
        v = acc[max(names, key=lambda k: len(acc[k]))]
        return sum(v) / len(v), len(v)

    fe = per_kernel(os.path.join(d, "fetch_counter_collection.csv"), "FETCH_SIZE")
    wr = per_kernel(os.path.join(d, "write_counter_collection.csv"), "WRITE_SIZE")
    cf, _ = pick(fe, "__amd_rocclr_copyBuffer")
    cw, _ = pick(wr, "__amd_rocclr_copyBuffer")
    fs, ws = copy_bytes / 1024 / cf, copy_bytes / 1024 / cw
    print(f"copy kernel ({copy_bytes} bytes): FETCH_SIZE {cf:.1f} KiB, WRITE_SIZE {cw:.1f} KiB "
          f"-> scales {fs:.4f}, {ws:.4f}")
    names = sorted({k for k in fe if "copyBuffer" not in k})
    for key in names:
        f, n = pick(fe, key)
        wv, n2 = pick(wr, key)
        print(f"| `{key[:60]}` | {f:.1f} | {wv:.1f} | {f * fs * 1024 / 1e6:.1f} MB | "
              f"{wv * ws * 1024 / 1e6:.1f} MB | {(f * fs + wv * ws) * 1024 / 1e6:.1f} MB | "
              f"{n}, {n2} dispatches")
    f, _ = pick(fe, "gemm_f6_persist")
    wv, _ = pick(wr, "gemm_f6_persist")
    rec = {"kernel": "gemm_f6_dequant", "workload": workload, "sources": GEMM_SOURCES,
           "sources_sha256": sources_sha(GEMM_SOURCES), "fetch_kib_per_dispatch": f,
           "write_kib_per_dispatch": wv,
           "copy_kernel": {"bytes": copy_bytes, "fetch_kib": cf, "write_kib": cw,
                           "fetch_scale": fs, "write_scale": ws},
           "traffic_bytes_per_launch": (f * fs + wv * ws) * 1024}
    out = os.path.join(ROOT, "profiles", f"gemm_f6_dequant_{workload}_traffic.json")
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(f"traffic per launch: {rec['traffic_bytes_per_launch'] / 1e6:.1f} MB -> {out}")


def main():
    args = parse()
    if args.write_traffic:
        write_traffic(args.write_traffic, args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): this build runs on a "
              "single GPU; across GPUs the layer would shard by tokens with no communication",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import hadamard_rotated_bit_amd as hq
    from hadamard_rotated_bit_amd import workloads as WL

    dev = torch.device("cuda:0")
    steps, warmup = args.steps, args.warmup
    head, L, r, Y = config_object(hq, torch, WL, args.workload, steps, warmup, dev)
    w = L.w
    fp6 = head["engine"].startswith("e2m3")
    k1, k2 = head["k1"], head["k2"]
    if k2["ms"] >= k1["ms"]:
        kname = "gemm_f6_dequant" if fp6 else "gemm_i8_dequant"
        roof = {"kernel": kname, "bound": "mfma", "achieved": k2["TOPS"], "peak": k2["peak_TOPS"],
                "unit": "TFLOP/s", "ops": ("e2m3" if fp6 else "int8") + " multiply-add x2",
                "frac": k2["mfma_frac"], "traffic": measured_traffic(kname, w.name),
                "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE)",
                "algorithmic_bytes": k2["bytes"]}
    else:
        roof = {"kernel": "act_stage", "bound": "hbm", "achieved": k1["GBs"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": k1["hbm_frac"], "traffic": None}
    out = {
        "metric": METRIC, "value": head["value"], "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "spin_up_s": SPIN_UP_S,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "e2m3" if fp6 else "int8", "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.T, "d_in": w.d_in, "d_out": w.d_out,
                   "block": w.block, "bits": f"W{w.w_bits}A{w.a_bits}", "center": int(w.center),
                   "smooth_alpha": w.alpha, "rank": w.rank, "io_dtype": w.dtype,
                   "gemm": head["engine"]},
        "effective_tops": head["effective_TOPS_step"],
        "roofline": roof,
        "wall_s_timed": round(r["wall"], 4),
        "host_cores": host_cores(),
        "headline": head,
    }
    if not args.no_cpu_baseline:
        sig = None if L.S is None else L.S.cpu().numpy()
        out["cpu_baseline"] = cpu_baseline(w, L.x, L.weight, L.bias, sig, L.l1, L.l2, Y,
                                           args.cpu_seconds)
    L.free()
    del L, r, Y
    if not args.no_extras:
        es, ew = min(steps, 20), min(warmup, 5)
        cfgs = {}
        for name in CONFIG_ORDER:
            if name == args.workload:
                continue
            obj, Lc, rc, Yc = config_object(hq, torch, WL, name, es, ew, dev)
            if name == "square4k":
                obj["center_off"], obj["centring_overhead"] = centring_off(hq, torch, Lc, rc,
                                                                          es, ew)
                obj["per_channel_centring"] = centring_modes(hq, torch, Lc, es, ew)
            Lc.free()
            del Lc, rc, Yc
            cfgs[name] = obj
        out["configs"] = cfgs
        out["group_wise"] = group_wise(hq, torch, WL, es, ew, dev)
        out["integer_layers"] = [integer_layer(hq, torch, WL, es, ew, dev, side)
                                 for side in (hq.HQ_INT_WH, hq.HQ_INT_DH)] + [
            integer_layer(hq, torch, WL, es, ew, dev, hq.HQ_INT_WH, gelu=True)]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
