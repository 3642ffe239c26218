#!/usr/bin/env python3
"""Throughput of the NVFP4 W4A4 routed-expert MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill|decode]

A step is one ``nvfp4_moe_forward``: route -> permute -> quantise A1 ->
grouped w13 GEMM (+SiLU*mul + requant) -> grouped w2 GEMM -> combine, on one
batch of seeded synthetic input that is already resident in HBM.  The
default workload is the prefill-shaped layer (4096 tokens, hidden 2816, 128
experts, intermediate 704, top-8, biased router).  Inputs rotate over three
sets so repeated steps are not served from the 256 MB last-level cache.

Printed as one JSON line: tokens/s of the layer (``value``), the dominant
kernel's roofline fraction (measured with HIP events on the library's
stream), the per-stage times, the quantiser's HBM GB/s on the
quantiser-alone workload (8192 x 2816, top-8 of 128), and the CPU oracle's
time on a bounded sample of the same workload (``cpu_baseline``).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E peak
MFMA_F16_PEAK_TFLOPS = 2500.0    # MI355X dense fp16/bf16 MFMA peak
MFMA_FP4_PEAK_TFLOPS = 10100.0   # MI355X dense FP4 (scaled MFMA) peak

METRIC = "NVFP4 MoE layer tokens/s (hidden 2816, 128 experts) + quantizer HBM GB/s"


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill", choices=["prefill", "decode", "stack"])
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode sub-measurement of the prefill run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-quantizer", action="store_true")
    ap.add_argument("--no-w4a16", action="store_true",
                    help="skip the weight-only (W4A16) sub-measurement")
    ap.add_argument("--no-mx", action="store_true",
                    help="skip the UE8M0 (MX-style) sub-measurement")
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the 30-layer stack sub-measurement of the prefill run")
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096)
    ap.add_argument("--cpu-passes", type=int, default=2,
                    help="oracle layer forwards timed over the sample (about 7 s each at 4096 tokens)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (the "
                         "known-size reference for the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def copy_calibration(torch):
    n = 1 << 28                                   # 2^28 fp32 = 1 GiB
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log("copy calibration: 3 x 1 GiB device copy done")


class HipEvents:
    """Raw hipEvent_t handles (the library records them on its own stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def record(self, ev, stream):
        if self.hip.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def create(self, n):
        out = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out[i] = h.value
        return out

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, arr):
        for h in arr:
            self.hip.hipEventDestroy(h)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "gemm1_w13_prefill_pmc.md")


def measured_traffic():
    """HBM bytes per launch of the w13 GEMM from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE record, or None when the kernel sources have
    changed since those counters were taken."""
    import hashlib
    try:
        rec = {}
        for line in open(TRAFFIC_RECORD):
            key, sep, val = line.partition(":")
            if sep and key.strip() and " " not in key.strip():
                rec[key.strip()] = val.strip()
        h = hashlib.sha256()
        for f in rec["sources"].split():
            with open(os.path.join(ROOT, f), "rb") as fh:
                h.update(fh.read())
        if h.hexdigest() != rec["sources_sha256"]:
            return None
        return int(rec["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def build_layer(w, torch, M, layer=0, mx=False):
    """Seeded bf16 expert weights -> NVFP4 with the library's quantiser;
    activation scales calibrated with the library's kernels on the layer's
    unbiased calibration batch (UE8M0 block scales throughout when mx)."""
    import synthetic as S
    t0 = time.time()
    w13_bits, w2_bits = S.expert_weights(w, layer=layer)
    w13 = M.bf16_tensor(w13_bits)
    w2 = M.bf16_tensor(w2_bits)
    del w13_bits, w2_bits
    w13c, w13s, w13s2 = M.quantize_expert_weights(w13, mx=mx)
    w2c, w2s, w2s2 = M.quantize_expert_weights(w2, mx=mx)
    del w13, w2
    xc, lc = S.calibration_batch(w, layer=layer)
    cal = M.calibrate_layer(w13c, w13s, w13s2, w2c, w2s, w2s2, M.bf16_tensor(xc),
                            torch.from_numpy(lc).cuda(), w.k, mx=mx)
    cls = M.NVFP4MXMoELayer if mx else M.NVFP4MoELayer
    lay = cls(w13c, w13s, w13s2, w2c, w2s, w2s2, cal.w13_input_scale,
              cal.w2_input_scale, cal.written13, cal.written2)
    torch.cuda.synchronize()
    log(f"{w.name} layer {layer}{' (UE8M0)' if mx else ''} prepared in {time.time() - t0:.1f}s")
    return lay


CLOCK_WARM_S = 0.5      # untimed GPU work before any timed pass


def warm_clocks(torch, step, seconds=CLOCK_WARM_S):
    """Run `step(i)` until `seconds` of wall time have passed, synchronising
    every few steps.  After the GPU has been idle, its first ~20 prefill
    steps (~13 ms) run 15% slower than the steady state (measured per step
    with events on an MI355X: 650-660 us, then 568-580 us from step ~50 on),
    which a handful of warm-up steps does not cover."""
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            step(i)
            i += 1
        torch.cuda.synchronize()
    return i


def time_steps(torch, L, events, runs, steps, warmup, T, k, stage_events=True, fwd=None):
    """Time `steps` calls of nvfp4_moe_forward cycling over `runs` (list of
    (weights, workspace tensor, x, logits, out)); HIP events on torch's
    current stream, which the library launches on.  `fwd` replaces
    nvfp4_moe_forward (the weight-only forward has the same signature).

    After the `warmup` steps and CLOCK_WARM_S of untimed steps, two passes
    over the same steps: the first records HIP events before the first launch
    and after every kernel of every step and gives the per-kernel times; the
    second, uninstrumented, gives the step time.  (An event record costs
    about 3.5 us of GPU time on this stack, so instrumenting the pass that
    gives the step time would add ~20 us to every step; running it second
    means it starts from a GPU that has been busy for a while.)  Returns
    (ms per step, host wall s, per-stage us or None, instrumented ms per step
    or None)."""
    fwd = fwd or L.moe_forward
    stream = torch.cuda.current_stream().cuda_stream
    nst = len(L.MOE_STAGES)

    def step(i, dbg=None):
        wst, ws, x, lg, out = runs[i % len(runs)]
        fwd(wst, x, lg, T, k, None, out, ws, ws.numel(), dbg, stream)

    def timed(dbgs):
        torch.cuda.synchronize()
        ev = events.create(2)
        events.record(ev[0], stream)
        t0 = time.perf_counter()
        for i in range(steps):
            step(i, dbgs[i] if dbgs else None)
        events.record(ev[1], stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = events.elapsed_ms(ev[0], ev[1]) / steps
        events.destroy(ev)
        return ms, wall

    for i in range(warmup):
        step(i)
    warm_clocks(torch, step)
    stage_us = ms_instr = None
    if stage_events:
        evs = [events.create(nst + 1) for _ in range(steps)]
        dbgs = [L.MoEDebug(stage_events=ctypes.cast(e, ctypes.POINTER(ctypes.c_void_p)))
                for e in evs]
        ms_instr, _ = timed(dbgs)
        stage_ms = np.zeros(nst)
        for e in evs:
            for s_ in range(nst):
                stage_ms[s_] += events.elapsed_ms(e[s_], e[s_ + 1])
            events.destroy(e)
        stage_us = {name: 1000.0 * v / steps for name, v in zip(L.MOE_STAGES, stage_ms)}
    ms_step, wall = timed(None)
    return ms_step, wall, stage_us, ms_instr


def bench_layer(args, torch, M, L, events, w, layer):
    """The layer on three rotating seeded input sets of workload w: the
    step time from an uninstrumented timed pass, the per-kernel times from
    an instrumented pass over the same steps (time_steps)."""
    import synthetic as S
    wst = layer.weights()
    ws = layer.workspace(w.T, w.k)
    runs = []
    for i in range(3):
        x = M.bf16_tensor(S.activations(w, layer=i))
        lg = torch.from_numpy(S.router_logits(w, layer=i)).cuda()
        runs.append((wst, ws, x, lg, torch.empty_like(x)))
    return time_steps(torch, L, events, runs, args.steps, args.warmup, w.T, w.k)


def bench_w4a16(args, torch, M, L, events, layers):
    """The weight-only (W4A16) forward over the same packed weights: the
    prefill layer (three input sets) and the 16-token decode step on two
    alternating layers.  Same stage events (the quantise stage is empty)."""
    import synthetic as S
    views = [M.NVFP4W4A16MoELayer.sharing(lay) for lay in layers]
    out = {}
    for name, steps, lays in (("prefill", args.steps, views[:1]),
                              ("decode", max(args.steps, 200), views)):
        w = S.WORKLOADS[name]
        runs = []
        for i in range(3):
            x = M.bf16_tensor(S.activations(w, layer=i))
            lg = torch.from_numpy(S.router_logits(w, layer=i)).cuda()
            for v in lays:
                runs.append((v.weights(), v.workspace(w.T, w.k), x, lg, torch.empty_like(x)))
        ms, _, st, ms_i = time_steps(torch, L, events, runs, steps, args.warmup, w.T, w.k,
                               fwd=L.moe_forward_w4a16)
        P = w.T * w.k
        f1 = 2.0 * P * (2 * w.I) * w.H
        f2 = 2.0 * P * w.H * w.I
        g1, g2 = st["gemm1_w13"], st["gemm2_w2"]
        out[name] = dict(tokens_per_s=round(w.T / (ms * 1e-3), 1), us_per_step=round(ms * 1000, 2),
                         us_per_step_instrumented=round(ms_i * 1000, 2),
                         stages_us={k_: round(v, 2) for k_, v in st.items()},
                         gemm1_tflops=round(f1 / (g1 * 1e-6) / 1e12, 1),
                         gemm2_tflops=round(f2 / (g2 * 1e-6) / 1e12, 1),
                         gemm1_frac_of_bf16_peak=round(f1 / (g1 * 1e-6) / 1e12
                                                       / MFMA_F16_PEAK_TFLOPS, 4))
    return out


def bench_mx(args, torch, M, L, events):
    """The UE8M0 (MX-style) mode: its own layers (weights quantised with
    UE8M0 scales, activation scales calibrated through that mode), the
    prefill layer and the 16-token decode step on two alternating layers.
    GEMM rates against the dense FP4 matrix peak."""
    import synthetic as S
    layers = [build_layer(S.WORKLOADS["decode"], torch, M, layer=i, mx=True) for i in range(2)]
    out = {}
    for name, steps, lays in (("prefill", args.steps, layers[:1]),
                              ("decode", max(args.steps, 200), layers)):
        w = S.WORKLOADS[name]
        runs = []
        for i in range(3):
            x = M.bf16_tensor(S.activations(w, layer=i))
            lg = torch.from_numpy(S.router_logits(w, layer=i)).cuda()
            for v in lays:
                runs.append((v.weights(), v.workspace(w.T, w.k), x, lg, torch.empty_like(x)))
        ms, _, st, ms_i = time_steps(torch, L, events, runs, steps, args.warmup, w.T, w.k,
                                     fwd=L.moe_forward_mx)
        P = w.T * w.k
        f1 = 2.0 * P * (2 * w.I) * w.H
        f2 = 2.0 * P * w.H * w.I
        g1, g2 = st["gemm1_w13"], st["gemm2_w2"]
        out[name] = dict(tokens_per_s=round(w.T / (ms * 1e-3), 1), us_per_step=round(ms * 1000, 2),
                         us_per_step_instrumented=round(ms_i * 1000, 2),
                         stages_us={k_: round(v, 2) for k_, v in st.items()},
                         gemm1_tflops=round(f1 / (g1 * 1e-6) / 1e12, 1),
                         gemm2_tflops=round(f2 / (g2 * 1e-6) / 1e12, 1),
                         gemm1_frac_of_fp4_peak=round(f1 / (g1 * 1e-6) / 1e12
                                                      / MFMA_FP4_PEAK_TFLOPS, 4))
    return out


def bench_decode(args, torch, M, L, events, layers):
    """16-token decode on two alternating layers (weights > last-level
    cache), three input sets each: tokens/s and the w13 GEMM's weight-
    streaming rate (NVFP4 bytes of the experts the batch hits)."""
    import synthetic as S
    w = S.WORKLOADS["decode"]
    runs, hits = [], []
    for li, lay in enumerate(layers):
        wst = lay.weights()
        ws = lay.workspace(w.T, w.k)
        for i in range(3):
            x = M.bf16_tensor(S.activations(w, layer=i))
            lg_np = S.router_logits(w, layer=i)
            hits.append(int(np.unique(np.argsort(-lg_np, axis=1, kind="stable")[:, :w.k]).size))
            runs.append((wst, ws, x, torch.from_numpy(lg_np).cuda(), torch.empty_like(x)))
    # order: layer 0 set 0, layer 1 set 0, ... so consecutive steps switch weights
    order = [runs[li * 3 + i] for i in range(3) for li in range(len(layers))]
    hit_order = [hits[li * 3 + i] for i in range(3) for li in range(len(layers))]
    steps = max(args.steps, 200)
    ms, wall, st, ms_i = time_steps(torch, L, events, order, steps, args.warmup, w.T, w.k)
    n_hit = float(np.mean(hit_order))
    per_expert = 2 * w.I * w.H * 9 // 16 + w.H * w.I * 9 // 16       # w13 + w2 codes+scales
    g1_bytes = n_hit * (2 * w.I * w.H * 9 // 16)
    g1 = st["gemm1_w13"]
    return dict(workload=f"decode MoE layer: {w.T} tokens, hidden {w.H}, {w.E} experts, "
                         f"intermediate {w.I}, top-{w.k}; 2 alternating layers x 3 input sets",
                tokens_per_s=round(w.T / (ms * 1e-3), 1), us_per_step=round(ms * 1000, 2),
                us_per_step_instrumented=round(ms_i * 1000, 2), experts_hit=round(n_hit, 1),
                weight_bytes_per_step=int(n_hit * per_expert),
                layer_weight_gbps=round(n_hit * per_expert / (ms * 1e-3) / 1e9, 1),
                # the whole step against the time the hit experts' weights take at peak HBM
                layer_frac_of_hbm_peak=round(n_hit * per_expert / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                gemm1_weight_gbps=round(g1_bytes / (g1 * 1e-6) / 1e9, 1),
                gemm1_frac_of_hbm_peak=round(g1_bytes / (g1 * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                stages_us={k_: round(v, 2) for k_, v in st.items()})


def bench_stack(args, torch, M, L, events):
    """The 30-layer stack: x_{l+1} = bf16(x_l + MoE_l(x_l)), each layer with
    its own weights, scales and Zipf router; 8192 tokens.  Times whole
    passes over the stack."""
    import synthetic as S
    w = S.WORKLOADS["stack"]
    layers = [build_layer(w, torch, M, layer=l) for l in range(w.layers)]
    wsts = [lay.weights() for lay in layers]
    nbytes = max(L.moe_workspace_size(w.T, w.k, wst) for wst in wsts)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    logits = [torch.from_numpy(S.router_logits(w, layer=l)).cuda() for l in range(w.layers)]
    x0 = M.bf16_tensor(S.activations(w, layer=0))
    bufs = [torch.empty_like(x0), torch.empty_like(x0)]
    stream = torch.cuda.current_stream().cuda_stream

    def one_pass():
        x = x0
        for l in range(w.layers):
            out = bufs[l % 2]
            L.moe_forward(wsts[l], x, logits[l], w.T, w.k, x, out, ws, nbytes, None, stream)
            x = out
        return x

    one_pass()
    torch.cuda.synchronize()
    warm_clocks(torch, lambda i: one_pass() if i % 8 == 0 else None)
    passes = 3
    ev = events.create(2)
    events.record(ev[0], stream)
    for _ in range(passes):
        one_pass()
    events.record(ev[1], stream)
    torch.cuda.synchronize()
    ms = events.elapsed_ms(ev[0], ev[1]) / passes
    events.destroy(ev)
    flops = 6.0 * w.T * w.k * w.H * w.I * w.layers
    tflops = flops / (ms * 1e-3) / 1e12
    return w, dict(workload=f"30-layer MoE stack: {w.T} tokens, hidden {w.H}, {w.E} experts, "
                            f"intermediate {w.I}, top-{w.k}, Zipf(1.1) routing with empty "
                            f"experts, residual add between layers",
                   ms_per_stack=round(ms, 3), tokens_per_s=round(w.T / (ms * 1e-3), 1),
                   layer_tokens_per_s=round(w.T * w.layers / (ms * 1e-3), 1),
                   expert_gemm_flops=flops, tflops_whole_stack=round(tflops, 1),
                   frac_of_f16_peak=round(tflops / MFMA_F16_PEAK_TFLOPS, 4), passes=passes)


def copy_ceiling(torch, events):
    """A plain 1 GiB device-to-device copy (torch's copy kernel), timed with
    HIP events: the practical HBM ceiling beside the 8 TB/s peak."""
    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    ev = events.create(2)
    events.record(ev[0], stream)
    for _ in range(10):
        b.copy_(a)
    events.record(ev[1], stream)
    torch.cuda.synchronize()
    ms = events.elapsed_ms(ev[0], ev[1]) / 10
    events.destroy(ev)
    del a, b
    return round(2 * 4 * n / (ms * 1e-3) / 1e9, 1)


def bench_quantizer(args, torch, M, L, events):
    """The quantiser alone on the quantiser workload, 3 rotating input/output
    sets (> last-level cache): nvfp4_quantize_pairs, the form the layer runs
    (each token row read once for its 8 destination rows; the headline), and
    the gather form nvfp4_quantize_experts over the permuted rows."""
    import synthetic as S
    w = S.WORKLOADS["quant"]
    xc, lc = S.calibration_batch(w)
    # per-expert input scale from the calibration batch, with the library's
    # calibration pass and load-time check
    dev = "cuda"
    Tc = xc.shape[0]
    ids = torch.empty((Tc, w.k), dtype=torch.int32, device=dev)
    wts = torch.empty((Tc, w.k), dtype=torch.float32, device=dev)
    off = torch.empty(w.E + 1, dtype=torch.int32, device=dev)
    src = torch.empty(Tc * w.k, dtype=torch.int32, device=dev)
    inv = torch.empty(Tc * w.k, dtype=torch.int32, device=dev)
    L.route_topk(torch.from_numpy(lc).cuda(), Tc, w.E, w.k, ids, wts)
    L.permute(ids, Tc, w.k, w.E, off, src, inv)
    s13 = torch.empty(w.E, dtype=torch.float32, device=dev)
    written = torch.empty(w.E, dtype=torch.uint8, device=dev)
    L.calibrate_input_scales(M.bf16_tensor(xc), w.H, w.H, src, w.k, off, w.E, Tc * w.k, s13,
                             written)
    st, gs, _, _ = L.validate_scales(s13.cpu().numpy(), written.cpu().numpy())
    if st != L.OK:
        raise RuntimeError("quantiser workload calibration left unwritten slots")
    gs_d = torch.from_numpy(gs).cuda()
    sets = []
    for i in range(3):
        x = M.bf16_tensor(S.activations(w, layer=i))
        lg = torch.from_numpy(S.router_logits(w, layer=i)).cuda()
        ids = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
        wts = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
        off = torch.empty(w.E + 1, dtype=torch.int32, device=dev)
        src = torch.empty(w.P, dtype=torch.int32, device=dev)
        inv = torch.empty(w.P, dtype=torch.int32, device=dev)
        L.route_topk(lg, w.T, w.E, w.k, ids, wts)
        L.permute(ids, w.T, w.k, w.E, off, src, inv)
        src_row = torch.div(src, w.k, rounding_mode="floor").to(torch.int32)
        codes = torch.empty((w.P, w.H // 2), dtype=torch.uint8, device=dev)
        sf = torch.empty((w.P, w.H // 16), dtype=torch.uint8, device=dev)
        sets.append((x, ids, inv, off, src_row, codes, sf))
    stream = torch.cuda.current_stream().cuda_stream

    def pairs(i):
        x, ids, inv, off, src_row, codes, sf = sets[i % 3]
        L.quantize_pairs(x, w.H, w.T, w.H, w.k, ids, None, w.E, gs_d, codes, sf, w.P, stream)

    def pairs_grouped(i):
        x, ids, inv, off, src_row, codes, sf = sets[i % 3]
        L.quantize_pairs(x, w.H, w.T, w.H, w.k, ids, inv, w.E, gs_d, codes, sf, w.P, stream)

    def gather(i):
        x, ids, inv, off, src_row, codes, sf = sets[i % 3]
        L.quantize_experts(x, w.H, w.H, src_row, w.T, w.P, off, w.E, gs_d, codes, sf, stream)

    def timed(step):
        for i in range(args.warmup):
            step(i)
        warm_clocks(torch, step)
        n = max(args.steps, 50)
        ev = events.create(2)
        events.record(ev[0], stream)
        for i in range(n):
            step(i)
        events.record(ev[1], stream)
        torch.cuda.synchronize()
        us = 1000.0 * events.elapsed_ms(ev[0], ev[1]) / n
        events.destroy(ev)
        return us

    us = timed(pairs)
    us_grouped = timed(pairs_grouped)
    us_gather = timed(gather)
    # algorithmic bytes: unique x once, the routing ids, the scales, packed
    # codes and E4M3 block scales written (the grouped forms also read one
    # destination / source index per row)
    read = w.T * w.H * 2 + w.P * 4 + w.E * 4
    write = w.P * (w.H // 2) + w.P * (w.H // 16)
    alg = read + write
    gbps = alg / (us * 1e-6) / 1e9
    return dict(workload="quantizer alone: 8192 tokens x hidden 2816 bf16, top-8 of 128 experts, "
                         "1% outlier channels x50",
                kernel="quantize_pairs_fast_kernel<false> (nvfp4_quantize_pairs, rows in "
                       "(token, slot) order: the layer's form)",
                us_per_launch=round(us, 3), algorithmic_bytes=int(alg),
                gbps=round(gbps, 1), peak_gbps=HBM_PEAK_GBPS, frac=round(gbps / HBM_PEAK_GBPS, 4),
                grouped_rows_us=round(us_grouped, 3),
                grouped_rows_gbps=round((alg + w.P * 4) / (us_grouped * 1e-6) / 1e9, 1),
                gather_form_us=round(us_gather, 3),
                gather_form_gbps=round((alg + w.P * 4) / (us_gather * 1e-6) / 1e9, 1))


def blas_info():
    """The BLAS library NumPy's fp64 GEMMs run on, and its thread count."""
    try:
        from threadpoolctl import threadpool_info
        for d in threadpool_info():
            if d.get("user_api") == "blas":
                return dict(vendor=d.get("internal_api"), version=d.get("version"),
                            threads=d.get("num_threads"))
    except Exception:                                     # reported as unknown
        pass
    return dict(vendor=None, version=None, threads=None)


def _timed_repeats(fn, min_seconds):
    """Call fn() until min_seconds have passed (at least once); return
    (calls, seconds)."""
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            return n, dt


def cpu_baseline(args, w):
    """The CPU oracle, unchanged, timed on bounded samples: the headline is
    the prefill layer (its own NVFP4 layer, prepared untimed, then
    ``cpu_passes`` layer forwards over the first ``cpu_sample_tokens`` tokens
    of the benchmark batch); beside it, the other workloads: the 64-token tiny
    layer, the quantiser alone on 512 tokens of its batch, the 16-token decode
    layer, and one layer of the 30-layer stack on 512 tokens."""
    import synthetic as S
    from oracle import moe as OM
    from oracle import quant as OQ
    threads = min(16, os.cpu_count() or 1)
    t0 = time.time()
    w13, w2 = S.expert_weights(w)
    xc, lc = S.calibration_batch(w)
    layer = OM.prepare_layer(w13, w2, xc, lc, w.k, threads=threads)
    del w13, w2
    log(f"oracle layer prepared in {time.time() - t0:.1f}s (untimed)")
    n = args.cpu_sample_tokens
    x = S.activations(w)[:n]
    lg = S.router_logits(w)[:n]
    passes = max(1, args.cpu_passes)
    t0 = time.perf_counter()
    for _ in range(passes):
        OM.layer_forward(layer, x, lg, w.k)
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    blas = blas_info()
    per = {}

    # the tiny layer (64 tokens, 4 experts, hidden 256, top-2), prepared untimed
    wt = S.WORKLOADS["tiny"]
    w13t, w2t = S.expert_weights(wt)
    tlayer = OM.prepare_layer(w13t, w2t, *S.calibration_batch(wt), wt.k, threads=threads)
    xt, lt = S.activations(wt), S.router_logits(wt)
    reps, sec = _timed_repeats(lambda: OM.layer_forward(tlayer, xt, lt, wt.k), 1.0)
    per["tiny"] = dict(tokens_per_s=round(reps * wt.T / sec, 3), seconds=round(sec, 2),
                       sample=f"{reps} full forwards of the {wt.T}-token tiny layer "
                              f"({wt.E} experts, hidden {wt.H}, top-{wt.k})")
    del tlayer, w13t, w2t

    # the 16-token decode layer (the same layer as the prefill one)
    wd = S.WORKLOADS["decode"]
    xd, ld = S.activations(wd), S.router_logits(wd)
    reps, sec = _timed_repeats(lambda: OM.layer_forward(layer, xd, ld, wd.k), 2.0)
    per["decode"] = dict(tokens_per_s=round(reps * wd.T / sec, 3), seconds=round(sec, 2),
                         sample=f"{reps} full forwards of the {wd.T}-token decode batch")
    del layer

    # the quantiser alone (route, permute and scales untimed; the timed part
    # is the per-expert quantisation of every routed row, as on the GPU)
    wq = S.WORKLOADS["quant"]
    nq = 512
    s13, written = OM.calibrate_input_scale(*S.calibration_batch(wq), wq.k, wq.E)
    ok, gs, _ = OM.validate_scales(s13, written)
    xq = S.activations(wq, tokens=nq)
    ids, _ = OM.route(S.router_logits(wq, tokens=nq), wq.k)
    off, src, _ = OM.permute(ids, wq.E)
    rexp = OM.row_experts(off)
    xp = xq[src // wq.k]
    reps, sec = _timed_repeats(lambda: OQ.quantize_experts(xp, rexp, gs), 2.0)
    qbytes = nq * wq.H * 2 + nq * wq.k * 8 + wq.E * 4 + nq * wq.k * (wq.H // 2 + wq.H // 16)
    per["quantizer"] = dict(tokens_per_s=round(reps * nq / sec, 3),
                            gbps=round(reps * qbytes / sec / 1e9, 4), seconds=round(sec, 2),
                            cores=1, sample=f"{reps} quantisations of the {nq * wq.k} routed "
                                            f"rows of the first {nq} tokens (NumPy, one core)")

    # one layer of the 30-layer stack
    ws = S.WORKLOADS["stack"]
    t0 = time.time()
    w13, w2 = S.expert_weights(ws, layer=0)
    xc, lc = S.calibration_batch(ws, layer=0)
    slayer = OM.prepare_layer(w13, w2, xc, lc, ws.k, threads=threads)
    del w13, w2
    log(f"oracle stack layer prepared in {time.time() - t0:.1f}s (untimed)")
    ns = 512
    xs, ls = S.activations(ws, tokens=ns), S.router_logits(ws, layer=0, tokens=ns)
    reps, sec = _timed_repeats(lambda: OM.layer_forward(slayer, xs, ls, ws.k, xs), 2.0)
    per["stack_layer"] = dict(tokens_per_s=round(reps * ns / sec, 3),
                              stack_tokens_per_s=round(reps * ns / sec / ws.layers, 3),
                              seconds=round(sec, 2),
                              sample=f"{reps} forwards of layer 0 of the stack on its first {ns} "
                                     f"tokens (Zipf routing, residual)")
    return dict(value=round(passes * n / dt, 3), unit="tokens/s", cores=cores, kind="oracle",
                seconds=round(dt, 2), blas=blas,
                sample=f"first {n} tokens of the {args.workload} batch, {passes} full layer "
                       f"forward(s) "
                       f"(route, permute, quantise, fp64 GEMMs over dequantised operands, "
                       f"SiLU*mul, requant, combine); NumPy elementwise work single-threaded, "
                       f"fp64 GEMMs on {blas['vendor']} with {blas['threads']} threads "
                       f"({cores} cores visible)",
                per_workload=per)


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(torch)
        return
    from nvfp4_w4a4_expert_amd import _lib as L
    from nvfp4_w4a4_expert_amd import moe as M
    events = HipEvents()

    import synthetic as S
    decode = copy_gbps = quant = cpu = w4a16 = mx = ms_instr = stack = None
    if args.workload == "stack":
        w, st = bench_stack(args, torch, M, L, events)
        ms_step, wall, stage_us = st["ms_per_stack"], None, None
        tokens_per_s = st["tokens_per_s"]
        log(f"stack: {st}")
        roofline = dict(kernel="whole stack (30 layers, every kernel) vs expert-GEMM flops",
                        bound="mfma", achieved=st["tflops_whole_stack"],
                        peak=MFMA_F16_PEAK_TFLOPS, unit="TFLOP/s", frac=st["frac_of_f16_peak"],
                        traffic=None, algorithmic_flops=st["expert_gemm_flops"])
        gemms = None
        extra = dict(stack=st)
    else:
        # the prefill and decode layers share one layer (weights and scales)
        layer = build_layer(S.WORKLOADS["decode"], torch, M)
        if args.workload == "prefill":
            w = S.WORKLOADS["prefill"]
            ms_step, wall, stage_us, ms_instr = bench_layer(args, torch, M, L, events, w, layer)
            tokens_per_s = w.T / (ms_step * 1e-3)
            log(f"layer: {ms_step * 1000:.1f} us/step, {tokens_per_s:.4g} tokens/s; "
                f"stages {stage_us}")
            P = w.T * w.k
            flops_gemm1 = 2.0 * P * (2 * w.I) * w.H
            flops_gemm2 = 2.0 * P * w.H * w.I
            g1 = stage_us["gemm1_w13"]
            ach = flops_gemm1 / (g1 * 1e-6) / 1e12
            roofline = dict(kernel="grouped_gemm_kernel<true> (w13 + SiLU*mul + requant)",
                            bound="mfma", achieved=round(ach, 1), peak=MFMA_F16_PEAK_TFLOPS,
                            unit="TFLOP/s", frac=round(ach / MFMA_F16_PEAK_TFLOPS, 4),
                            traffic=measured_traffic(),
                            algorithmic_flops=flops_gemm1, us_per_launch=round(g1, 2))
            gemm_us = stage_us["gemm1_w13"] + stage_us["gemm2_w2"]
            tf = (flops_gemm1 + flops_gemm2) / (gemm_us * 1e-6) / 1e12
            gemms = dict(us=round(gemm_us, 2), tflops=round(tf, 1),
                         frac_of_f16_peak=round(tf / MFMA_F16_PEAK_TFLOPS, 4))
            if not args.no_decode or not args.no_w4a16:
                second = build_layer(S.WORKLOADS["decode"], torch, M, layer=1)
                if not args.no_decode:
                    decode = bench_decode(args, torch, M, L, events, [layer, second])
                    log(f"decode: {decode}")
                if not args.no_w4a16:
                    w4a16 = bench_w4a16(args, torch, M, L, events, [layer, second])
                    log(f"w4a16: {w4a16}")
                del second
            if not args.no_mx:
                mx = bench_mx(args, torch, M, L, events)
                log(f"mx: {mx}")
            if not args.no_stack:
                _, stack = bench_stack(args, torch, M, L, events)
                log(f"stack: {stack}")
        else:                                             # decode
            w = S.WORKLOADS["decode"]
            second = build_layer(w, torch, M, layer=1)
            decode = bench_decode(args, torch, M, L, events, [layer, second])
            log(f"decode: {decode}")
            ms_step, wall, stage_us = decode["us_per_step"] / 1000.0, None, decode["stages_us"]
            ms_instr = decode["us_per_step_instrumented"] / 1000.0
            tokens_per_s = decode["tokens_per_s"]
            g1 = stage_us["gemm1_w13"]
            roofline = dict(kernel="grouped_gemm_kernel<true> (w13, weight streaming)",
                            bound="hbm", achieved=decode["gemm1_weight_gbps"],
                            peak=HBM_PEAK_GBPS, unit="GB/s",
                            frac=decode["gemm1_frac_of_hbm_peak"], traffic=None,
                            experts_hit=decode["experts_hit"], us_per_launch=round(g1, 2))
            gemms = None
        extra = dict(decode=decode, w4a16=w4a16, mx=mx, stack=stack)
        del layer

    if args.workload == "prefill":
        if not args.no_quantizer:
            quant = bench_quantizer(args, torch, M, L, events)
            log(f"quantizer: {quant}")
        copy_gbps = copy_ceiling(torch, events)
        log(f"device copy: {copy_gbps} GB/s (read + write)")
        if not args.no_cpu_baseline:
            cpu = cpu_baseline(args, w)
            log(f"cpu baseline: {cpu}")

    rec = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "ms_per_step_instrumented": round(ms_instr, 5) if ms_instr is not None else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": (("30-layer MoE stack" if args.workload == "stack" else
                          f"{args.workload} MoE layer") +
                         f": {w.T} tokens, hidden {w.H}, {w.E} experts, "
                         f"intermediate {w.I}, top-{w.k}, NVFP4 W4A4 (E2M1 + E4M3/16 + fp32), "
                         f"fp16 MFMA over exactly dequantised operands, fp32 accumulate"),
            "tokens": w.T, "hidden": w.H, "experts": w.E, "inter": w.I, "topk": w.k,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "stages_us": {k: round(v, 2) for k, v in stage_us.items()} if stage_us else None,
        "expert_gemms": gemms,
        "quantizer": quant,
        "hbm_copy_gbps": copy_gbps,
        "host_wall_s": round(wall, 4) if wall is not None else None,
    }
    rec.update(extra)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
