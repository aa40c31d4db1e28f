#!/usr/bin/env python3
"""Throughput of one sigmoid-routed int4 x Q8_0 MoE layer on one MI355X.

Default workload: GLM-5.2-shaped decode at batch 1 (1 token per step, hidden
6144, 256 routed experts, top-8, one shared expert, intermediate 2048). A
step is one full coli_moe_forward: Q8_0(x), router + top-k, bucketing,
gate/up + SwiGLU + requant, down, weighted combine. Every step uses a new
seeded token and the next of R layer replicas (distinct seeded weights), so
the 256 MB Infinity Cache never serves a previous step's weights.

Prints one JSON line (see the fields below). Options: --config picks another
workload (0 tiny, 1 decode, 2 MTP verify T=3, 3 prefill T=512, 4 the 8-layer
pre-norm residual stack at T=4096); --gpus must be 1 (one GPU).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0

# HBM bytes per launch of the dominant kernel from rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE (two runs), scaled by what the counters read for a plain device
# copy of known size (FETCH_SIZE x 2, WRITE_SIZE x 1). Keyed by (kernel,
# workload as the JSON line names it); dropped whenever that kernel changes.
TRAFFIC = {
    # profiles/dec_kernels_decode_T1.txt
    ("dec_gateup", "decode T1 H6144 E256 K8 I2048"): (55670.6 * 2 + 38.4) * 1024,
    # profiles/dec_kernels_decode_T1_int8.txt, profiles/dec_kernels_decode_T1_int2.txt
    ("dec_gateup", "decode T1 H6144 E256 K8 I2048 int8 weights"): (111687.3 * 2 + 38.4) * 1024,
    ("dec_gateup", "decode T1 H6144 E256 K8 I2048 int2 weights"): (28007.7 * 2 + 38.4) * 1024,
    # profiles/dec_kernels_mtp_verify_T3.txt (mean over the counter run's steps)
    ("dec_gateup", "mtp-verify T3 correlated"): (95923.0 * 2 + 84.8) * 1024,
    # profiles/pf_kernels_prefill_T512.txt, profiles/pf_kernels_prefill_T512_int8.txt
    ("pf_gateup", "prefill T512 zipf-bias"): (1819205.2 * 2 + 14437.5) * 1024,
    ("pf_gateup", "prefill T512 zipf-bias int8 weights"): (3383330.9 * 2 + 14460.6) * 1024,
    # profiles/pack_fp8_int4_layer.txt (the gate/up launch)
    ("pack_fp8_gateup", "pack_fp8 layer H6144 I2048 experts257"): (3164334.8 * 2 + 3166240.7) * 1024,
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", type=int, default=1)
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="time budget of the oracle CPU-baseline sample (0 = skip)")
    ap.add_argument("--no-profile", action="store_true", help="skip the per-kernel event pass")
    ap.add_argument("--sweep", type=str, default="",
                    help="comma-separated token counts: time the layer of --config at each "
                         "(one JSON line per count) instead of the default run")
    ap.add_argument("--bits", type=int, default=4, choices=(2, 4, 8),
                    help="width of the expert weight codes (int8 and int2 run on the grouped "
                         "MFMA kernels at every token count)")
    ap.add_argument("--groups", type=str, default="",
                    help="NG,TG: group-limited expert selection (NG groups, the TG best kept)")
    ap.add_argument("--op", choices=("layer", "pack_fp8"), default="layer",
                    help="pack_fp8: time the FP8 e4m3 (128 x 128 block scales) -> int4 "
                         "conversion of one layer's expert weights instead of the layer")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MiB",
                    help="only run a plain device copy of this many MiB a few times (the "
                         "reference kernel that scales HBM byte counters) and exit")
    return ap.parse_args()


def calibrate_copy(mib: int):
    import torch
    torch.cuda.set_device(0)
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n,
                      "launches": 5}), flush=True)


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU: the layer is not sharded "
                                   "across GPUs (use --gpus 1)", "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import coli_synth as cs
    import int4_quantized_moe_sigmoid_amd as C

    torch.cuda.set_device(0)
    cfg = cs.CONFIGS[args.config]
    if args.op == "pack_fp8":
        run_pack_fp8(args, cfg)
        return
    if cfg.n_layers > 1:
        run_stack(args, cfg)
        return
    if args.sweep:
        run_sweep(args, cfg, [int(v) for v in args.sweep.split(",") if v])
        return
    T, H, I, E, K, S = cfg.n_tok, cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.n_shared
    ng, tg = (int(v) for v in args.groups.split(",")) if args.groups else (1, 1)
    bits = args.bits
    lc = C.make_cfg(H, I, E, K, S, cfg.norm_topk, cfg.rho, ng, tg, bits)
    R = max(1, args.replicas)
    n_steps, n_warm = args.steps, args.warmup
    n_inputs = n_steps + n_warm

    t_setup = time.time()
    pack = lambda w, qv, sv: C.coli_pack_weights(w, bits, qv, sv)
    layers = []
    for r in range(R):
        wr, b, q, s = cs.build_layer(cfg, r, "cuda", pack, bits=bits)
        layers.append(C.LayerWeights(lc, wr, b, q, s))
        print(f"[bench] replica {r} packed ({(q.numel() + 4 * s.numel()) / 1e9:.2f} GB)",
              file=sys.stderr, flush=True)
    # distinct seeded inputs for every step, RMS-normalised on the GPU when the
    # workload's input is normalised
    xs = []
    for i in range(n_inputs):
        raw = cs.activations(cfg, i % R, "cuda", n_tok=T, first_tok=(i // R) * T)
        if cfg.rmsnorm_input:
            xn = torch.empty_like(raw)
            C.coli_rmsnorm(raw, xn, 1e-5)
            raw = xn
        xs.append(raw)
    ys = [torch.empty((T, H), dtype=torch.float32, device="cuda") for _ in range(2)]
    ws = torch.empty(C.coli_moe_workspace_bytes(lc, T), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup

    def step(i):
        C.coli_moe_forward(layers[i % R], xs[i], ys[i & 1], ws)

    for i in range(n_warm):
        step(n_steps + i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / n_steps
    tok_s = T * n_steps / elapsed

    # bytes that must cross HBM per step: unique experts' packed weights + scales,
    # the router weight, activations in and out
    lay = C.coli_moe_workspace_layout(lc, T, 0)
    eb = 3 * I * H * bits // 8 + 4 * (2 * I + H)

    # ---- per-kernel durations with HIP events on the same stream -------------
    kern = {}
    unique_counts = []
    if not args.no_profile:
        names = None
        nev = 32  # start and stop of each launch
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(nev)]
        for e in evs:
            e.record()
        torch.cuda.synchronize()
        handles = [e.cuda_event for e in evs]
        sums = {}
        n_prof = n_steps
        counts_view = ws[lay.counts:lay.counts + 4 * (E + S)].view(torch.int32)
        for i in range(n_prof):
            names = C.coli_moe_forward_profiled(layers[i % R], xs[i], ys[i & 1], ws, handles)
            torch.cuda.synchronize()
            for j in range(len(names)):
                sums[names[j]] = sums.get(names[j], 0.0) + \
                    evs[2 * j].elapsed_time(evs[2 * j + 1])
            unique_counts.append(int((counts_view[:E] > 0).sum().item()) + S)
        kern = {k: v / n_prof for k, v in sums.items()}
    uniq_avg = float(np.mean(unique_counts)) if unique_counts else float(min(E, T * K) + S)

    # algorithmic HBM bytes of the gate/up launch: the packed gate and up rows and
    # their scales of every expert in use, Q8_0(x) in, Q8_0(h) out (+ the fp64
    # router logits the decode kernel reads to redo the top-k)
    gate_up_bytes = uniq_avg * (2 * I * H * bits // 8 + 4 * 2 * I) + T * (H + H // 8) + \
        T * (K + S) * (I + I // 8)
    step_bytes = uniq_avg * eb + 4 * E * H + 4 * E + 8 * T * H
    weight_gbps = uniq_avg * eb / (ms_per_step * 1e-3) / 1e9

    roofline = gateup_roofline(kern, cfg, gate_up_bytes, T, bits)
    ceiling = read_ceiling_gbps(C)
    if roofline:
        roofline["frac_of_read_ceiling"] = round(roofline["achieved"] / ceiling, 4)

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(cfg, args.cpu_seconds)

    out = {
        "metric": "MoE-layer tokens/s; decode int4 expert-weight GB/s as % of HBM peak",
        "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1, "steps": n_steps,
        "warmup": n_warm, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": f"int{bits}xint8 (int32 block dots, f64 scales)",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights packed by "
                "coli_pack_weights)",
        "config": {"workload": cfg.name + (f" groups {ng}/{tg}" if ng > 1 else "") +
                   (f" int{bits} weights" if bits != 4 else ""),
                   "tokens_per_step": T, "hidden": H, "inter": I,
                   "n_experts": E, "top_k": K, "n_shared": S, "weight_replicas": R,
                   "n_group": ng, "topk_group": tg, "weight_bits": bits,
                   "parallelism": "none (1 GPU)"},
        "expert_weight_gbps": round(weight_gbps, 1),
        "expert_weight_frac_hbm": round(weight_gbps / HBM_PEAK_GBPS, 4),
        "read_ceiling_gbps": ceiling,
        "expert_weight_frac_read_ceiling": round(weight_gbps / ceiling, 4),
        "unique_experts_per_step": round(uniq_avg, 2),
        "algorithmic_bytes_per_step": int(step_bytes),
        "kernel_avg_us": {k: round(v * 1e3, 2) for k, v in kern.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(out), flush=True)


def run_pack_fp8(args, cfg):
    """One step = the FP8 -> int4 conversion of one layer's expert weights
    (E routed + S shared experts) as two launches: the gate and up rows of
    every expert stacked into one [(E+S)*2I, H] matrix, the down rows into one
    [(E+S)*H, I] matrix (rows are independent, so stacking changes nothing in
    the result). Synthetic codes: seeded N(0, 64^2) rounded to e4m3; block
    scales 2^k * U(1, 2). With power-of-two block scales instead, many w / s
    are exact half-integers and most chunks take the kernel's exact-division
    path (about twice the time)."""
    import torch

    import int4_quantized_moe_sigmoid_amd as C
    H, I, n_exp = cfg.hidden, cfg.inter, cfg.n_experts + cfg.n_shared
    mats = []
    g = torch.Generator(device="cuda").manual_seed(17)
    for rows_per, cols in ((2 * I, H), (H, I)):
        rows = n_exp * rows_per
        q8 = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
        for r0 in range(0, rows, 8192):
            r1 = min(rows, r0 + 8192)
            w = torch.randn((r1 - r0, cols), generator=g, device="cuda") * 64.0
            q8[r0:r1] = w.to(torch.float8_e4m3fn).view(torch.uint8)
        nb = ((rows + 127) // 128, (cols + 127) // 128)
        # block scales as a block-wise FP8 quantiser writes them (block max / 448):
        # arbitrary fp32 values of a few binades
        bs = torch.exp2(torch.randint(-14, -6, nb, generator=g, device="cuda").float()) * \
            (1.0 + torch.rand(nb, generator=g, device="cuda"))
        q = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda")
        sc = torch.empty(rows, dtype=torch.float32, device="cuda")
        mats.append((q8, bs, q, sc))
    torch.cuda.synchronize()

    def step():
        for q8, bs, q, sc in mats:
            C.coli_pack_fp8_int4(q8, bs, q, sc)

    n_steps, n_warm = max(1, args.steps), args.warmup
    for _ in range(n_warm):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # algorithmic bytes: every code read once, half a byte written per code, the
    # row scales written, the block scales read
    step_bytes = sum(q8.numel() * 1.5 + 4 * sc.numel() + 4 * bs.numel()
                     for q8, bs, q, sc in mats)
    # per-launch durations with HIP events on the launch stream
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    dur = [0.0, 0.0]
    n_prof = min(n_steps, 10)
    for _ in range(n_prof):
        evs[0].record()
        for j, (q8, bs, q, sc) in enumerate(mats):
            C.coli_pack_fp8_int4(q8, bs, q, sc)
            evs[j + 1].record()
        torch.cuda.synchronize()
        for j in range(2):
            dur[j] += evs[j].elapsed_time(evs[j + 1]) / n_prof
    gu_bytes = mats[0][0].numel() * 1.5 + 4 * mats[0][3].numel() + 4 * mats[0][1].numel()
    achieved = gu_bytes / (dur[0] * 1e-3) / 1e9
    ms = 1e3 * elapsed / n_steps
    gbps = step_bytes / (ms * 1e-3) / 1e9
    workload = f"pack_fp8 layer H{H} I{I} experts{n_exp}"
    print(json.dumps({
        "metric": "FP8 e4m3 (128x128 block scales) -> int4 conversion of one layer's experts, "
                  "algorithmic HBM GB/s",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": n_steps,
        "warmup": n_warm, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8 e4m3 -> f32 -> int4",
        "data": "synthetic (seeded N(0, 64^2) rounded to e4m3, block scales 2^k * U(1, 2))",
        "config": {"workload": workload,
                   "launches_per_step": 2, "parallelism": "none (1 GPU)"},
        "kernel_avg_us": {"pack_fp8_gateup": round(dur[0] * 1e3, 1),
                          "pack_fp8_down": round(dur[1] * 1e3, 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "kernel": "k_pack_fp8_int4_wave (gate/up rows)",
                     "algorithmic_bytes": int(gu_bytes),
                     "traffic": TRAFFIC.get(("pack_fp8_gateup", workload))},
        "cpu_baseline": None,
    }), flush=True)


def read_ceiling_gbps(C, gib=4, reps=10):
    """Measured HBM streaming-read ceiling: coli_stream_read over a buffer far
    larger than the 256 MB last-level cache, HIP events on the launch stream."""
    import torch
    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(2):
        C.coli_stream_read(buf, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        C.coli_stream_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbps = buf.numel() / (ms * 1e-3) / 1e9
    del buf
    torch.cuda.empty_cache()
    return round(gbps, 1)


def gateup_roofline(kern, cfg, gate_up_bytes, T, bits=4):
    """Roofline of the gate/up kernel (the dominant launch of every path):
    algorithmic HBM bytes per launch / its mean event-timed duration, with the
    stored counter traffic of that kernel and workload where there is one."""
    gk = next((k for k in ("dec_gateup", "pf_gateup", "gateup") if k in kern), None)
    if gk is None:
        return None
    if gk == "dec_gateup":
        gate_up_bytes += 8 * T * cfg.n_experts  # the fp64 logits the kernel reads
    ms = kern[gk]
    wl = cfg.name + (f" int{bits} weights" if bits != 4 else "")
    ach = gate_up_bytes / (ms * 1e-3) / 1e9
    out = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
           "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
           "traffic": (int(TRAFFIC[(gk, wl)]) if (gk, wl) in TRAFFIC else None),
           "kernel": gk, "bytes_per_launch": int(gate_up_bytes),
           "avg_launch_us": round(ms * 1e3, 2)}
    if gk == "pf_gateup":
        # useful int8 ops of the launch: 2 per MAC over T*(K+S) (token, expert)
        # pairs x 2I rows x H
        ops = 2.0 * T * (cfg.top_k + cfg.n_shared) * 2 * cfg.inter * cfg.hidden
        out["int8_tops"] = round(ops / (ms * 1e-3) / 1e12, 1)
        out["int8_frac_of_5000_tops"] = round(ops / (ms * 1e-3) / 5.0e15, 4)
    return out


def run_sweep(args, cfg, counts):
    """Layer time against the number of tokens per call, on the weights and
    input recipe of `cfg` (the few-token kernels serve T <= 4, with int2
    weights T <= 2; the grouped MFMA kernels the rest)."""
    import torch

    import coli_synth as cs
    import int4_quantized_moe_sigmoid_amd as C

    H, I, E, K, S = cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.n_shared
    ng, tg = (int(v) for v in args.groups.split(",")) if args.groups else (1, 1)
    bits = args.bits
    lc = C.make_cfg(H, I, E, K, S, cfg.norm_topk, cfg.rho, ng, tg, bits)
    R = max(1, args.replicas)
    layers = [C.LayerWeights(lc, *cs.build_layer(
        cfg, r, "cuda", lambda w, qv, sv: C.coli_pack_weights(w, bits, qv, sv), bits=bits))
        for r in range(R)]
    Tmax = max(counts)
    ws = torch.empty(C.coli_moe_workspace_bytes(lc, Tmax), dtype=torch.uint8, device="cuda")
    lay_counts = None
    for T in counts:
        n_in = 16
        xs = []
        for i in range(n_in):
            raw = cs.activations(cs.with_tokens(cfg, T), i % R, "cuda", n_tok=T,
                                 first_tok=(i // R) * T)
            if cfg.rmsnorm_input:
                xn = torch.empty_like(raw)
                C.coli_rmsnorm(raw, xn, 1e-5)
                raw = xn
            xs.append(raw)
        y = torch.empty((T, H), dtype=torch.float32, device="cuda")
        for i in range(8):
            C.coli_moe_forward(layers[i % R], xs[i % n_in], y, ws)
        torch.cuda.synchronize()
        steps = max(20, min(args.steps, int(2e5 / (T + 20))))
        t0 = time.perf_counter()
        for i in range(steps):
            C.coli_moe_forward(layers[i % R], xs[i % n_in], y, ws)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        lay = C.coli_moe_workspace_layout(lc, T, 0)
        cnt = ws[lay.counts:lay.counts + 4 * (E + S)].view(torch.int32)
        uniq = int((cnt[:E] > 0).sum().item()) + S
        print(json.dumps({"sweep": cfg.name, "tokens": T, "us_per_call": round(dt * 1e6, 2),
                          "tokens_per_s": round(T / dt, 1), "experts_in_use": uniq,
                          "path": "few-token" if T <= (2 if bits == 2 else 4) else "grouped-mfma",
                          "weight_bits": bits,
                          "expert_weight_gbps": round(
                              uniq * (3 * I * H * bits // 8 + 4 * (2 * I + H)) / dt / 1e9, 1)}),
              flush=True)


def run_stack(args, cfg):
    """The stacked workload: x <- x + MoE_l(RMSNorm(x)) for every layer l, one
    step = all layers over one batch of T tokens."""
    import numpy as np
    import torch

    import coli_synth as cs
    import int4_quantized_moe_sigmoid_amd as C

    T, H, I, E, K, S = cfg.n_tok, cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.n_shared
    NL = cfg.n_layers
    bits = args.bits
    lc = C.make_cfg(H, I, E, K, S, cfg.norm_topk, cfg.rho, weight_bits=bits)
    n_steps, n_warm = args.steps, args.warmup
    t_setup = time.time()
    layers = []
    for l in range(NL):
        wr, b, q, s = cs.build_layer(cfg, l, "cuda",
                                     lambda w, qv, sv: C.coli_pack_weights(w, bits, qv, sv),
                                     bits=bits)
        layers.append(C.LayerWeights(lc, wr, b, q, s))
        print(f"[bench] layer {l} packed", file=sys.stderr, flush=True)
    xs = [cs.activations(cfg, 0, "cuda", n_tok=T, first_tok=i * T) for i in range(n_steps + n_warm)]
    xn = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(C.coli_moe_workspace_bytes(lc, T), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup

    def step(x):
        for l in range(NL):
            C.coli_rmsnorm(x, xn, 1e-5)
            C.coli_moe_forward(layers[l], xn, x, ws, C.COLI_FWD_ACCUM)

    for i in range(n_warm):
        step(xs[n_steps + i])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_steps):
        step(xs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / n_steps

    kern = {}
    uniq = []
    if not args.no_profile:
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(32)]  # 2 per launch
        for e in evs:
            e.record()
        torch.cuda.synchronize()
        hs = [e.cuda_event for e in evs]
        lay = C.coli_moe_workspace_layout(lc, T, 0)
        counts_view = ws[lay.counts:lay.counts + 4 * (E + S)].view(torch.int32)
        x = cs.activations(cfg, 0, "cuda", n_tok=T, first_tok=10 ** 6)
        for l in range(NL):
            C.coli_rmsnorm(x, xn, 1e-5)
            names = C.coli_moe_forward_profiled(layers[l], xn, x, ws, hs, C.COLI_FWD_ACCUM)
            torch.cuda.synchronize()
            for j in range(len(names)):
                kern[names[j]] = kern.get(names[j], 0.0) + \
                    evs[2 * j].elapsed_time(evs[2 * j + 1]) / NL
            uniq.append(int((counts_view[:E] > 0).sum().item()) + S)
    uniq_avg = float(np.mean(uniq)) if uniq else float(E + S)
    gate_up_bytes = uniq_avg * (2 * I * H * bits // 8 + 4 * 2 * I) + T * (H + H // 8) + \
        T * (K + S) * (I + I // 8)
    out = {
        "metric": "MoE-stack tokens/s (8 pre-norm residual MoE layers)",
        "value": round(T * n_steps / elapsed, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": n_steps, "warmup": n_warm, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"int{bits}xint8 (int32 block dots, f64 scales)",
        "data": "synthetic (seeded N(0,1) tokens, N(0,0.02) weights packed by coli_pack_weights)",
        "config": {"workload": cfg.name + (f" int{bits} weights" if bits != 4 else ""),
                   "tokens_per_step": T, "layers": NL, "hidden": H,
                   "inter": I, "n_experts": E, "top_k": K, "n_shared": S, "weight_bits": bits,
                   "parallelism": "none (1 GPU)"},
        "ms_per_layer": round(ms_per_step / NL, 4),
        "unique_experts_per_layer": round(uniq_avg, 2),
        "kernel_avg_us_per_layer": {k: round(v * 1e3, 2) for k, v in kern.items()},
        "roofline": gateup_roofline(kern, cfg, gate_up_bytes, T, bits),
        "cpu_baseline": None,
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(cfg, budget_s):
    """The oracle (plain C++ CPU reference, fp64) on a bounded sample of the
    same workload: tokens of replica 0, one forward per token, until the time
    budget is spent. Expert fp32 weights are drawn by coli_synth (on the GPU for
    speed; the draw is bit-identical to the CPU draw) and packed by the oracle."""
    import numpy as np
    import torch

    import coli_synth as cs
    import oracle

    H, I = cfg.hidden, cfg.inter
    wr, b = cs.router(cfg, 0, "cpu")
    wr, b = wr.numpy(), b.numpy()
    OL = oracle.OracleLayer(H, I, cfg.n_experts, cfg.top_k, cfg.n_shared, cfg.norm_topk,
                            cfg.rho, wr, b, {})
    timed = 0.0
    n_tok = 0
    while timed < budget_s and n_tok < 4096:
        x = cs.activations(cfg, 0, "cpu", n_tok=cfg.n_tok, first_tok=n_tok).numpy()
        if cfg.rmsnorm_input:
            x = oracle.rmsnorm(x, float(np.float32(1e-5)))
        idx, _, _ = oracle.route(x, wr, b, cfg.top_k, cfg.norm_topk, cfg.rho)
        need = set(int(e) for e in np.unique(idx)) | ({cfg.n_experts} if cfg.n_shared else set())
        for e in sorted(need - set(OL.experts)):
            OL.add_expert(e, oracle.pack_expert(*[cs.expert_matrix(cfg, 0, e, m, "cuda").cpu().numpy()
                                                  for m in ("gate", "up", "down")]))
        t0 = time.perf_counter()
        OL.forward(x)
        timed += time.perf_counter() - t0
        n_tok += cfg.n_tok
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")),
                             None)
    except OSError:
        pass
    return {"value": round(n_tok / timed, 4), "unit": "tokens/s", "cores": oracle.num_threads(),
            "cpu_model": cpu_model, "kind": "oracle",
            "sample": f"{n_tok} tokens of {cfg.name}, replica 0, one oracle forward per "
                      f"{cfg.n_tok} token(s), {timed:.1f} s timed"}


if __name__ == "__main__":
    main()
