#!/usr/bin/env python3
"""Throughput of one sigmoid-routed int4 x Q8_0 MoE layer on one MI355X.

Default run: the five synthetic workloads in one JSON line. The headline
(`value`) is the GLM-5.2-shaped decode at batch 1 (1 token per step, hidden
6144, 256 routed experts, top-8, one shared expert, intermediate 2048); a step
is one full coli_moe_forward: Q8_0(x), router + top-k, bucketing, gate/up +
SwiGLU + requant, down, weighted combine. Every step uses a new seeded token
and the next of R layer replicas (distinct seeded weights), so the 256 MB
Infinity Cache never serves a previous step's weights. `configs` holds the
same measurement for the tiny layer, MTP verify (3 correlated tokens),
prefill (512 tokens, zipf-skewed routing) and the 8-layer pre-norm residual
stack at 4096 tokens, each with its roofline and an oracle CPU baseline.

Options: --config N measures one workload alone (0 tiny, 1 decode, 2 MTP
verify T=3, 3 prefill T=512, 4 the stack); --gpus must be 1 (one GPU).
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

# int8 MFMA + exact int64 per-block epilogue at 2 waves per SIMD (the grouped
# gate/up kernel's occupancy), as a fraction of 5.0 POP/s: bench.py --op
# mfma_ceiling, profiles/mfma_epilogue_ceiling.txt
EPILOGUE_CEILING = 0.300

# HBM bytes per launch of the dominant kernel from rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE (two runs), scaled by what the counters read for a plain device
# copy of known size (FETCH_SIZE x 2, WRITE_SIZE x 1). Keyed by (kernel,
# workload as the JSON line names it); dropped whenever that kernel changes.
TRAFFIC = {
    # profiles/dec_kernels_decode_T1.txt
    ("dec_gateup", "decode T1 H6144 E256 K8 I2048"): (55669.1 * 2 + 38.4) * 1024,
    # profiles/dec_kernels_decode_T1_int8.txt, profiles/dec_kernels_decode_T1_int2.txt
    ("dec_gateup", "decode T1 H6144 E256 K8 I2048 int8 weights"): (111685.5 * 2 + 38.4) * 1024,
    ("dec_gateup", "decode T1 H6144 E256 K8 I2048 int2 weights"): (27999.9 * 2 + 38.4) * 1024,
    # profiles/dec_kernels_mtp_verify_T3.txt (mean over the counter run's steps)
    ("dec_gateup", "mtp-verify T3 correlated"): (95841.8 * 2 + 103.2) * 1024,
    # profiles/pf_kernels_prefill_T512.txt, profiles/pf_kernels_prefill_T512_int8.txt
    ("pf_gateup", "prefill T512 zipf-bias"): (1661012.2 * 2 + 14304.2) * 1024,
    ("pf_gateup", "prefill T512 zipf-bias int8 weights"): (3234193.0 * 2 + 13049.4) * 1024,
    # profiles/pf_kernels_stack_T4096.txt (k_pf32_gateup, per layer)
    ("pf_gateup", "stack8 T4096 uniform"): (2743552.1 * 2 + 96107.1) * 1024,
    # profiles/pack_fp8_int4_layer.txt (the gate/up launch)
    ("pack_fp8_gateup", "pack_fp8 layer H6144 I2048 experts257"): (3164334.8 * 2 + 3166240.7) * 1024,
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", type=int, default=None,
                    help="measure one workload alone (default: all five, decode as the headline)")
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="time budget of the headline's oracle CPU-baseline sample (the "
                         "other workloads take about half; 0 = skip every baseline)")
    ap.add_argument("--no-profile", action="store_true", help="skip the per-kernel event pass")
    ap.add_argument("--sweep", type=str, default="",
                    help="comma-separated token counts: time the layer of --config at each "
                         "(one JSON line per count) instead of the default run")
    ap.add_argument("--bits", type=int, default=4, choices=(2, 4, 8),
                    help="width of the expert weight codes (int8 and int2 run on the grouped "
                         "MFMA kernels at every token count)")
    ap.add_argument("--groups", type=str, default="",
                    help="NG,TG: group-limited expert selection (NG groups, the TG best kept)")
    ap.add_argument("--op", choices=("layer", "pack_fp8", "mfma_ceiling", "graph"),
                    default="layer",
                    help="pack_fp8: time the FP8 e4m3 (128 x 128 block scales) -> int4 "
                         "conversion of one layer's expert weights instead of the layer; "
                         "mfma_ceiling: issue rates of the int8 MFMA forms and of the exact "
                         "per-block epilogue (coli_mfma_probe)")
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

    import torch

    import coli_synth as cs
    import int4_quantized_moe_sigmoid_amd as C

    torch.cuda.set_device(0)
    if args.op == "pack_fp8":
        run_pack_fp8(args, cs.CONFIGS[1 if args.config is None else args.config])
        return
    if args.op == "mfma_ceiling":
        run_mfma_ceiling()
        return
    if args.op == "graph":
        run_graph_compare(args, cs.CONFIGS[1 if args.config is None else args.config])
        return
    if args.sweep:
        run_sweep(args, cs.CONFIGS[2 if args.config is None else args.config],
                  [int(v) for v in args.sweep.split(",") if v])
        return
    # the measured streaming-read ceiling first: it also brings the GPU out of idle
    ceiling = read_ceiling_gbps(C)
    if args.config is not None:
        cfg = cs.CONFIGS[args.config]
        res = measure_stack(args, cfg) if cfg.n_layers > 1 else measure_layer(args, cfg)
        print(json.dumps(headline(res, ceiling)), flush=True)
        return
    head = measure_layer(args, cs.CONFIGS[1])
    out = headline(head, ceiling)
    sub = {}
    half = argparse.Namespace(**{**vars(args), "cpu_seconds": args.cpu_seconds / 2})
    for cid in (0, 2, 3, 4):
        cfg = cs.CONFIGS[cid]
        res = measure_stack(half, cfg) if cfg.n_layers > 1 else measure_layer(half, cfg)
        sub[f"C{cid}"] = summary(res, ceiling)
        torch.cuda.empty_cache()
    out["configs"] = {"C1": summary(head, ceiling), **sub}
    print(json.dumps(out), flush=True)


def headline(res, ceiling):
    """The JSON line of one workload (the driver's fields first)."""
    out = {
        "metric": "MoE-layer tokens/s; decode int4 expert-weight GB/s as % of HBM peak",
        "value": res["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": res["steps"],
        "warmup": res["warmup"], "ms_per_step": res["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": res["dtype"],
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights packed by "
                "coli_pack_weights)",
        "config": res["config"],
        "read_ceiling_gbps": ceiling,
    }
    for k, v in res.items():
        if k not in out and k not in ("tokens_per_s", "steps", "warmup"):
            out[k] = v
    if "expert_weight_gbps" in res:
        out["expert_weight_frac_read_ceiling"] = round(res["expert_weight_gbps"] / ceiling, 4)
    if out.get("roofline") and out["roofline"]["unit"] == "GB/s":
        out["roofline"]["frac_of_read_ceiling"] = round(out["roofline"]["achieved"] / ceiling, 4)
    return out


def summary(res, ceiling):
    """Per-workload entry of the default line."""
    keep = ("config", "ms_per_step", "ms_per_layer", "tokens_per_s", "steps", "warmup",
            "expert_weight_gbps", "expert_weight_frac_hbm", "unique_experts_per_step",
            "unique_experts_per_layer", "algorithmic_bytes_per_step", "kernel_avg_us",
            "kernel_avg_us_per_layer", "roofline", "cpu_baseline")
    out = {k: res[k] for k in keep if k in res}
    if out.get("roofline") and out["roofline"]["unit"] == "GB/s":
        out["roofline"]["frac_of_read_ceiling"] = round(out["roofline"]["achieved"] / ceiling, 4)
    return out


def kernel_events(C, run_profiled, n_prof):
    """Mean duration (ms) of each launch of a forward, from the launches' own
    start and stop HIP events (coli_moe_forward_profiled; the events are
    stamped by the packet processor on the launch stream). run_profiled(i,
    handles) enqueues forward i and returns its launch names."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(40)]  # 2 per launch
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    hs = [e.cuda_event for e in evs]
    sums = {}
    for i in range(n_prof):
        names = run_profiled(i, hs)
        torch.cuda.synchronize()
        for j, nm in enumerate(names):
            sums[nm] = sums.get(nm, 0.0) + evs[2 * j].elapsed_time(evs[2 * j + 1])
    return {k: v / n_prof for k, v in sums.items()}


def measure_layer(args, cfg):
    """One MoE layer per step over a new seeded batch of cfg.n_tok tokens, the
    layer taken round robin from R independently seeded replicas."""
    import numpy as np
    import torch

    import coli_synth as cs
    import int4_quantized_moe_sigmoid_amd as C

    T, H, I, E, K, S = cfg.n_tok, cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.n_shared
    ng, tg = (int(v) for v in args.groups.split(",")) if args.groups else (1, 1)
    bits = args.bits
    lc = C.make_cfg(H, I, E, K, S, cfg.norm_topk, cfg.rho, ng, tg, bits)
    # every step reads a different set of experts; a layer whose experts all fit
    # the 256 MB last-level cache or that reads them all every step (prefill)
    # needs no replicas
    R = max(1, args.replicas) if T < 64 and E * cfg.expert_bytes() > (1 << 28) else 1
    n_steps, n_warm = args.steps, args.warmup
    n_inputs = n_steps + n_warm

    t_setup = time.time()
    pack = lambda w, qv, sv: C.coli_pack_weights(w, bits, qv, sv)
    layers = []
    for r in range(R):
        wr, b, q, s = cs.build_layer(cfg, r, "cuda", pack, bits=bits)
        layers.append(C.LayerWeights(lc, wr, b, q, s))
        print(f"[bench] {cfg.name}: replica {r} packed ({(q.numel() + 4 * s.numel()) / 1e9:.2f} GB)",
              file=sys.stderr, flush=True)
    # distinct seeded inputs for every step, RMS-normalised on the GPU when the
    # workload's input is normalised
    xs = []
    for i in range(n_inputs if T * H * n_inputs < (1 << 28) else 2 * R):
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
        C.coli_moe_forward(layers[i % R], xs[i % len(xs)], ys[i & 1], ws)

    for i in range(n_warm):
        step(n_steps + i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / n_steps

    # ---- per-kernel durations with HIP events on the launch stream -----------
    lay = C.coli_moe_workspace_layout(lc, T, 0)
    counts_view = ws[lay.counts:lay.counts + 4 * (E + S)].view(torch.int32)
    kern, unique_counts = {}, []
    if not args.no_profile:
        def prof(i, hs):
            names = C.coli_moe_forward_profiled(layers[i % R], xs[i % len(xs)], ys[i & 1], ws,
                                                hs)
            torch.cuda.synchronize()
            unique_counts.append(int((counts_view[:E] > 0).sum().item()) + S)
            return names
        kern = kernel_events(C, prof, max(1, min(n_steps, 200)))
    uniq_avg = float(np.mean(unique_counts)) if unique_counts else float(min(E, T * K) + S)

    # bytes that must cross HBM per step: unique experts' packed weights + scales,
    # the router weight, activations in and out
    eb = 3 * I * H * bits // 8 + 4 * (2 * I + H)
    # algorithmic HBM bytes of the gate/up launch: the packed gate and up rows and
    # their scales of every expert in use, Q8_0(x) in, Q8_0(h) out
    gate_up_bytes = uniq_avg * (2 * I * H * bits // 8 + 4 * 2 * I) + T * (H + H // 8) + \
        T * (K + S) * (I + I // 8)
    step_bytes = uniq_avg * eb + 4 * E * H + 4 * E + 8 * T * H
    weight_gbps = uniq_avg * eb / (ms_per_step * 1e-3) / 1e9
    cpu = cpu_baseline(cfg, args.cpu_seconds) if args.cpu_seconds > 0 else None
    wl = cfg.name + (f" groups {ng}/{tg}" if ng > 1 else "") + \
        (f" int{bits} weights" if bits != 4 else "")
    res = {
        "config": {"workload": wl, "tokens_per_step": T, "hidden": H, "inter": I,
                   "n_experts": E, "top_k": K, "n_shared": S, "weight_replicas": R,
                   "n_group": ng, "topk_group": tg, "weight_bits": bits,
                   "parallelism": "none (1 GPU)"},
        "dtype": f"int{bits}xint8 (int32 block dots, f64 scales)",
        "steps": n_steps, "warmup": n_warm,
        "ms_per_step": round(ms_per_step, 5),
        "tokens_per_s": round(T * n_steps / elapsed, 2),
        "expert_weight_gbps": round(weight_gbps, 1),
        "expert_weight_frac_hbm": round(weight_gbps / HBM_PEAK_GBPS, 4),
        "unique_experts_per_step": round(uniq_avg, 2),
        "algorithmic_bytes_per_step": int(step_bytes),
        "kernel_avg_us": {k: round(v * 1e3, 2) for k, v in kern.items()},
        "roofline": gateup_roofline(kern, cfg, wl, gate_up_bytes, T, mfma_bound=False),
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    del layers, xs, ws
    return res


def measure_stack(args, cfg):
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
        print(f"[bench] {cfg.name}: layer {l} packed", file=sys.stderr, flush=True)
    # distinct seeded batches (up to 32, then reused: each step adds its layers'
    # outputs into its batch in place, as the residual stream does)
    xs = [cs.activations(cfg, 0, "cuda", n_tok=T, first_tok=i * T)
          for i in range(min(32, n_steps + n_warm))]
    xn = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(C.coli_moe_workspace_bytes(lc, T), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup

    def step(i):
        x = xs[i % len(xs)]
        for l in range(NL):
            C.coli_rmsnorm(x, xn, 1e-5)
            C.coli_moe_forward(layers[l], xn, x, ws, C.COLI_FWD_ACCUM)

    for i in range(n_warm):
        step(n_steps + i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / n_steps

    kern = {}
    uniq = []
    x = cs.activations(cfg, 0, "cuda", n_tok=T, first_tok=10 ** 6)
    if not args.no_profile:
        lay = C.coli_moe_workspace_layout(lc, T, 0)
        counts_view = ws[lay.counts:lay.counts + 4 * (E + S)].view(torch.int32)

        def prof(l, hs):
            C.coli_rmsnorm(x, xn, 1e-5)
            names = C.coli_moe_forward_profiled(layers[l], xn, x, ws, hs, C.COLI_FWD_ACCUM)
            torch.cuda.synchronize()
            uniq.append(int((counts_view[:E] > 0).sum().item()) + S)
            return names
        kern = kernel_events(C, prof, NL)
    uniq_avg = float(np.mean(uniq)) if uniq else float(E + S)
    gate_up_bytes = uniq_avg * (2 * I * H * bits // 8 + 4 * 2 * I) + T * (H + H // 8) + \
        T * (K + S) * (I + I // 8)
    cpu = cpu_baseline_stack(cfg, args.cpu_seconds) if args.cpu_seconds > 0 else None
    wl = cfg.name + (f" int{bits} weights" if bits != 4 else "")
    res = {
        "metric_note": "MoE-stack tokens/s (8 pre-norm residual MoE layers per step)",
        "config": {"workload": wl, "tokens_per_step": T, "layers": NL, "hidden": H,
                   "inter": I, "n_experts": E, "top_k": K, "n_shared": S, "weight_bits": bits,
                   "parallelism": "none (1 GPU)"},
        "dtype": f"int{bits}xint8 (int32 block dots, f64 scales)",
        "steps": n_steps, "warmup": n_warm,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_layer": round(ms_per_step / NL, 4),
        "tokens_per_s": round(T * n_steps / elapsed, 2),
        "unique_experts_per_layer": round(uniq_avg, 2),
        "kernel_avg_us_per_layer": {k: round(v * 1e3, 2) for k, v in kern.items()},
        "roofline": gateup_roofline(kern, cfg, wl, gate_up_bytes, T, mfma_bound=True),
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    del layers, ws
    return res


def gateup_roofline(kern, cfg, wl, gate_up_bytes, T, mfma_bound):
    """Roofline of the gate/up kernel (the dominant launch of every path):
    algorithmic HBM bytes per launch / its mean event-timed duration against
    8 TB/s, with the stored counter traffic of that kernel and workload where
    there is one; for the grouped MFMA kernel also the useful int8 ops (2 per
    MAC over T*(K+S) (token, expert) pairs x 2I rows x H) against 5.0 POP/s.
    mfma_bound: the stacked workload sits at the ridge and is reported against
    the int8 MFMA peak."""
    gk = next((k for k in ("dec_gateup", "pf_gateup", "gateup") if k in kern), None)
    if gk is None:
        return None
    if gk == "dec_gateup":
        # the fp64 sigmoid and selection scores (two per expert) the kernel reads
        gate_up_bytes += 16 * T * cfg.n_experts
    ms = kern[gk]
    ach = gate_up_bytes / (ms * 1e-3) / 1e9
    traffic = TRAFFIC.get((gk, wl))
    out = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
           "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
           "traffic": (int(traffic) if traffic is not None else None),
           "kernel": gk, "bytes_per_launch": int(gate_up_bytes),
           "avg_launch_us": round(ms * 1e3, 2)}
    if gk == "pf_gateup":
        ops = 2.0 * T * (cfg.top_k + cfg.n_shared) * 2 * cfg.inter * cfg.hidden
        tops = ops / (ms * 1e-3) / 1e12
        out["int8_tops"] = round(tops, 1)
        out["int8_frac_of_5000_tops"] = round(tops / 5000.0, 4)
        if mfma_bound:
            out = {"bound": "mfma", "achieved": round(tops, 1), "peak": 5000.0,
                   "unit": "TOP/s (int8)", "frac": round(tops / 5000.0, 4),
                   "traffic": out["traffic"], "kernel": gk, "int8_ops_per_launch": ops,
                   "hbm_gbps": round(ach, 1), "hbm_frac": round(ach / HBM_PEAK_GBPS, 4),
                   "bytes_per_launch": int(gate_up_bytes), "avg_launch_us": round(ms * 1e3, 2),
                   "epilogue_ceiling_frac": EPILOGUE_CEILING,
                   "frac_of_epilogue_ceiling": round(tops / 5000.0 / EPILOGUE_CEILING, 4)}
    return out


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
        "cpu_baseline": (cpu_baseline_pack_fp8(mats[0][0], mats[0][1], args.cpu_seconds)
                         if args.cpu_seconds > 0 else None),
    }), flush=True)


def cpu_baseline_pack_fp8(q8, bs, budget_s, rows=1024):
    """The oracle's FP8 -> int4 conversion on a bounded sample of the same
    workload: consecutive 1024-row chunks (whole 128-row scale blocks) of the
    gate/up matrix, copied to the host untimed, until the time budget is spent;
    the rate counts the same algorithmic bytes as the GPU figure."""
    import oracle
    timed, done, r0, chunks = 0.0, 0, 0, 0
    n_rows, cols = q8.shape
    while timed < budget_s and r0 < n_rows:
        r1 = min(n_rows, r0 + rows)
        qh = q8[r0:r1].cpu().numpy()
        bh = bs[r0 // 128:(r1 + 127) // 128].cpu().numpy()
        t0 = time.perf_counter()
        oracle.pack_fp8_int4(qh, bh)
        timed += time.perf_counter() - t0
        done += r1 - r0
        chunks += 1
        r0 = r1
    nbytes = done * cols * 1.5 + 4 * done + 4 * ((done + 127) // 128) * ((cols + 127) // 128)
    return {"value": round(nbytes / timed / 1e9, 3), "unit": "GB/s", "cores": oracle.num_threads(),
            "cpu_model": _cpu_model(), "kind": "oracle",
            "sample": f"{done} gate/up rows of {cols} codes ({chunks} chunks of up to {rows} "
                      f"rows), {timed:.1f} s timed"}


def run_mfma_ceiling():
    """Issue rates of the int8 MFMA forms and of the exact per-block epilogue
    (coli_mfma_probe) at 1, 2 and 4 waves per SIMD (256 x 1, 2, 4 workgroups
    of 4 waves), one JSON line per mix: shader-clock cycles per loop
    iteration per wave, and the int8 rate against 5.0 POP/s from the launch's
    event time. The epilogue mixes bound the grouped kernels: every MFMA
    result needs one scaled add per 32-block."""
    import torch

    import int4_quantized_moe_sigmoid_amd as C
    mixes = {0: ("8 x mfma_i32_16x16x32_i8", 8 * 16384), 1: ("8 x mfma_i32_16x16x64_i8", 8 * 32768),
             2: ("4 x mfma_i32_32x32x32_i8", 4 * 65536), 3: ("16 x v_mad_i64_i32", 0),
             4: ("16 x (v_cvt_f64_i32 + v_fma_f64)", 0),
             5: ("2 x 32x32x32 + int64 epilogue (32 v_mad_i64_i32)", 2 * 65536),
             6: ("2 x 32x32x32 + fp64 epilogue (32 cvt + 32 fma)", 2 * 65536),
             7: ("4 x 16x16x32 + int64 epilogue (16 v_mad_i64_i32)", 4 * 16384)}
    iters = 4000
    for wpc in (1, 2, 4):
        nwg = 256 * wpc
        cyc = torch.zeros(4 * nwg + 1, dtype=torch.int64, device="cuda")
        for kind, (name, ops) in mixes.items():
            C.coli_mfma_probe(kind, nwg, iters, cyc)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            C.coli_mfma_probe(kind, nwg, iters, cyc)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            per_it = float(cyc[:4 * nwg].double().mean().item()) / iters
            tops = ops * iters * nwg * 4 / (ms * 1e-3) / 1e12
            print(json.dumps({"probe": name, "waves_per_simd": wpc,
                              "cycles_per_iter_per_wave": round(per_it, 1),
                              "int8_tops": round(tops, 1),
                              "int8_frac_of_5000_tops": round(tops / 5000.0, 4),
                              "ms": round(ms, 3)}), flush=True)


def run_graph_compare(args, cfg, per_graph=8):
    """Layer steps launched one by one against replays of a HIP graph that
    holds `per_graph` of them (captured from the same calls, replicas round
    robin): whether launching from a graph shortens the gaps between the
    layer's data-dependent launches. Every replay is checked bit for bit
    against the eager results, with eager work and synchronisations between
    replays. Prints one JSON line per mode and round."""
    import torch

    import coli_synth as cs
    import int4_quantized_moe_sigmoid_amd as C

    T, H = cfg.n_tok, cfg.hidden
    lc = C.make_cfg(H, cfg.inter, cfg.n_experts, cfg.top_k, cfg.n_shared, cfg.norm_topk,
                    cfg.rho, 1, 1, 4)
    R = max(1, args.replicas) if T < 64 and cfg.n_experts * cfg.expert_bytes() > (1 << 28) else 1
    pack = lambda w, qv, sv: C.coli_pack_weights(w, 4, qv, sv)
    layers = []
    for r in range(R):
        wr, b, q, s = cs.build_layer(cfg, r, "cuda", pack, bits=4)
        layers.append(C.LayerWeights(lc, wr, b, q, s))
    xs = []
    for i in range(per_graph):
        raw = cs.activations(cfg, i % R, "cuda", n_tok=T, first_tok=(i // R) * T)
        if cfg.rmsnorm_input:
            xn = torch.empty_like(raw)
            C.coli_rmsnorm(raw, xn, 1e-5)
            raw = xn
        xs.append(raw)
    ys = [torch.empty((T, H), dtype=torch.float32, device="cuda") for _ in range(per_graph)]
    ws = torch.empty(C.coli_moe_workspace_bytes(lc, T), dtype=torch.uint8, device="cuda")

    def eager():
        for j in range(per_graph):
            C.coli_moe_forward(layers[j % R], xs[j], ys[j], ws)

    eager()
    torch.cuda.synchronize()
    ref = [y.clone() for y in ys]
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        eager()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        eager()
    torch.cuda.synchronize()
    for rep in range(3):
        for y in ys:
            y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if not all(torch.equal(a, b) for a, b in zip(ys, ref)):
            raise RuntimeError(f"graph replay {rep} differs from the eager forward")
        eager()
        torch.cuda.synchronize()
    rounds = max(1, args.steps // per_graph)
    for k in range(2):
        for mode in ("eager", "graph"):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(rounds):
                if mode == "eager":
                    eager()
                else:
                    g.replay()
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
            print(json.dumps({"op": "graph", "workload": cfg.name, "mode": mode, "round": k,
                              "steps": rounds * per_graph,
                              "us_per_step": round(1e6 * dt / (rounds * per_graph), 2),
                              "replays_checked": 3}), flush=True)


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


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            return next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")),
                        None)
    except OSError:
        return None


def _oracle_layer(cfg, layer, x, OL=None):
    """Oracle layer (from coli_synth's fp32 draws, packed by the oracle) holding
    the experts tokens x select plus the shared expert."""
    import numpy as np

    import coli_synth as cs
    import oracle
    wr, b = cs.router(cfg, layer, "cpu")
    wr, b = wr.numpy(), b.numpy()
    if OL is None:
        OL = oracle.OracleLayer(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.n_shared,
                                cfg.norm_topk, cfg.rho, wr, b, {})
    idx, _, _ = oracle.route(x, wr, b, cfg.top_k, cfg.norm_topk, cfg.rho)
    need = set(int(e) for e in np.unique(idx)) | ({cfg.n_experts} if cfg.n_shared else set())
    for e in sorted(need - set(OL.experts)):
        OL.add_expert(e, oracle.pack_expert(*[cs.expert_matrix(cfg, layer, e, m, "cuda").cpu()
                                              .numpy() for m in ("gate", "up", "down")]))
    return OL


def cpu_baseline(cfg, budget_s):
    """The oracle (plain C++ CPU reference, fp64) on a bounded sample of the
    same workload: batches of cfg.n_tok tokens of replica 0 (at most 32 tokens
    per forward), until the time budget is spent. Expert fp32 weights are drawn
    by coli_synth (on the GPU for speed; the draw is bit-identical to the CPU
    draw) and packed by the oracle; drawing and packing are not timed."""
    import numpy as np

    import coli_synth as cs
    import oracle

    B = min(cfg.n_tok, 32)
    timed, n_tok = 0.0, 0
    OL = None
    while timed < budget_s and n_tok < 4096:
        x = cs.activations(cfg, 0, "cpu", n_tok=B, first_tok=n_tok).numpy()
        if cfg.rmsnorm_input:
            x = oracle.rmsnorm(x, float(np.float32(1e-5)))
        OL = _oracle_layer(cfg, 0, x, OL)
        t0 = time.perf_counter()
        OL.forward(x)
        timed += time.perf_counter() - t0
        n_tok += B
    part = "" if B == cfg.n_tok else f" (a {B}-token part of each {cfg.n_tok}-token batch)"
    return {"value": round(n_tok / timed, 4), "unit": "tokens/s", "cores": oracle.num_threads(),
            "cpu_model": _cpu_model(), "kind": "oracle",
            "sample": f"{n_tok} tokens of {cfg.name}{part}, replica 0, {B} token(s) per oracle "
                      f"forward, {timed:.1f} s timed"}


def cpu_baseline_stack(cfg, budget_s):
    """The oracle on a bounded sample of the stacked workload: layer 0 only, on
    batches of 32 RMS-normalised tokens of the stack's input, until the time
    budget is spent; the stack's rate is that layer rate divided by the number
    of layers (every layer has the same shape and the same per-token work)."""
    import numpy as np

    import coli_synth as cs
    import oracle

    B = 32
    timed, n_tok = 0.0, 0
    OL = None
    while timed < budget_s and n_tok < cfg.n_tok:
        x = cs.activations(cfg, 0, "cpu", n_tok=B, first_tok=n_tok).numpy()
        xn = oracle.rmsnorm(x, float(np.float32(1e-5)))
        OL = _oracle_layer(cfg, 0, xn, OL)
        t0 = time.perf_counter()
        OL.forward(xn, y_in=x)
        timed += time.perf_counter() - t0
        n_tok += B
    return {"value": round(n_tok / timed / cfg.n_layers, 4), "unit": "tokens/s",
            "cores": oracle.num_threads(), "cpu_model": _cpu_model(), "kind": "oracle",
            "sample": f"layer 0 of {cfg.name} on {n_tok} tokens ({B} per oracle forward, "
                      f"RMSNorm + residual), {timed:.1f} s timed; stack rate = layer rate / "
                      f"{cfg.n_layers}"}


if __name__ == "__main__":
    main()
