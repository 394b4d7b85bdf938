#!/usr/bin/env python3
"""Benchmark of the dual-path outlier-separated GEMM on one MI355X.

    python bench.py [--steps K] [--warmup W] [--sweep] [--no-cpu]

Workload: the Llama-3-70B-shaped prefill linears (M = 4096 tokens;
8192->8192, 8192->28672, 28672->8192) at outlier fraction 1/16, bf16 input
activations, bf16 outlier branch, seeded synthetic data (no model weights or
datasets exist here).  Channel selection and weight packing are offline and
run once before timing.  One step = for each of the three layers: the online
activation quantise/split kernel, then the fused dual GEMM -- every online
step of the path, inputs resident in HBM.

Prints ONE JSON line.  ``value`` is effective TOPS = sum(2*M*N*K) / step
time.  ``roofline`` describes the dominant kernel (the dual GEMM): achieved
algorithmic ops (2*M*N*K per launch) / its average launch time measured with
HIP events on the stream it runs on, against the int8 MFMA peak;
``traffic`` is HBM bytes per GEMM launch from the committed rocprofv3
counter summary, or null if the kernel source changed since it was taken.
``cpu_baseline`` times the scalar CPU oracle on a bounded row sample of the
same step.  ``--sweep`` adds the outlier-fraction sweep (1/2 ... 1/16).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dual-path W4A4+outlier GEMM effective TOPS and % of int8 MFMA peak, 1 GPU"
PEAK_INT8_TOPS = 5000.0  # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
GEMM_SOURCES = ["outlier_split_mixed_amd/csrc/k_gemm.hip", "outlier_split_mixed_amd/csrc/sqf_device.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_k_dual_gemm_llama3_70b_f16.txt")


def kernel_sha() -> str:
    h = hashlib.sha256()
    for p in GEMM_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per GEMM launch from the committed counter summary, if it was
    taken on the current kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_sha") != kernel_sha():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def dual_bound_frac(k_low, k_out):
    """Largest share of the int8 peak the dual path can reach when the bf16
    branch runs at half the int8 rate: K / (K_low + 2 K_out)."""
    return (k_low + k_out) / (k_low + 2.0 * k_out)


class LayerRun:
    def __init__(self, sqf, torch, lay, k_out, stream):
        self.lay = lay
        self.m, self.k, self.n, self.k_out = lay.m, lay.k, lay.n, k_out
        with torch.cuda.stream(stream):
            x_cal = torch.from_numpy(lay.x_cal).cuda()
            w = torch.from_numpy(lay.w).cuda()
            _, self.map, _, _ = sqf.sqf_select_channels(x_cal, w, k_out, stream=stream)
            self.w = sqf.sqf_pack_weights(w, self.map, stream=stream)
            from outlier_split_mixed_amd import synth

            bits = synth.to_bf16_bits(lay.x)
            self.x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
            self.acts = sqf.alloc_acts(lay.m, lay.k - k_out, k_out)
            self.y = torch.empty((lay.m, lay.n), dtype=torch.float32, device="cuda")
            self.yb = None  # bf16 Y buffer when the step writes bf16
            del w, x_cal
        stream.synchronize()
        self.sqf = sqf

    def step(self, stream, ev=None):
        if ev is not None:
            ev[0].record(stream)
        self.sqf.sqf_quantize_split_act(self.x, self.map, self.acts, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        if self.yb is None:
            self.sqf.sqf_dual_gemm(self.acts, self.w, y=self.y, stream=stream)
        else:
            self.sqf.sqf_dual_gemm(self.acts, self.w, y=self.yb, stream=stream, y_dtype="bf16")
        if ev is not None:
            ev[2].record(stream)

    @property
    def ops(self):
        return 2.0 * self.m * self.n * self.k

    @property
    def act_bytes(self):
        a = self.acts
        return self.m * (self.k * 2 + a.ldk + a.ldo * 2 + 4) + self.k * 4


def time_layers(torch, runs, stream, steps, warmup):
    for _ in range(warmup):
        for r in runs:
            r.step(stream)
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in runs]
           for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for s in range(steps):
        for i, r in enumerate(runs):
            r.step(stream, evs[s][i])
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    act_ms = np.zeros(len(runs))
    gemm_ms = np.zeros(len(runs))
    for s in range(steps):
        for i in range(len(runs)):
            e = evs[s][i]
            act_ms[i] += e[0].elapsed_time(e[1])
            gemm_ms[i] += e[1].elapsed_time(e[2])
    return total_ms / steps, act_ms / steps, gemm_ms / steps


def cpu_baseline(runs, rows_per_layer):
    """The oracle (untuned) on a bounded sample of the same step: the online
    stages (activation quantise/split + dual GEMM) for `rows_per_layer` token
    rows of each layer.  Offline packing is outside the step, as on the GPU."""
    import oracle
    from outlier_split_mixed_amd import synth

    total_ops, total_s = 0.0, 0.0
    for r in runs:
        lay = r.lay
        _, o_mp, _, _ = oracle.select_channels(lay.x_cal, lay.w, r.k_out)
        o_w = oracle.pack_weights(lay.w, o_mp)
        xs = synth.to_bf16_bits(lay.x[:rows_per_layer])
        t = time.perf_counter()
        o_a = oracle.quantize_split_act(xs, o_mp, x_fmt="bf16")
        oracle.dual_gemm(o_a, o_w)
        total_s += time.perf_counter() - t
        total_ops += 2.0 * rows_per_layer * r.n * r.k
    return dict(value=round(total_ops / total_s / 1e12, 6), unit="TOPS", cores=oracle.num_threads(),
                kind="oracle",
                sample=f"{rows_per_layer} token rows x all outputs of each of the 3 layers "
                       f"(act quantise/split + dual GEMM), {total_s:.1f} s")


def time_call(torch, stream, fn, iters=10, warmup=2):
    """Average time (ms) of fn() on `stream`, measured with events on that stream."""
    for _ in range(warmup):
        fn()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(iters):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def rows_section(sqf, torch, stream):
    """Every hot-path row on its own workload, each against its roofline:
    offline selection and packing (timed once), the activation split
    (HBM-bound), the grouped MoE expert path (HBM-bound: the fp32 outputs
    dominate its bytes) and the weight-side SQ-format GEMM (MFMA-bound: the
    low and the masked pass are two int8 passes over K_low, plus the int8
    branch)."""
    from outlier_split_mixed_amd import synth

    out = []
    with torch.cuda.stream(stream):
        # a0/a1 offline, on the widest layer of the step
        lay = synth.llama3_70b(1, 16)
        x_cal = torch.from_numpy(lay.x_cal).cuda()
        w = torch.from_numpy(lay.w).cuda()
        k_out = lay.k // 16
        t = time_call(torch, stream, lambda: sqf.sqf_select_channels(x_cal, w, k_out, stream=stream),
                      iters=3, warmup=1)
        _, mp, _, _ = sqf.sqf_select_channels(x_cal, w, k_out, stream=stream)
        # algorithmic bytes: x_cal and W read once, scores / hdiag / map / idx written
        b0 = 4 * lay.x_cal.size + 4 * lay.k * lay.n + (8 + 4 + 4) * lay.k + 4 * k_out
        out.append(dict(row="a0 select (offline)", shape=f"{lay.k}x{lay.n}, {lay.x_cal.shape[0]} cal rows",
                        ms=round(t, 3), gbs=round(b0 / t / 1e6, 1), frac_hbm=round(b0 / t / 1e6 / PEAK_HBM_GBS, 3)))
        t = time_call(torch, stream, lambda: sqf.sqf_pack_weights(w, mp, stream=stream), iters=3, warmup=1)
        # W and the map read once; int4 rows, bf16 branch rows and scales written
        ldk = sqf.sqf_pad_k_low(lay.k - k_out) // 2
        ldo = sqf.sqf_pad_k_out(k_out, "bf16")
        b1 = 4 * lay.k * lay.n + 4 * lay.k + lay.n * (ldk + 2 * ldo + 4)
        out.append(dict(row="a1 pack (offline)", shape=f"{lay.k}x{lay.n}", ms=round(t, 3),
                        gbs=round(b1 / t / 1e6, 1), frac_hbm=round(b1 / t / 1e6 / PEAK_HBM_GBS, 3)))
        del w, x_cal, mp
        torch.cuda.empty_cache()

        # a6: grouped experts (Qwen3-30B-A3B-shaped)
        moe = synth.qwen3_moe()
        ro = torch.from_numpy(moe.offsets).cuda()
        rows = int(moe.offsets[-1])
        for name, lays, br in (("up", moe.up, "bf16"), ("down", moe.down, "bf16"),
                               ("down", moe.down, "fp8")):
            k, n, ko = lays[0].k, lays[0].n, lays[0].k_out
            maps = torch.stack([sqf.sqf_select_channels(torch.from_numpy(l.x_cal).cuda(),
                                                        torch.from_numpy(l.w).cuda(), ko,
                                                        stream=stream)[1] for l in lays])
            wt = sqf.sqf_pack_weights(torch.from_numpy(np.stack([l.w for l in lays])).cuda(), maps,
                                      branch=br, stream=stream)
            xt = torch.from_numpy(synth.to_bf16_bits(np.concatenate([l.x for l in lays])).view(np.int16))
            xt = xt.view(torch.bfloat16).cuda()
            a = sqf.alloc_acts(rows, k - ko, ko, branch=br)
            y = torch.empty((rows, n), dtype=torch.float32, device="cuda")
            ta = time_call(torch, stream, lambda: sqf.sqf_quantize_split_act_grouped(
                xt, ro, maps, a, stream=stream))
            tg = time_call(torch, stream, lambda: sqf.sqf_dual_gemm_grouped(a, wt, ro, y=y, stream=stream))
            esz = 2 if br == "bf16" else 1
            act_b = rows * (k * 2 + a.ldk + a.ldo * esz + 4)
            gemm_b = rows * (a.ldk + a.ldo * esz + 8) + len(lays) * n * (a.ldk + a.ldo * esz + 8) + rows * n * 4
            out.append(dict(row=f"a6 grouped {name} ({br} branch)",
                            shape=f"{len(lays)} experts, {rows} rows, {k}->{n}, k_out {ko}",
                            act_us=round(ta * 1e3, 1),
                            act_frac_hbm=round(act_b / (ta * 1e-3) / 1e9 / PEAK_HBM_GBS, 3),
                            gemm_us=round(tg * 1e3, 1),
                            gemm_tops=round(2.0 * rows * n * k / (tg * 1e-3) / 1e12, 1),
                            gemm_gbs=round(gemm_b / (tg * 1e-3) / 1e9, 1),
                            gemm_frac_hbm=round(gemm_b / (tg * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)))
            # the same GEMM writing bf16 Y (half the output bytes)
            yb = torch.empty((rows, n), dtype=torch.bfloat16, device="cuda")
            tb = time_call(torch, stream, lambda: sqf.sqf_dual_gemm_grouped(a, wt, ro, y=yb, stream=stream,
                                                                           y_dtype="bf16"))
            gemm_bb = gemm_b - rows * n * 2
            out[-1].update(gemm_bf16y_us=round(tb * 1e3, 1),
                           gemm_bf16y_frac_hbm=round(gemm_bb / (tb * 1e-3) / 1e9 / PEAK_HBM_GBS, 3))
            del wt, xt, a, y, yb, maps
            torch.cuda.empty_cache()
        del moe

        # a7: SQ-format weight side
        lay = synth.sq_weight()
        k_out = lay.k_out
        k_low = lay.k - k_out
        x_cal = torch.from_numpy(lay.x_cal).cuda()
        w = torch.from_numpy(lay.w).cuda()
        _, mp, _, hd = sqf.sqf_select_channels(x_cal, w, k_out, stream=stream)
        wt = sqf.sqf_pack_weights(w, mp, branch="i8", hdiag=hd, sq_nnz=k_low // 8, stream=stream)
        xt = torch.from_numpy(synth.to_bf16_bits(lay.x).view(np.int16)).view(torch.bfloat16).cuda()
        a = sqf.alloc_acts(lay.m, k_low, k_out, low="i8", branch="i8")
        y = torch.empty((lay.m, lay.n), dtype=torch.float32, device="cuda")
        ta = time_call(torch, stream, lambda: sqf.sqf_quantize_split_act(xt, mp, a, stream=stream))
        tg = time_call(torch, stream, lambda: sqf.sqf_dual_gemm(a, wt, y=y, stream=stream), iters=5)
        mfma_ops = 2.0 * lay.m * lay.n * (2 * k_low + k_out)
        out.append(dict(row="a7 SQ-format weight side (int8 acts, masked int8 part, int8 branch)",
                        shape=f"{lay.m}x{lay.k}->{lay.n}, nnz {k_low // 8}/row",
                        act_us=round(ta * 1e3, 1), gemm_us=round(tg * 1e3, 1),
                        gemm_eff_tops=round(2.0 * lay.m * lay.n * lay.k / (tg * 1e-3) / 1e12, 1),
                        mfma_tops=round(mfma_ops / (tg * 1e-3) / 1e12, 1),
                        frac_int8_peak=round(mfma_ops / (tg * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4)))
        del wt, xt, a, y, w, x_cal
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sweep", action="store_true", help="also time outlier fractions 1/2..1/16")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=128)
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the per-row section (offline steps, grouped experts, SQ-format)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after timing, copy a buffer of this many bytes (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this path runs without sharding or collectives "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import torch

    from outlier_split_mixed_amd import sqf, synth

    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    t_setup = time.time()
    runs = [LayerRun(sqf, torch, synth.llama3_70b(i, 16), 8192 // 16 if i < 2 else 28672 // 16,
                     stream) for i in range(3)]
    setup_s = time.time() - t_setup
    step_ms, act_ms, gemm_ms = time_layers(torch, runs, stream, args.steps, args.warmup)
    total_ops = sum(r.ops for r in runs)
    value = total_ops / (step_ms * 1e-3) / 1e12
    gemm_ops = sum(r.ops for r in runs)
    achieved = gemm_ops / (gemm_ms.sum() * 1e-3) / 1e12
    detail = []
    for r, a, g in zip(runs, act_ms, gemm_ms):
        tops = r.ops / (g * 1e-3) / 1e12
        detail.append(dict(shape=f"{r.m}x{r.k}->{r.n}", k_out=r.k_out, act_us=round(a * 1e3, 2),
                           act_gbs=round(r.act_bytes / (a * 1e-3) / 1e9, 1),
                           gemm_us=round(g * 1e3, 2), gemm_tops=round(tops, 1),
                           pct_int8_peak=round(100 * tops / PEAK_INT8_TOPS, 2),
                           pct_dual_bound=round(100 * tops / (PEAK_INT8_TOPS * dual_bound_frac(
                               r.k - r.k_out, r.k_out)), 2)))
    # the same step with bf16 Y (an output-type option, not the measured
    # configuration; with the rows section): its GEMM times per layer
    bf16_y = None
    if not args.no_rows:
        for r in runs:
            r.yb = torch.empty((r.m, r.n), dtype=torch.bfloat16, device="cuda")
        step_b, _, gemm_b = time_layers(torch, runs, stream, args.steps, args.warmup)
        for r, d, g in zip(runs, detail, gemm_b):
            d["gemm_bf16y_us"] = round(float(g) * 1e3, 2)
            r.yb = None
        torch.cuda.empty_cache()
        bf16_y = {"ms_per_step": round(step_b, 4), "tops": round(total_ops / (step_b * 1e-3) / 1e12, 2),
                  "gemm_top_s": round(gemm_ops / (gemm_b.sum() * 1e-3) / 1e12, 1)}
    traffic = read_traffic()
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4*int4->int32 + bf16->fp32",
        "data": "synthetic (seeded Gaussian, token-persistent outlier channels)",
        "config": {"workload": "llama3_70b_prefill_linears_f1/16", "m": 4096,
                   "shapes_k_n": [[8192, 8192], [8192, 28672], [28672, 8192]],
                   "outlier_fraction": "1/16", "x_dtype": "bf16", "branch": "bf16",
                   "parallelism": "none (1 GPU)"},
        "pct_int8_peak": round(100 * value / PEAK_INT8_TOPS, 2),
        "roofline": {"bound": "mfma", "kernel": "k_dual_gemm", "achieved": round(achieved, 1),
                     "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                     "frac": round(achieved / PEAK_INT8_TOPS, 4),
                     "traffic": traffic, "traffic_unit": "bytes per launch",
                     "avg_launch_us": round(float(gemm_ms.mean()) * 1e3, 2),
                     "ops_per_launch": gemm_ops / 3},
        "detail": detail,
        "bf16_y_step": bf16_y,
        "setup_s": round(setup_s, 1),
    }
    if args.sweep:
        sweep = []
        for den in (2, 4, 8, 16):
            for i in range(3):
                lay = synth.llama3_70b(i, den)
                r = LayerRun(sqf, torch, lay, lay.k // den, stream)
                s_ms, a_ms, g_ms = time_layers(torch, [r], stream, max(5, args.steps // 2), 2)
                tops = r.ops / (g_ms[0] * 1e-3) / 1e12
                sweep.append(dict(frac=f"1/{den}", shape=f"{r.m}x{r.k}->{r.n}",
                                  gemm_us=round(float(g_ms[0]) * 1e3, 1), gemm_tops=round(tops, 1),
                                  pct_int8_peak=round(100 * tops / PEAK_INT8_TOPS, 2),
                                  pct_dual_bound=round(100 * tops / (PEAK_INT8_TOPS * dual_bound_frac(
                                      r.k - r.k_out, r.k_out)), 2)))
                del r
                torch.cuda.empty_cache()
        out["sweep"] = sweep
    if not args.no_rows:
        out["rows"] = rows_section(sqf, torch, stream)
    if args.copy_bytes:
        # plain device copy of a known size: the reference that scales the
        # memory-traffic counters of a profiled run to bytes
        src = torch.empty(args.copy_bytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = args.copy_bytes
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(runs, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
