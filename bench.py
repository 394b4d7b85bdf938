#!/usr/bin/env python3
"""Benchmark of the dual-path outlier-separated GEMM on one MI355X.

    python bench.py [--steps K] [--warmup W] [--no-sweep] [--no-rows] [--no-cpu]

Workload: the Llama-3-70B-shaped prefill linears (M = 4096 tokens;
8192->8192, 8192->28672, 28672->8192) at outlier fraction 1/16, bf16 input
activations, bf16 outlier branch, seeded synthetic data (no model weights or
datasets exist here).  Channel selection and weight packing are offline and
run once before timing.  One step = for each of the three layers: the online
activation quantise/split kernel, then the fused dual GEMM -- every online
step of the path, inputs resident in HBM.  The int4 codes are stored in
6-bit E2M3 fields (the value c/8) and multiplied on the FP6 matrix unit,
whose fp32 sums of these products are exact (every partial sum is a multiple
of 1/64 far below 2^24), so the results are those of an int32 accumulation;
the same step with the codes packed two per byte on the int8 matrix unit is
timed beside it (``packed_int4_step``).

Prints ONE JSON line.  ``value`` is effective TOPS = sum(2*M*N*K) / step
time.  ``roofline`` describes the dominant kernel (the dual GEMM): achieved
algorithmic ops (2*M*N*K per launch) / its average launch time measured with
HIP events on the stream it runs on, against the kernel's own matrix-core
ceiling (the low path's operations at the FP6 peak plus the branch's at the
bf16 peak); ``traffic`` is HBM bytes per GEMM launch from the committed
rocprofv3 counter summary, or null if the kernel source changed since it was
taken.  ``cpu_baseline`` times the scalar CPU oracle on a bounded row sample
of the same step.  ``sweep`` holds the outlier-fraction sweep (1/2 ... 1/16)
of the same layers and the Llama-3-8B-shaped layers; ``rows`` every other
row of the path on its own workload.
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
PEAK_FP6_TFLOPS = 10100.0  # MI355X dense FP6 / FP4 MFMA, 10.1 PFLOP/s
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
GEMM_SOURCES = ["outlier_split_mixed_amd/csrc/k_gemm6.hip", "outlier_split_mixed_amd/csrc/sqf_device.h"]
HEADLINE_LOW = "i4e2m3"  # the int4 codes in 6-bit E2M3 fields on the FP6 matrix unit
LOW_PEAK = {"i4": PEAK_INT8_TOPS, "i4e2m3": PEAK_FP6_TFLOPS, "mxfp4": PEAK_FP6_TFLOPS}  # FP4 = FP6 rate
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_k_gemm6_llama3_70b_f16.txt")


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


def mfma_bound_us(m, n, k_low, k_out, low_peak=PEAK_INT8_TOPS, branch_peak=PEAK_BF16_TFLOPS):
    """Shortest time the method's own arithmetic can take on the matrix cores:
    2*M*N*K_low low-path operations at the low path's peak plus 2*M*N*K_out
    branch operations at the branch's peak (TOP/s in, microseconds out)."""
    return 2.0 * m * n * (k_low / low_peak + k_out / branch_peak) / 1e6


def pct(v, q):
    return round(float(np.percentile(np.asarray(v), q)), 2)


class LayerRun:
    def __init__(self, sqf, torch, lay, k_out, stream, low=HEADLINE_LOW):
        self.lay = lay
        self.m, self.k, self.n, self.k_out = lay.m, lay.k, lay.n, k_out
        with torch.cuda.stream(stream):
            x_cal = torch.from_numpy(lay.x_cal).cuda()
            w = torch.from_numpy(lay.w).cuda()
            _, self.map, _, _ = sqf.sqf_select_channels(x_cal, w, k_out, stream=stream)
            self.low = low
            self.w = sqf.sqf_pack_weights(w, self.map, stream=stream, low=low)
            from outlier_split_mixed_amd import synth

            bits = synth.to_bf16_bits(lay.x)
            self.x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
            self.acts = sqf.alloc_acts(lay.m, lay.k - k_out, k_out, low=low)
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
    act = np.zeros((steps, len(runs)))
    gemm = np.zeros((steps, len(runs)))
    for s in range(steps):
        for i in range(len(runs)):
            e = evs[s][i]
            act[s, i] = e[0].elapsed_time(e[1])
            gemm[s, i] = e[1].elapsed_time(e[2])
    time_layers.samples = (act, gemm)
    return total_ms / steps, act.mean(0), gemm.mean(0)


def measured_peaks():
    """Matrix-unit rates measured on this GPU (TOP/s), with the dual GEMM's
    register pattern (8 A x 4 B fragments, 32 accumulators per wave, two
    waves per SIMD, one 512-thread block per CU; libsqf_bench.so, built
    beside libsqf.so).  Two operand kinds: drawn like the workload's (int4
    codes of normal values, E2M1 codes, 16*c, bf16 values), which is the
    rate the GEMM's data allows, and a low-entropy pattern, the unit's upper
    bound (the 6-/4-bit unit sustains markedly less on real data)."""
    import ctypes

    path = os.path.join(ROOT, "outlier_split_mixed_amd", "libsqf_bench.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build with __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    lib.sqfb_mfma_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.POINTER(ctypes.c_double)]
    out = {"workload": {}, "pattern": {}}
    for data, key in ((1, "workload"), (0, "pattern")):
        for name, kind in (("fp6", 0), ("fp4", 1), ("int8", 2), ("bf16", 3)):
            v = ctypes.c_double()
            rc = lib.sqfb_mfma_rate(kind, data, 256, 2048, 5, ctypes.byref(v))
            if rc != 0:
                raise RuntimeError(f"sqfb_mfma_rate({name}, {key}) failed: {rc}")
            out[key][name] = round(v.value, 1)
    return out


def clone_run(r):
    """A LayerRun over fresh device copies of every buffer it touches (same
    contents, different memory)."""
    import copy

    c = copy.copy(r)
    c.x = r.x.clone()
    c.map = r.map.clone()
    c.y = r.y.clone()
    c.w = copy.copy(r.w)
    c.w.t = {k: (v.clone() if v is not None else None) for k, v in r.w.t.items()}
    c.acts = copy.copy(r.acts)
    c.acts.t = {k: (v.clone() if v is not None else None) for k, v in r.acts.t.items()}
    return c


def time_rotated(torch, sets, stream, steps, warmup):
    """Steps back to back over rotating buffer sets: step s runs set s % len(sets),
    so each step's operands were last touched len(sets) - 1 steps earlier."""
    n = len(sets)
    for s in range(warmup):
        for r in sets[s % n]:
            r.step(stream)
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in sets[0]] for _ in range(steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for s in range(steps):
        for i, r in enumerate(sets[s % n]):
            r.step(stream, evs[s][i])
    t1.record(stream)
    torch.cuda.synchronize()
    act = np.array([[e[0].elapsed_time(e[1]) for e in row] for row in evs])
    gemm = np.array([[e[1].elapsed_time(e[2]) for e in row] for row in evs])
    return t0.elapsed_time(t1) / steps, act, gemm


def time_cold(torch, runs, stream, steps, flush_bytes=1 << 30):
    """Each step timed alone after overwriting a 1 GiB device buffer on the
    same stream, which evicts the L2s and the 256 MiB last-level cache: no
    operand of the step is resident in any cache when it starts."""
    buf = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    for s in range(steps):
        with torch.cuda.stream(stream):
            buf.fill_(float(s))
        evs[s][0].record(stream)
        for r in runs:
            r.step(stream)
        evs[s][1].record(stream)
    torch.cuda.synchronize()
    del buf
    return np.array([a.elapsed_time(b) for a, b in evs])


def cpu_baseline(lays, rows_per_layer):
    """The oracle (untuned) on a bounded sample of the same step: the online
    stages (activation quantise/split + dual GEMM) for `rows_per_layer` token
    rows of each layer.  Offline packing is outside the step, as on the GPU."""
    import oracle
    from outlier_split_mixed_amd import synth

    total_ops, total_s = 0.0, 0.0
    for lay in lays:
        _, o_mp, _, _ = oracle.select_channels(lay.x_cal, lay.w, lay.k_out)
        o_w = oracle.pack_weights(lay.w, o_mp)
        xs = synth.to_bf16_bits(lay.x[:rows_per_layer])
        t = time.perf_counter()
        o_a = oracle.quantize_split_act(xs, o_mp, x_fmt="bf16")
        oracle.dual_gemm(o_a, o_w)
        total_s += time.perf_counter() - t
        total_ops += 2.0 * rows_per_layer * lay.n * lay.k
    return dict(value=round(total_ops / total_s / 1e12, 6), unit="TOPS", cores=oracle.num_threads(),
                kind="oracle", cpu_model=cpu_model(),
                sample=f"{rows_per_layer} token rows x all outputs of each of the 3 layers "
                       f"(act quantise/split + dual GEMM), {total_s:.1f} s")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def progress(msg):
    """One line per finished section on stderr (stdout carries only the JSON)."""
    print(f"# bench: {msg}", file=sys.stderr, flush=True)


def _add(out, row):
    out.append(row)
    progress(row["row"])


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
        _add(out, dict(row="a0 select (offline)", shape=f"{lay.k}x{lay.n}, {lay.x_cal.shape[0]} cal rows",
                        ms=round(t, 3), gbs=round(b0 / t / 1e6, 1), frac_hbm=round(b0 / t / 1e6 / PEAK_HBM_GBS, 3)))
        t = time_call(torch, stream, lambda: sqf.sqf_pack_weights(w, mp, stream=stream), iters=3, warmup=1)
        # W and the map read once; int4 rows, bf16 branch rows and scales written
        ldk = sqf.sqf_pad_k_low(lay.k - k_out) // 2
        ldo = sqf.sqf_pad_k_out(k_out, "bf16")
        b1 = 4 * lay.k * lay.n + 4 * lay.k + lay.n * (ldk + 2 * ldo + 4)
        _add(out, dict(row="a1 pack (offline)", shape=f"{lay.k}x{lay.n}", ms=round(t, 3),
                        gbs=round(b1 / t / 1e6, 1), frac_hbm=round(b1 / t / 1e6 / PEAK_HBM_GBS, 3)))
        del w, x_cal, mp
        torch.cuda.empty_cache()

        # f2: the RMS norm fused into the split (E2M3 storage, bf16 X), on the
        # 70B step's two row widths, against the split alone; a separate norm
        # kernel would add a read and a write of X (2 * M * K * 2 bytes)
        for li in (0, 2):
            lay = synth.llama3_70b(li, 16)
            x_cal = torch.from_numpy(lay.x_cal).cuda()
            w = torch.from_numpy(lay.w).cuda()
            _, mp, _, _ = sqf.sqf_select_channels(x_cal, w, lay.k_out, stream=stream)
            del w, x_cal
            xt = torch.from_numpy(synth.to_bf16_bits(lay.x).view(np.int16)).view(torch.bfloat16).cuda()
            g = torch.ones(lay.k, dtype=torch.float32, device="cuda")
            a = sqf.alloc_acts(lay.m, lay.k - lay.k_out, lay.k_out, low=HEADLINE_LOW)
            t0 = time_call(torch, stream, lambda: sqf.sqf_quantize_split_act(xt, mp, a, stream=stream))
            t1 = time_call(torch, stream, lambda: sqf.sqf_rmsnorm_quantize_split_act(
                xt, g, 1e-5, mp, a, stream=stream))
            b = lay.m * (lay.k * 2 + a.ldk + a.ldo * 2 + 4)
            _add(out, dict(row=f"f2 RMS norm fused into the split ({lay.m}x{lay.k}, E2M3 codes)",
                           split_us=round(t0 * 1e3, 1), fused_us=round(t1 * 1e3, 1),
                           fused_frac_hbm=round(b / (t1 * 1e-3) / 1e9 / PEAK_HBM_GBS, 3),
                           separate_norm_min_us=round(2 * lay.m * lay.k * 2 / (PEAK_HBM_GBS * 1e9) * 1e6, 1)))
            del xt, a, g, mp
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
            _add(out, dict(row=f"a6 grouped {name} ({br} branch)",
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

        # a7: SQ-format weight side, one bank per row and banks of 64 slots
        lay = synth.sq_weight()
        k_out = lay.k_out
        k_low = lay.k - k_out
        x_cal = torch.from_numpy(lay.x_cal).cuda()
        w = torch.from_numpy(lay.w).cuda()
        _, mp, _, hd = sqf.sqf_select_channels(x_cal, w, k_out, stream=stream)
        xt = torch.from_numpy(synth.to_bf16_bits(lay.x).view(np.int16)).view(torch.bfloat16).cuda()
        a = sqf.alloc_acts(lay.m, k_low, k_out, low="i8", branch="i8")
        y = torch.empty((lay.m, lay.n), dtype=torch.float32, device="cuda")
        ta = time_call(torch, stream, lambda: sqf.sqf_quantize_split_act(xt, mp, a, stream=stream))
        nnz = k_low // 8
        for bank in (0, 64):
            tp = time_call(torch, stream, lambda: sqf.sqf_pack_weights(
                w, mp, branch="i8", hdiag=hd, sq_nnz=nnz, sq_bank=bank, stream=stream), iters=2, warmup=1)
            wt = sqf.sqf_pack_weights(w, mp, branch="i8", hdiag=hd, sq_nnz=nnz, sq_bank=bank, stream=stream)
            tg = time_call(torch, stream, lambda: sqf.sqf_dual_gemm(a, wt, y=y, stream=stream), iters=5)
            # the same product with the gather done once per call into a
            # workspace (decode kernel + GEMM on the decoded tiles, both timed)
            ws = torch.empty(sqf.sqf_sq_workspace_bytes(wt), dtype=torch.uint8, device="cuda")
            tw = time_call(torch, stream, lambda: sqf.sqf_dual_gemm_sq_ws(a, wt, y=y, workspace=ws,
                                                                          stream=stream), iters=5)
            # the method's own work: every low slot, every marked value and
            # every branch channel once (2*M*N*(K_low + nnz + K_out) int8 operations)
            own_ops = 2.0 * lay.m * lay.n * (k_low + nnz + k_out)
            # what the kernel issues: two dense int8 passes over K_low plus the branch
            mfma_ops = 2.0 * lay.m * lay.n * (2 * k_low + k_out)
            what = "one bank per row" if bank == 0 else f"banks of {bank} slots, {nnz * bank // k_low} marks each"
            _add(out, dict(row=f"a7 SQ-format weight side ({what}; int8 acts, masked int8 part, int8 branch)",
                            shape=f"{lay.m}x{lay.k}->{lay.n}, nnz {nnz}/row",
                            pack_ms=round(tp, 3),
                            act_us=round(ta * 1e3, 1), gemm_us=round(tg * 1e3, 1),
                            gemm_eff_tops=round(2.0 * lay.m * lay.n * lay.k / (tg * 1e-3) / 1e12, 1),
                            own_work_tops=round(own_ops / (tg * 1e-3) / 1e12, 1),
                            frac_int8_peak=round(own_ops / (tg * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
                            issued_mfma_tops=round(mfma_ops / (tg * 1e-3) / 1e12, 1),
                            ws_call_us=round(tw * 1e3, 1),
                            ws_workspace_mib=round(ws.numel() / 2**20, 1),
                            ws_frac_int8_peak=round(own_ops / (tw * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4)))
            del wt, ws
        # f4: the floating-point form (E2M1 low codes with the mark, E4M3
        # values, E4M3 activations and branch), one bank per row
        af = sqf.alloc_acts(lay.m, k_low, k_out, low="fp8", branch="fp8")
        taf = time_call(torch, stream, lambda: sqf.sqf_quantize_split_act(xt, mp, af, stream=stream))
        tp = time_call(torch, stream, lambda: sqf.sqf_pack_weights(
            w, mp, branch="fp8", hdiag=hd, sq_nnz=nnz, low="fp4", stream=stream), iters=2, warmup=1)
        wt = sqf.sqf_pack_weights(w, mp, branch="fp8", hdiag=hd, sq_nnz=nnz, low="fp4", stream=stream)
        tg = time_call(torch, stream, lambda: sqf.sqf_dual_gemm(af, wt, y=y, stream=stream), iters=5)
        ws = torch.empty(sqf.sqf_sq_workspace_bytes(wt), dtype=torch.uint8, device="cuda")
        tw = time_call(torch, stream, lambda: sqf.sqf_dual_gemm_sq_ws(af, wt, y=y, workspace=ws,
                                                                      stream=stream), iters=5)
        own_ops = 2.0 * lay.m * lay.n * (k_low + nnz + k_out)
        bits = (wt.t["w_low"].numel() * 8 + wt.t["sq_val"].numel() * 8) / (lay.n * sqf.sqf_pad_k_low(k_low))
        _add(out, dict(row="f4 SQ-format, FP8/FP4 (E2M1 low with the mark, E4M3 values, E4M3 acts and branch)",
                        shape=f"{lay.m}x{lay.k}->{lay.n}, nnz {nnz}/row",
                        bits_per_low_weight=round(bits, 3),
                        pack_ms=round(tp, 3), act_us=round(taf * 1e3, 1), gemm_us=round(tg * 1e3, 1),
                        gemm_eff_tops=round(2.0 * lay.m * lay.n * lay.k / (tg * 1e-3) / 1e12, 1),
                        own_work_tops=round(own_ops / (tg * 1e-3) / 1e12, 1),
                        frac_fp8_peak=round(own_ops / (tg * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
                        ws_call_us=round(tw * 1e3, 1),
                        ws_workspace_mib=round(ws.numel() / 2**20, 1),
                        ws_frac_fp8_peak=round(own_ops / (tw * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4)))
        del wt, af, ws
        del xt, a, y, w, x_cal
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the outlier-fraction sweep and the Llama-3-8B-shaped layers")
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
    progress(f"setup of the three layers done ({setup_s:.1f} s)")
    step_ms, act_ms, gemm_ms = time_layers(torch, runs, stream, args.steps, args.warmup)
    act_s, gemm_s = time_layers.samples
    progress(f"step timed: {step_ms:.4f} ms")
    cold = time_cold(torch, runs, stream, max(5, args.steps // 2))
    progress(f"cold steps timed: median {np.median(cold):.4f} ms")
    # four buffer sets in rotation (every buffer of a step: X, codes, weights, Y)
    sets = [runs] + [[clone_run(r) for r in runs] for _ in range(3)]
    set_bytes = sum(t.numel() * t.element_size() for r in runs
                    for t in [r.x, r.y, *r.w.t.values(), *r.acts.t.values()] if t is not None)
    rot_ms, rot_act, rot_gemm = time_rotated(torch, sets, stream, args.steps, args.warmup)
    del sets
    torch.cuda.empty_cache()
    progress(f"rotated steps timed: {rot_ms:.4f} ms")
    total_ops = sum(r.ops for r in runs)
    value = total_ops / (step_ms * 1e-3) / 1e12
    gemm_ops = sum(r.ops for r in runs)
    achieved = gemm_ops / (gemm_ms.sum() * 1e-3) / 1e12
    # the GEMM's own ceiling: each layer's low part at the FP6 peak and its
    # bf16 branch at the bf16 peak, summed over the three launches
    low_peak = LOW_PEAK[HEADLINE_LOW]
    bound_us = sum(mfma_bound_us(r.m, r.n, r.k - r.k_out, r.k_out, low_peak) for r in runs)
    peak_eff = gemm_ops / (bound_us * 1e-6) / 1e12
    detail = []
    for i, (r, a, g) in enumerate(zip(runs, act_ms, gemm_ms)):
        tops = r.ops / (g * 1e-3) / 1e12
        b_us = mfma_bound_us(r.m, r.n, r.k - r.k_out, r.k_out, low_peak)
        detail.append(dict(shape=f"{r.m}x{r.k}->{r.n}", k_out=r.k_out, act_us=round(a * 1e3, 2),
                           act_us_p10_p50_p90=[pct(act_s[:, i] * 1e3, q) for q in (10, 50, 90)],
                           act_gbs=round(r.act_bytes / (a * 1e-3) / 1e9, 1),
                           act_frac_hbm=round(r.act_bytes / (a * 1e-3) / 1e9 / PEAK_HBM_GBS, 3),
                           gemm_us=round(g * 1e3, 2),
                           gemm_us_p10_p50_p90=[pct(gemm_s[:, i] * 1e3, q) for q in (10, 50, 90)],
                           gemm_tops=round(tops, 1),
                           pct_int8_peak=round(100 * tops / PEAK_INT8_TOPS, 2),
                           mfma_bound_us=round(b_us, 1),
                           frac_mfma_bound=round(b_us / (g * 1e3), 4)))
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
    progress("bf16-Y step timed")
    lays = [r.lay for r in runs]
    lays_shapes = [(r.m, r.n, r.k, r.k_out) for r in runs]
    del runs
    torch.cuda.empty_cache()
    # the same step with the int4 codes packed two per byte (the int8 matrix
    # unit, codes unpacked in registers): same layers, same results
    runs4 = [LayerRun(sqf, torch, l, l.k_out, stream, low="i4") for l in lays]
    step4, act4, gemm4 = time_layers(torch, runs4, stream, args.steps, args.warmup)
    i4_step = {"low": "packed int4 (two codes per byte) on the int8 MFMA",
               "ms_per_step": round(step4, 4),
               "tops": round(total_ops / (step4 * 1e-3) / 1e12, 2),
               "act_us": [round(float(v) * 1e3, 2) for v in act4],
               "gemm_us": [round(float(v) * 1e3, 2) for v in gemm4],
               "gemm_frac_mfma_bound": [round(mfma_bound_us(r.m, r.n, r.k - r.k_out, r.k_out,
                                                            PEAK_INT8_TOPS) / (float(g) * 1e3), 4)
                                        for r, g in zip(runs4, gemm4)]}
    del runs4
    torch.cuda.empty_cache()
    progress(f"packed-int4 step timed: {step4:.4f} ms")
    # the MXFP4 low path (E2M1 codes, one E8M0 scale per 32 slots) on the same
    # layers: a different number format (its own quantisation), same shapes
    runs_mx = [LayerRun(sqf, torch, l, l.k_out, stream, low="mxfp4") for l in lays]
    step_mx, act_mx, gemm_mx = time_layers(torch, runs_mx, stream, args.steps, args.warmup)
    mx_bound = [mfma_bound_us(r.m, r.n, r.k - r.k_out, r.k_out, LOW_PEAK["mxfp4"]) for r in runs_mx]
    mx_step = {"low": "MXFP4 (E2M1 codes, E8M0 scale per 32 slots) on the FP4 MFMA",
               "ms_per_step": round(step_mx, 4),
               "tops": round(total_ops / (step_mx * 1e-3) / 1e12, 2),
               "act_us": [round(float(v) * 1e3, 2) for v in act_mx],
               "gemm_us": [round(float(v) * 1e3, 2) for v in gemm_mx],
               "gemm_tops": round(gemm_ops / (gemm_mx.sum() * 1e-3) / 1e12, 1),
               "gemm_frac_mfma_bound": [round(b / (float(g) * 1e3), 4) for b, g in zip(mx_bound, gemm_mx)],
               "roofline_frac": round(sum(mx_bound) / (gemm_mx.sum() * 1e3), 4),
               "peak_basis": "2MN*K_low at the 10.1 PFLOP/s FP4 peak + 2MN*K_out at 2.5 PFLOP/s bf16"}
    del runs_mx
    torch.cuda.empty_cache()
    progress(f"MXFP4 step timed: {step_mx:.4f} ms")
    traffic = read_traffic()
    meas = measured_peaks()
    progress(f"measured matrix-unit rates: {meas}")
    # the same kernel bound with the rates measured on workload-shaped operands
    # (and on the pattern) in place of the spec peaks
    def bound_at(rates):
        return sum(2.0 * m * n * ((k - ko) / rates["fp6"] + ko / rates["bf16"]) / 1e6
                   for m, n, k, ko in lays_shapes)
    bound_meas_us, bound_pat_us = bound_at(meas["workload"]), bound_at(meas["pattern"])
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
        "dtype": "int4 codes (as E2M3 values c/8, FP6 MFMA, exact fp32 sums) + bf16 -> fp32",
        "data": "synthetic (seeded Gaussian, token-persistent outlier channels)",
        "config": {"workload": "llama3_70b_prefill_linears_f1/16", "m": 4096,
                   "shapes_k_n": [[8192, 8192], [8192, 28672], [28672, 8192]],
                   "outlier_fraction": "1/16", "x_dtype": "bf16", "branch": "bf16",
                   "low_storage": "int4 codes in 6-bit E2M3 fields (K-blocked, lane order)",
                   "parallelism": "none (1 GPU)"},
        "pct_int8_peak": round(100 * value / PEAK_INT8_TOPS, 2),
        "roofline": {"bound": "mfma", "kernel": "k_gemm6", "achieved": round(achieved, 1),
                     "peak": round(peak_eff, 1), "unit": "TOP/s",
                     "frac": round(achieved / peak_eff, 4),
                     "traffic": traffic, "traffic_unit": "bytes per launch",
                     "peak_basis": "2MN*K_low at the 10.1 PFLOP/s FP6 peak + 2MN*K_out at the "
                                   "2.5 PFLOP/s bf16 peak, over the three launches",
                     "frac_int8_peak": round(achieved / PEAK_INT8_TOPS, 4),
                     "avg_launch_us": round(float(gemm_ms.mean()) * 1e3, 2),
                     "ops_per_launch": gemm_ops / 3,
                     "measured_peaks_tops": meas,
                     "frac_of_measured_bound": round(bound_meas_us / (float(gemm_ms.sum()) * 1e3), 4),
                     "frac_of_pattern_bound": round(bound_pat_us / (float(gemm_ms.sum()) * 1e3), 4),
                     "measured_basis": "the same two terms at the rates the matrix units sustain on this "
                                       "GPU with operands drawn like the workload's (frac_of_measured_bound) "
                                       "and on a low-entropy pattern (frac_of_pattern_bound)"},
        "detail": detail,
        "cold_step": {"protocol": "each step timed alone (HIP events on its stream) after a 1 GiB device "
                                  "buffer is overwritten on the same stream: L2s and the 256 MiB last-level "
                                  "cache hold no operand; the steps above run back to back (warm)",
                      "steps": int(cold.size),
                      "ms_p10_p50_p90": [round(float(np.percentile(cold, q)), 4) for q in (10, 50, 90)],
                      "tops_at_p50": round(total_ops / (float(np.median(cold)) * 1e-3) / 1e12, 2)},
        "rotated_step": {"protocol": "steps back to back over 4 buffer sets in rotation (X, codes, packed "
                                     "weights, Y: every buffer of a step), each set "
                                     f"{set_bytes / 2**30:.2f} GiB, so a step's operands were last touched "
                                     "3 steps (about 4.5 GiB of traffic) earlier, beyond the 256 MiB "
                                     "last-level cache",
                         "ms_per_step": round(rot_ms, 4),
                         "tops": round(total_ops / (rot_ms * 1e-3) / 1e12, 2),
                         "act_us_p50": [pct(rot_act[:, i] * 1e3, 50) for i in range(rot_act.shape[1])],
                         "gemm_us_p50": [pct(rot_gemm[:, i] * 1e3, 50) for i in range(rot_gemm.shape[1])]},
        "bf16_y_step": bf16_y,
        "packed_int4_step": i4_step,
        "mxfp4_step": mx_step,
        "setup_s": round(setup_s, 1),
    }
    if not args.no_sweep:
        # the Llama-3-70B-shaped layers at outlier fractions 1/2 ... 1/16, and
        # the Llama-3-8B-shaped layers at 1/16 (M = 2048)
        sweep = []
        cases = [(f"1/{den}", synth.llama3_70b(i, den)) for den in (2, 4, 8, 16) for i in range(3)]
        cases += [("1/16", synth.llama3_8b(i)) for i in range(3)]
        for frac, lay in cases:
            r = LayerRun(sqf, torch, lay, lay.k_out, stream)
            s_ms, a_ms, g_ms = time_layers(torch, [r], stream, max(5, args.steps // 2), 5)
            g_us = float(g_ms[0]) * 1e3
            tops = r.ops / (g_us * 1e-6) / 1e12
            b_us = mfma_bound_us(r.m, r.n, r.k - r.k_out, r.k_out, low_peak)
            sweep.append(dict(workload=lay.name.split(".")[0], frac=frac,
                              shape=f"{r.m}x{r.k}->{r.n}", k_out=r.k_out,
                              act_us=round(float(a_ms[0]) * 1e3, 1),
                              gemm_us=round(g_us, 1), gemm_tops=round(tops, 1),
                              layer_us=round(float(a_ms[0] + g_ms[0]) * 1e3, 1),
                              pct_int8_peak=round(100 * tops / PEAK_INT8_TOPS, 2),
                              frac_mfma_bound=round(b_us / g_us, 4)))
            del r
            torch.cuda.empty_cache()
            progress(f"sweep {lay.name} {frac}: {g_us:.1f} us")
        out["sweep"] = sweep
    if not args.no_rows:
        out["rows"] = rows_section(sqf, torch, stream)
        progress("rows section done")
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
        out["cpu_baseline"] = cpu_baseline(lays, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
