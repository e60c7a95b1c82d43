#!/usr/bin/env python3
"""Benchmark of the quantized GEMM hot path on one MI355X.

Default workload: dense W4A16 (uint4 codes, uint4 zero points, bf16 group-128 scales,
bf16 activations), N = K = 8192, swept over M = 1, 16, 128, 1024, 4096.  One step runs
qg_gemm once per M.  Inputs are resident in HBM before timing starts; the prepared
weights are rotated over enough copies (>= 1 GiB in total) that every launch streams its
weights from HBM rather than from the 256 MB last-level cache -- the pages time kernels
with a cold L2.

Output: one JSON line with the metric, whole-job throughput (TFLOP/s over the sweep),
a per-M breakdown, the roofline of the dominant kernel (per-launch HIP-event
durations) and the CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload dense_w4a16_asym_bf16|...]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "quantized_gemm_amd", "csrc")
# sources that define the MFMA-bound kernel (the dominant launch of the default sweep)
MFMA_SOURCES = ["qg_mfma_kernel.h", "qg_device.h", "qg_kernels.h", "qg_mfma_int4.hip"]
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}

# Workloads: (builder, sweep, arithmetic type of the MFMAs (selects the peak), description).
# The W4A8 products run on fp8 MFMAs (int4 converted to e4m3 in the kernel) above the
# streaming sizes; below them the streaming kernel multiplies exact bf16 images of both.
WORKLOADS = {
    "dense_w4a16_asym_bf16": dict(sweep=[1, 16, 128, 1024, 4096], n=8192, k=8192, dtype="bf16",
                                  desc="dense W4A16 uint4 + uint4 zero points, bf16 group-128 scales, "
                                       "bf16 activations and output"),
    "dense_w4a16_sym_f16": dict(sweep=[16], n=512, k=1024, dtype="f16",
                                desc="dense W4A16 symmetric int4, f16 group-128 scales, f16 activations"),
    "dense_w8a8_fp8": dict(sweep=[1, 64, 512, 4096], n=7168, k=7168, dtype="fp8",
                           desc="dense W8A8 e4m3 per-channel x per-token scales, bf16 output"),
    "moe_w4a16_mxfp4": dict(sweep=[16, 256, 4096], n=4096, k=7168, dtype="bf16", moe=dict(experts=128, topk=8),
                            desc="MoE W4A16 MXFP4 (e2m1 + UE8M0/32), E=128 top-8, fused gate+up N=4096, K=7168, "
                                 "bf16 activations; T sweep"),
    "dense_w8a8_fp8_block": dict(sweep=[1, 64, 512, 4096], n=7168, k=7168, dtype="fp8",
                                 desc="dense W8A8 e4m3 with 128 x 128 weight-block scales and per-(token, 128-K) "
                                      "activation scales, bf16 output; M sweep"),
    "dense_w4a8_mxfp4": dict(sweep=[1, 16, 128, 1024, 4096], n=8192, k=8192, dtype="fp8",
                             desc="dense W4A8 MXFP4 (e2m1 + UE8M0/32 weights x per-token e4m3 activations, scaled "
                                  "fp8 x fp4 MFMAs), N=K=8192; M sweep"),
    "moe_w4a8_mxfp4": dict(sweep=[16, 256, 4096], n=4096, k=7168, dtype="fp8", moe=dict(experts=128, topk=8),
                           desc="MoE W4A8 MXFP4 (e2m1 + UE8M0/32 x per-token e4m3, scaled fp8 x fp4 MFMAs), E=128 "
                                "top-8, fused gate+up N=4096, K=7168; T sweep"),
    "dense_w4a4_mxfp4": dict(sweep=[1, 16, 128, 1024, 4096], n=8192, k=8192, dtype="fp4",
                             desc="dense W4A4 MXFP4 (e2m1 + UE8M0/32 weights x e2m1 + UE8M0/32 activations, scaled "
                                  "fp4 x fp4 MFMAs), N=K=8192; M sweep"),
    "moe_w4a4_mxfp4": dict(sweep=[16, 256, 4096], n=4096, k=7168, dtype="fp4", moe=dict(experts=128, topk=8),
                           desc="MoE W4A4 MXFP4 (e2m1 + UE8M0/32 on both sides, scaled fp4 x fp4 MFMAs), E=128 "
                                "top-8, fused gate+up N=4096, K=7168; T sweep"),
    "moe_w4a8_int4": dict(sweep=[64, 1024, 8192], n=2816, k=4096, dtype="fp8", moe=dict(experts=64, topk=6),
                          desc="MoE W4A8 int4 weights with bf16 group-128 scales x per-token e4m3 activations, "
                               "E=64 top-6, N=2816, K=4096, 20% of tokens biased to 4 hot experts; T sweep"),
}


DEFAULT_WORKLOAD = "dense_w4a16_asym_bf16"
# The other benchmark workloads the default line carries (each its own sweep and roofline).
EXTRA_WORKLOADS = ["dense_w4a16_sym_f16", "dense_w8a8_fp8", "moe_w4a16_mxfp4", "moe_w4a8_int4"]


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def measure_ceilings(args):
    """Measured ceilings of this GPU: a streaming read of cold buffers the size of the dense
    W4A16 layer's weight stream (34 865 152 bytes), rotated over >= 1 GiB so every launch
    reads from HBM, and of 256 MiB buffers; back-to-back MFMAs of each arithmetic type."""
    import torch
    import quantized_gemm_amd as qg
    stream = torch.cuda.current_stream()
    out = {"read_us": {}, "read_GBps_by_loads_per_lane": {}}
    pool = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    pool.fill_(1)
    sink = torch.empty(1 << 20, dtype=torch.int32, device="cuda")
    reps = max(20, args.steps)
    for size, label in ((34865152, "weights_34.9MB"), (256 << 20, "256MiB")):
        stride = (size + 4095) // 4096 * 4096
        nbuf = (1 << 30) // stride
        best = None
        for u in (2, 4, 8, 16):
            def launch(i):
                qg.ceiling_read(pool[(i % nbuf) * stride:], size, u, sink)
            for i in range(3):
                launch(i)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(reps):
                launch(i)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            gbps = size / (us * 1e-6) / 1e9
            out["read_GBps_by_loads_per_lane"][f"{label}_u{u}"] = round(gbps, 1)
            if best is None or us < best[0]:
                best = (us, gbps, u)
        out["read_us"][label] = round(best[0], 2)
        out[f"read_GBps_{label}"] = round(best[1], 1)
    out["read_GBps"] = out["read_GBps_weights_34.9MB"]
    del pool
    flop_per = {0: 32768, 1: 131072, 2: 131072}
    names = {0: "bf16", 1: "fp8", 2: "fp4"}
    out["mfma_tflops"] = {}
    wgs, iters = 512, 4000
    msink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    for dt in (0, 1, 2):
        qg.ceiling_mfma(dt, 100, wgs, msink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        qg.ceiling_mfma(dt, iters, wgs, msink)
        e1.record(stream)
        torch.cuda.synchronize()
        s = e0.elapsed_time(e1) * 1e-3
        out["mfma_tflops"][names[dt]] = round(wgs * 4 * iters * 4 * flop_per[dt] / s / 1e12, 1)
    out["mfma_tflops"]["f16"] = out["mfma_tflops"]["bf16"]
    # LDS reads: one workgroup of 8 waves per CU, 16 bytes per lane per read
    lwg, liters = 256, 20000
    lsink = torch.empty(lwg * 512, dtype=torch.int32, device="cuda")
    qg.ceiling_lds(100, lwg, lsink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    qg.ceiling_lds(liters, lwg, lsink)
    e1.record(stream)
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) * 1e-3
    lds_bytes = lwg * 512 * liters * 8 * 16
    out["lds_read_TBps"] = round(lds_bytes / s / 1e12, 2)
    out["lds_read_bytes_per_clk_per_cu_at_2.4GHz"] = round(lds_bytes / s / 256 / 2.4e9, 1)
    out["method"] = ("read: qg_ceiling_read, best of 2/4/8/16 16-byte loads per lane, back-to-back launches "
                     "between HIP events over buffers rotated through 1 GiB; mfma: qg_ceiling_mfma, 512 "
                     "workgroups x 4 waves x 4 independent 32x32 MFMAs per iteration")
    return out


def weight_bytes(layer):
    """Algorithmic weight bytes of ONE expert: packed codes + scales + zero points (4-bit packed)."""
    bits = 8 if layer.w_type == "e4m3" else 4
    g = 1 if layer.group == 0 else layer.k // layer.group
    sb = {"f16": 2, "bf16": 2, "f32": 4, "ue8m0": 1}[layer.s_type]
    b = layer.n * layer.k * bits // 8 + layer.n * g * sb
    if layer.z is not None:
        b += layer.n * g // 2
    return b


def sources_sha1(names):
    import hashlib
    h = hashlib.sha1()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload, m):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if the kernel
    sources are unchanged since the counters were taken; else None."""
    import json as _json
    path = os.path.join(PROFILES, f"traffic_{workload}_m{m}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = _json.load(f)
    if t.get("kernel_sources_sha1") != sources_sha1(MFMA_SOURCES):
        return None
    return t.get("traffic_bytes")


def copy_calibration(mib, reps=5):
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    src.fill_(7)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_mib": mib, "reps": reps}))


def cpu_baseline(builder, wl, budget_cols):
    """The oracle, untuned, on a column slice of the same layer: all M of the sweep."""
    from oracle import reference as R
    import copy
    layer, acts = builder(m=max(wl["sweep"]), n=wl["n"], k=wl["k"], seed=0)
    sl = copy.copy(layer)
    cols = np.arange(budget_cols)
    x_all = R.activations(acts, layer.a_type)
    t0 = time.perf_counter()
    w = R.dequant_rows(layer, 0, cols)
    flops = 0
    for m in wl["sweep"]:
        R.dense_gemm(x_all[:m], w)
        flops += 2 * m * budget_cols * layer.k
    dt = time.perf_counter() - t0
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads") or 0) for i in threadpool_info()) or None
    except Exception:
        pass
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads or os.cpu_count(),
            "cpu_model": cpu_model(), "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"float64 dequant + numpy.matmul of the first {budget_cols} of {layer.n} output columns, "
                      f"every M of the sweep {wl['sweep']}"}


# The rest of each MoE layer (--layer): the down projection (K = half the gate/up width) and
# the activation type between the two products.
LAYERS = {
    "moe_w4a16_mxfp4": dict(down="moe_down_mxfp4", hidden=7168, inter=2048, act="bf16",
                            desc="MoE layer MXFP4 W4A16, E=128 top-8, hidden 7168, intermediate 2048: "
                                 "align + gate/up + SwiGLU + down + combine"),
    "moe_w4a8_mxfp4": dict(down="moe_down_w4a8_mxfp4", hidden=7168, inter=2048, act="e4m3",
                           desc="MoE layer W4A8 MXFP4, E=128 top-8, hidden 7168, intermediate 2048: per-token e4m3 "
                                "quantization of bf16 hidden states + align + gate/up + "
                                "SwiGLU with per-row e4m3 quantization + down + combine"),
    "moe_w4a4_mxfp4": dict(down="moe_down_w4a4_mxfp4", hidden=7168, inter=2048, act="e2m1",
                           desc="MoE layer W4A4 MXFP4, E=128 top-8, hidden 7168, intermediate 2048: MXFP4 "
                                "quantization of bf16 hidden states + align + gate/up + SwiGLU with MXFP4 output "
                                "+ down + combine"),
    "moe_w4a8_int4": dict(down="moe_down_w4a8", hidden=4096, inter=1408, act="e4m3",
                          desc="MoE layer W4A8 int4, E=64 top-6 skewed, hidden 4096, intermediate 1408: per-token "
                               "e4m3 quantization of bf16 hidden states + align + gate/up + SwiGLU with per-row e4m3 "
                               "quantization + down + combine"),
}


def bench_moe_layer(args, wl):
    """Whole MoE layers: (FP8-activation layers: per-token e4m3 quantization of bf16 hidden
    states) -> align -> gate/up product -> SwiGLU -> down product (one row per slot) ->
    routing-weighted combine, each step timed with HIP events on the launch stream."""
    import torch
    import quantized_gemm_amd as qg
    from quantized_gemm_amd import layers, synth

    lw = LAYERS[args.workload]
    moe = wl["moe"]
    topk, experts = moe["topk"], moe["experts"]
    torch.cuda.set_device(0)
    tmax = max(wl["sweep"])
    up, acts = getattr(synth, args.workload)(t=tmax, n=wl["n"], k=wl["k"], seed=0, **moe)
    down = getattr(synth, lw["down"])(experts=experts, n=lw["hidden"], k=lw["inter"], seed=100)
    pu, bu = layers.prepare_layer(up)
    pd, bd = layers.prepare_layer(down)
    copies = args.copies or max(1, int(np.ceil((1 << 30) / (bu.numel() + bd.numel()))))
    hs = [(pu, pd)]
    keep = [bu, bd]
    for _ in range(copies - 1):
        b1, b2 = bu.clone(), bd.clone()
        h1, h2 = qg.Prepared.from_buffer_copy(pu), qg.Prepared.from_buffer_copy(pd)
        h1.dev, h2.dev = b1.data_ptr(), b2.data_ptr()
        keep += [b1, b2]
        hs.append((h1, h2))
    x_all, xs_all = layers.acts_to_dev(acts)
    # FP8-activation layers start from bf16 hidden states, quantized per token on the GPU
    # (timed as the layer's first step)
    q_in = up.a_type in ("e4m3", "e2m1")
    if q_in:
        h_bits, _ = synth.act_rows(tmax, up.k, "bf16", sigma=1.0, seed=7)
        h_all = layers.to_dev(h_bits)
    ids_all = torch.from_numpy(np.ascontiguousarray(acts.topk_ids)).cuda()
    w_all = torch.from_numpy(np.ascontiguousarray(acts.topk_weights)).cuda()
    a_e4m3 = lw["act"] == "e4m3"
    a_e2m1 = lw["act"] == "e2m1"
    st = {}
    for t in wl["sweep"]:
        rows = t * topk
        bm = qg.moe_block_m(pu, t, topk)
        assert qg.moe_block_m(pd, rows, 1) == bm
        cs, cb = qg.moe_capacity(t, topk, experts, bm)
        st[t] = dict(
            bm=bm, sid=torch.empty(cs, dtype=torch.int32, device="cuda"),
            eid=torch.empty(cb, dtype=torch.int32, device="cuda"), npp=torch.empty(1, dtype=torch.int32, device="cuda"),
            ids=ids_all[:t].contiguous(), w=w_all[:t].contiguous(),
            y1=torch.empty((rows, 2 * lw["inter"]), dtype=torch.bfloat16, device="cuda"),
            act=None if a_e2m1 else
            torch.empty((rows, lw["inter"]), dtype=torch.uint8 if a_e4m3 else torch.bfloat16, device="cuda"),
            asc=torch.empty(rows, dtype=torch.float32, device="cuda") if a_e4m3 else
            (torch.empty((rows, lw["inter"] // 32), dtype=torch.uint8, device="cuda") if a_e2m1 else None),
            aq=torch.empty((rows, lw["inter"] // 2), dtype=torch.uint8, device="cuda") if a_e2m1 else None,
            y2=torch.empty((rows, lw["hidden"]), dtype=torch.bfloat16, device="cuda"),
            out=torch.empty((t, lw["hidden"]), dtype=torch.bfloat16, device="cuda"),
            ws1=torch.zeros(max(1, qg.workspace_bytes(pu, t, topk)), dtype=torch.uint8, device="cuda"),
            ws2=torch.zeros(max(1, qg.workspace_bytes(pd, rows, 1)), dtype=torch.uint8, device="cuda"))
    stream = torch.cuda.current_stream()
    names = (["quant"] if q_in else []) + ["align", "gate_up", "swiglu", "down", "combine"]
    call = [0]

    def one_step(ev=None):
        for i, t in enumerate(wl["sweep"]):
            h1, h2 = hs[call[0] % copies]
            call[0] += 1
            d = st[t]
            rows = t * topk
            xs = None if xs_all is None else xs_all[:t]
            nxt = [0]

            def mark():
                if ev is not None:
                    ev[i][nxt[0]].record(stream)
                nxt[0] += 1

            mark()
            x = x_all[:t]
            if q_in:
                if up.a_type == "e2m1":
                    qg.quantize_e2m1_rows(h_all[:t], t, up.k, qg.A_BF16, x, xs)
                else:
                    qg.quantize_e4m3_rows(h_all[:t], t, up.k, qg.A_BF16, x, xs)
                mark()
            qg.moe_align(d["ids"], t, topk, experts, d["bm"], d["sid"], d["eid"], d["npp"])
            mark()
            qg.moe_gemm(h1, x, xs, d["sid"], d["eid"], d["npp"], t, topk, d["bm"], d["y1"], d["ws1"])
            mark()
            a_in = d["aq"] if a_e2m1 else d["act"]
            qg.moe_swiglu(d["y1"], rows, lw["inter"], qg.O_BF16,
                          qg.A_FP8_E4M3 if a_e4m3 else qg.A_FP4_E2M1 if a_e2m1 else qg.A_BF16, a_in, d["asc"])
            mark()
            qg.moe_gemm(h2, a_in, d["asc"], d["sid"], d["eid"], d["npp"], rows, 1, d["bm"], d["y2"], d["ws2"])
            mark()
            qg.moe_combine(d["y2"], d["w"], d["ids"], t, topk, experts, lw["hidden"], qg.O_BF16, d["out"])
            mark()

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in wl["sweep"]]
          for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for s_ in range(args.steps):
        one_step(ev[s_])
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    wb_up, wb_down = weight_bytes(up), weight_bytes(down)
    per_t, flops_step = {}, 0
    peak = MFMA_PEAK_TFLOPS[wl["dtype"]]
    for i, t in enumerate(wl["sweep"]):
        us = {nm: float(np.mean([ev[s_][i][j].elapsed_time(ev[s_][i][j + 1]) for s_ in range(args.steps)])) * 1e3
              for j, nm in enumerate(names)}
        tot = sum(us.values())
        rows = t * topk
        f_up = 2 * rows * up.n * up.k
        f_dn = 2 * rows * down.n * down.k
        flops_step += f_up + f_dn
        touched = len(np.unique(acts.topk_ids[:t]))
        wb = touched * (wb_up + wb_down)
        per_t[str(t)] = {"us": {k: round(v, 2) for k, v in us.items()}, "layer_us": round(tot, 2),
                         "gemm_us": round(us["gate_up"] + us["down"], 2),
                         "tflops_gemms": round((f_up + f_dn) / ((us["gate_up"] + us["down"]) * 1e-6) / 1e12, 2),
                         "tflops_layer": round((f_up + f_dn) / (tot * 1e-6) / 1e12, 2),
                         "weight_GBps_gemms": round(wb / ((us["gate_up"] + us["down"]) * 1e-6) / 1e9, 1),
                         "hbm_frac_gemms": round(wb / ((us["gate_up"] + us["down"]) * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                         "mfma_frac_gemms": round((f_up + f_dn) / ((us["gate_up"] + us["down"]) * 1e-6) / 1e12 / peak, 4),
                         "touched_experts": touched, "block_m": st[t]["bm"]}
    result = {
        "metric": "W4A16 qGEMM TFLOP/s + weight HBM GB/s (% roofline), M=1..4096, dense & MoE",
        "value": round(flops_step / (ms_per_step * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl["dtype"], "data": "synthetic",
        "config": {"workload": lw["desc"], "t_sweep": wl["sweep"], "weight_copies_rotated": copies,
                   "weight_bytes_per_expert": {"gate_up": wb_up, "down": wb_down}},
        "per_t": per_t,
    }
    print(json.dumps(result), flush=True)


def run_workload(args, name, wl):
    """Time one workload's sweep: `warmup` untimed steps, then exactly `steps` timed steps
    (one launch per M of the sweep each), bracketed by device synchronisations; then each
    M alone over `steps` back-to-back launches for the per-launch durations."""
    import torch
    import quantized_gemm_amd as qg
    from quantized_gemm_amd import layers, synth

    builder = getattr(synth, name)
    torch.cuda.set_device(0)
    mmax = max(wl["sweep"])
    moe = wl.get("moe")
    if moe:
        layer, acts = builder(t=mmax, n=wl["n"], k=wl["k"], seed=0, **moe)
    else:
        layer, acts = builder(m=mmax, n=wl["n"], k=wl["k"], seed=0)
    p0, buf0 = layers.prepare_layer(layer)
    wbytes_expert = weight_bytes(layer)
    # weight bytes a launch must stream: the dense layer, or the experts the first m tokens touch
    wbytes_of = {}
    for m in wl["sweep"]:
        if moe:
            touched = len(np.unique(acts.topk_ids[:m]))
            wbytes_of[m] = touched * wbytes_expert
        else:
            wbytes_of[m] = wbytes_expert
    wbytes = wbytes_expert
    copies = args.copies or max(2, int(np.ceil((1 << 30) / buf0.numel())))
    bufs, handles = [buf0], [p0]
    for _ in range(copies - 1):
        b = buf0.clone()
        h = qg.Prepared.from_buffer_copy(p0)
        h.dev = b.data_ptr()
        bufs.append(b)
        handles.append(h)
    x_all, xs_all = layers.acts_to_dev(acts)
    rows_of = {m: m * (moe["topk"] if moe else 1) for m in wl["sweep"]}
    ys = {m: torch.empty((rows_of[m], layer.n), dtype=layers.out_dtype(layer), device="cuda") for m in wl["sweep"]}
    ws = {m: torch.zeros(max(1, qg.workspace_bytes(p0, m, moe["topk"] if moe else 0)), dtype=torch.uint8,
                         device="cuda") for m in wl["sweep"]}
    stream = torch.cuda.current_stream()
    align = {}
    if moe:
        ids_all = torch.from_numpy(np.ascontiguousarray(acts.topk_ids)).cuda()
        for m in wl["sweep"]:
            bm = qg.moe_block_m(p0, m, moe["topk"])
            cs, cb = qg.moe_capacity(m, moe["topk"], moe["experts"], bm)
            align[m] = (bm, torch.empty(cs, dtype=torch.int32, device="cuda"),
                        torch.empty(cb, dtype=torch.int32, device="cuda"), torch.empty(1, dtype=torch.int32, device="cuda"),
                        ids_all[:m].contiguous())

    call = [0]
    # every launch's arguments converted once per (weight copy, M): the timing loops then cost
    # one C call per launch on the host, well under the smallest kernel's GPU time
    launches = {}
    for m in wl["sweep"]:
        xs = None if xs_all is None else xs_all[:m]
        for c, h in enumerate(handles):
            if moe:
                bm, sid, eid, npp, ids = align[m]
                launches[(c, m)] = qg.moe_gemm_call(h, x_all[:m], xs, sid, eid, npp, m, moe["topk"], bm, ys[m], ws[m],
                                                    stream)
            else:
                launches[(c, m)] = qg.gemm_call(h, x_all[:m], xs, ys[m], m, ws[m], stream)

    def one_step(events=None):
        for i, m in enumerate(wl["sweep"]):
            launch = launches[(call[0] % copies, m)]
            call[0] += 1
            if moe:
                bm, sid, eid, npp, ids = align[m]
                if events is not None:
                    events[i][2].record(stream)
                qg.moe_align(ids, m, moe["topk"], moe["experts"], bm, sid, eid, npp, stream)
                if events is not None:
                    events[i][0].record(stream)
            elif events is not None:
                events[i][0].record(stream)
            launch()
            if events is not None:
                events[i][1].record(stream)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()

    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in wl["sweep"]]
          for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(args.steps):
        one_step(ev[s])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps

    # Per-launch durations: each M alone, `steps` back-to-back launches (rotating weight
    # copies) between two events on the launch stream, so that one event pair's overhead is
    # spread over many launches (the figure rocprof's kernel trace gives as the average
    # duration).  The single-launch event pairs of the timed steps are reported beside it.
    batch = {}
    for m in wl["sweep"]:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        seq = [launches[((call[0] + j) % copies, m)] for j in range(args.steps)]
        call[0] += args.steps
        e0.record(stream)
        for launch in seq:
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        batch[m] = e0.elapsed_time(e1) * 1e-3 / args.steps

    flops_step = sum(2 * rows_of[m] * layer.n * layer.k for m in wl["sweep"])
    per_m = {}
    for i, m in enumerate(wl["sweep"]):
        d = np.array([ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)]) * 1e-3
        avg = batch[m]
        fl = 2 * rows_of[m] * layer.n * layer.k
        wb = wbytes_of[m]
        per_m[str(m)] = {"us": round(avg * 1e6, 2), "us_single_launch": round(float(d.mean()) * 1e6, 2),
                         "us_single_median": round(float(np.median(d)) * 1e6, 2),
                         "tflops": round(fl / avg / 1e12, 2), "weight_GBps": round(wb / avg / 1e9, 1),
                         "hbm_frac": round(wb / avg / 1e9 / HBM_PEAK_GBPS, 4),
                         "mfma_frac": round(fl / avg / 1e12 / MFMA_PEAK_TFLOPS[wl["dtype"]], 4)}
        if moe:
            da = np.array([ev[s][i][2].elapsed_time(ev[s][i][0]) for s in range(args.steps)]) * 1e-3
            per_m[str(m)]["align_us"] = round(float(da.mean()) * 1e6, 2)
            per_m[str(m)]["weight_bytes"] = wb
    # dominant kernel = the launch with the largest average duration
    dom = max(wl["sweep"], key=lambda m: per_m[str(m)]["us"])
    dom_s = per_m[str(dom)]["us"] * 1e-6
    dom_flops = 2 * rows_of[dom] * layer.n * layer.k
    # the sweep's bound switches with M: weight bytes bound small M, the MFMA bounds large M
    mfma_bound = dom_flops / (MFMA_PEAK_TFLOPS[wl["dtype"]] * 1e12) > wbytes_of[dom] / (HBM_PEAK_GBPS * 1e9)
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(dom_flops / dom_s / 1e12, 2),
                "peak": MFMA_PEAK_TFLOPS[wl["dtype"]], "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(wbytes_of[dom] / dom_s / 1e9, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(name, dom) if mfma_bound else None
    roof["kernel"] = f"{'qg_moe_gemm T' if moe else 'qg_gemm M'}={dom}"

    result = {
        "metric": "W4A16 qGEMM TFLOP/s + weight HBM GB/s (% roofline), M=1..4096, dense & MoE",
        "value": round(flops_step / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl["dtype"], "data": "synthetic",
        "config": {"workload": wl["desc"], "n": layer.n, "k": layer.k, "m_sweep": wl["sweep"],
                   "weight_bytes": wbytes * layer.experts, "weight_copies_rotated": copies},
        "per_m": per_m,
        "roofline": roof,
    }
    return result, builder, layer


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dense_w4a16_asym_bf16", choices=list(WORKLOADS))
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0: enough for >= 1 GiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-cols", type=int, default=8192)
    ap.add_argument("--sweep", type=str, default="", help="comma-separated M values overriding the workload's sweep")
    ap.add_argument("--layer", action="store_true",
                    help="MoE workloads: time the whole layer (align, gate/up, SwiGLU, down, combine)")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the headline workload (no other workloads, no measured ceilings)")
    ap.add_argument("--ceilings", action="store_true", help="only measure the read and MFMA ceilings")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.ceilings:
        torch.cuda.set_device(0)
        print(json.dumps({"ceilings": measure_ceilings(args)}), flush=True)
        return
    wl = dict(WORKLOADS[args.workload])
    if args.sweep:
        wl["sweep"] = [int(v) for v in args.sweep.split(",")]
    if args.layer:
        if args.workload not in LAYERS:
            print(f"--layer needs an MoE workload ({', '.join(LAYERS)})", file=sys.stderr)
            sys.exit(2)
        bench_moe_layer(args, wl)
        return
    result, builder, layer = run_workload(args, args.workload, wl)
    if not args.no_cpu_baseline and not wl.get("moe"):
        result["cpu_baseline"] = cpu_baseline(builder, wl, min(args.cpu_cols, layer.n))
    if not args.no_extras and args.workload == DEFAULT_WORKLOAD and not args.sweep:
        extras = {}
        for other in EXTRA_WORKLOADS:
            r, _, _ = run_workload(args, other, dict(WORKLOADS[other]))
            extras[other] = {key: r[key] for key in ("value", "unit", "ms_per_step", "dtype", "per_m", "roofline")}
            extras[other]["workload"] = r["config"]["workload"]
            torch.cuda.empty_cache()
        result["other_workloads"] = extras
        result["ceilings"] = measure_ceilings(args)
        roof = result["roofline"]
        ceil = result["ceilings"]["mfma_tflops"].get(wl["dtype"]) if roof["bound"] == "mfma" else \
            result["ceilings"]["read_GBps"]
        if ceil:
            roof["measured_ceiling"] = ceil
            roof["frac_of_measured"] = round(roof["achieved"] / ceil, 4)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
