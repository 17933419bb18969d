"""Benchmark of the MoE expert layer on one MI355X.

Workload: the FP8 decode layer (H=4096, E=64, top-8, I=1536, e4m3 weights
with 128x128 fp32 block scales, per-token per-128 FP8 activations, uniform
routing), swept over T in {1, 8, 32, 64, 128, 256} tokens.  One step is one
moe_layer call at every T of the sweep plus one stage-by-stage pass at the
roofline point (T=64).  Before every timed call a 1 GiB buffer is read (a
reduction: the caches refill with clean lines, so no write-back lands in the
timed region) so that neither L2 nor the 256 MB memory-side cache holds the
weights; a warm call right after is timed too, as a diagnostic.  Inputs are synthetic,
seeded, and resident in HBM before timing starts.

Output: one JSON line.  value = aggregate effective weight bandwidth over
the sweep (touched-expert weight bytes / HIP-event layer time).  After the
timed decode steps, a "prefill" section measures the MXFP4 layer at T=4096
(H=7168, E=256, top-8, I=2048): layer latency and TFLOP/s, per-stage times,
and GEMM1's rate against the MFMA peak of its operand formats.
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

HBM_PEAK_GBS = 8000.0
# dense MFMA peak for an e2m1 x e4m3 contraction: the scaled MFMA takes the
# FP8 rate when either operand is FP8 (MI355X dense FP8: 5.0 PFLOP/s)
MFMA_PEAK_TFLOPS = 5000.0
FP4_PEAK_TFLOPS = 10100.0
FLUSH_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm1_decode_fp8_T64.json")
KERNEL_SRC = os.path.join(ROOT, "bit_grouped_gemm_amd", "csrc", "moe_kernels.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_fp8")
    ap.add_argument("--tokens", default=None, help="comma-separated T values (default: the workload's sweep)")
    ap.add_argument("--roofline-T", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the T=4096 MXFP4 prefill section")
    ap.add_argument("--prefill-reps", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle timing")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (3 times): the known-size "
                         "reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def kernel_sha() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(workload: str, T: int):
    """HBM bytes per GEMM1 launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source and on this workload and T;
    else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_src_sha") != kernel_sha() or t.get("workload") != f"{workload} T={T}":
        return None
    return float(t["hbm_bytes_per_launch"])


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the layer is one GPU's "
              "share of an expert-parallel MoE and no multi-GPU path is built", file=sys.stderr)
        sys.exit(2)
    import torch

    import bit_grouped_gemm_amd as moe
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_mib:
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": args.copy_mib << 20, "launches": 3}))
        return
    moe.load()
    wl = synth.WORKLOADS[args.workload]
    Ts = [int(t) for t in args.tokens.split(",")] if args.tokens else list(wl.tokens)
    RT = args.roofline_T if args.roofline_T in Ts else Ts[len(Ts) // 2]

    t0 = time.time()
    w_rowmajor = synth.gen_weights(wl, seed=0, device=dev)
    # one-time reorder into the tiled layout the GEMMs read (weight load time, not timed)
    w = moe.moe_prepack_weights(moe.Cfg.for_workload(wl, 1), w_rowmajor)
    cases = {}
    for T in Ts:
        x, ids, tw = synth.gen_inputs(wl, T, seed=0, device=dev)
        cfg = moe.Cfg.for_workload(wl, T)
        ws = moe.workspace(cfg, dev)
        out = torch.empty(T, wl.H, dtype=torch.bfloat16, device=dev)
        wbytes = synth.weight_bytes_touched(wl, w_rowmajor, ids)
        cases[T] = dict(x=x, ids=ids, tw=tw, cfg=cfg, ws=ws, out=out, wbytes=wbytes,
                        touched=synth.touched_experts(ids, wl.E), flops=synth.layer_flops(wl, T, ids))
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def one_step(rec):
        for T in Ts:
            c = cases[T]
            flush.sum(dtype=torch.int64)
            a, b, d, e = ev(), ev(), ev(), ev()
            a.record(stream)
            moe.moe_layer(c["cfg"], c["x"], c["ids"], c["tw"], w, ws=c["ws"], out=c["out"])
            b.record(stream)
            d.record(stream)
            moe.moe_layer(c["cfg"], c["x"], c["ids"], c["tw"], w, ws=c["ws"], out=c["out"])
            e.record(stream)
            if rec is not None:
                rec["layer"][T].append((a, b))
                rec["warm"][T].append((d, e))
        # stage-by-stage pass at the roofline point: each kernel bracketed by events
        c = cases[RT]
        flush.sum(dtype=torch.int64)
        evs = [ev() for _ in range(5)]
        evs[0].record(stream)
        counts, offsets, eidx, rtok, xq, xs = moe.moe_permute(c["cfg"], c["x"], c["ids"])
        evs[1].record(stream)
        hq, hs = moe.moe_grouped_gemm1_swiglu(c["cfg"], xq, xs, rtok, offsets, w, c["ws"])
        evs[2].record(stream)
        y = moe.moe_grouped_gemm2(c["cfg"], hq, hs, offsets, w, c["ws"])
        evs[3].record(stream)
        moe.moe_combine(c["cfg"], y, eidx, offsets, c["tw"])
        evs[4].record(stream)
        if rec is not None:
            rec["stages"].append(evs)

    for _ in range(args.warmup):
        one_step(None)
    rec = {"layer": {T: [] for T in Ts}, "warm": {T: [] for T in Ts}, "stages": []}
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        one_step(rec)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start

    ms = lambda p: p[0].elapsed_time(p[1])
    sweep = {}
    tot_bytes = tot_ms = 0.0
    for T in Ts:
        lat = np.array([ms(p) for p in rec["layer"][T]]) * 1e3   # us
        warm = np.array([ms(p) for p in rec["warm"][T]]) * 1e3
        c = cases[T]
        med = float(np.median(lat))
        sweep[str(T)] = {
            "latency_us_median": round(med, 2), "latency_us_p10": round(float(np.percentile(lat, 10)), 2),
            "latency_us_p90": round(float(np.percentile(lat, 90)), 2),
            "warm_latency_us_median": round(float(np.median(warm)), 2),
            "touched_experts": c["touched"], "weight_bytes": c["wbytes"],
            "weight_GBps": round(c["wbytes"] / med / 1e3, 1),
            "hbm_frac": round(c["wbytes"] / med / 1e3 / HBM_PEAK_GBS, 4),
            "TFLOPs": round(c["flops"] / med / 1e6, 2),
        }
        tot_bytes += c["wbytes"] * len(lat)
        tot_ms += float(lat.sum()) / 1e3
    value = tot_bytes / (tot_ms * 1e-3) / 1e9

    st = np.array([[rec_ev[i].elapsed_time(rec_ev[i + 1]) for i in range(4)] for rec_ev in rec["stages"]]) * 1e3
    stage_us = {n: round(float(np.mean(st[:, i])), 2) for i, n in
                enumerate(["permute_quant", "gemm1_swiglu", "gemm2", "combine"])}
    # algorithmic bytes of one GEMM1 launch at the roofline point: W1 codes + scales of every
    # touched expert, the FP8 activations and their scales read, the requantised h written
    c = cases[RT]
    e1 = w.w1[0].numel() * w.w1.element_size() + w.w1s[0].numel() * w.w1s.element_size()
    T = RT
    R = int(((c["ids"] >= 0) & (c["ids"] < wl.E)).sum().item())
    g1_bytes = c["touched"] * e1 + T * wl.H + T * (wl.H // wl.act_group) * 4 + R * wl.I + R * (wl.I // wl.act_group) * 4
    g1_us = stage_us["gemm1_swiglu"]
    achieved = g1_bytes / g1_us / 1e3
    traffic = load_traffic(wl.name, RT)
    stream_gbs = stream_read_gbs(moe, flush, stream, ev)

    line = {
        "metric": "MoE layer latency (us) + weight GB/s vs HBM peak at T=1..256; TFLOP/s at T=4096",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3" if wl.wfmt == synth.FMT_FP8 else "fp8e4m3 x e2m1",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights quantised, uniform top-k routing)",
        "config": {"workload": f"{wl.name}: H={wl.H} E={wl.E} top-{wl.topk} I={wl.I} "
                               f"{'e4m3 128x128-block' if wl.wfmt == 0 else 'MXFP4'} weights, "
                               f"T sweep {','.join(map(str, Ts))}, cold caches",
                   "tokens": Ts, "roofline_T": RT},
        "sweep": sweep,
        "stages_us_at_roofline_T": stage_us,
        "roofline": {"kernel": "k_gemm1 (grouped GEMM1 + SwiGLU + requant)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "algorithmic_bytes": int(g1_bytes), "avg_launch_us": g1_us,
                     "stream_read_GBps": round(stream_gbs, 1),
                     "frac_of_stream_read": round(achieved / stream_gbs, 4)},
        "setup_s": round(setup_s, 1),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, w_rowmajor, cases[RT], RT, args.cpu_seconds)
    if not args.no_prefill:
        del cases, w, w_rowmajor, flush
        torch.cuda.empty_cache()
        line["prefill"] = prefill(moe, synth, torch, dev, args.prefill_reps)
    print(json.dumps(line), flush=True)


def prefill(moe, synth, torch, dev, reps):
    """The MXFP4 layer at T=4096: its 6 GB of weights exceed every cache, so
    each call streams them from HBM."""
    wl = synth.WORKLOADS["prefill_mxfp4"]
    T = wl.tokens[0]
    w_rm = synth.gen_weights(wl, seed=0, device=dev)
    w = moe.moe_prepack_weights(moe.Cfg.for_workload(wl, 1), w_rm)
    wbytes_all = w_rm.nbytes_expert() * wl.E
    del w_rm
    x, ids, tw = synth.gen_inputs(wl, T, seed=0, device=dev)
    cfg = moe.Cfg.for_workload(wl, T)
    ws = moe.workspace(cfg, dev)
    out = torch.empty(T, wl.H, dtype=torch.bfloat16, device=dev)
    flops = synth.layer_flops(wl, T, ids)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    for _ in range(2):
        moe.moe_layer(cfg, x, ids, tw, w, ws=ws, out=out)
    lat, st = [], []
    for _ in range(reps):
        a, b = ev(), ev()
        a.record()
        moe.moe_layer(cfg, x, ids, tw, w, ws=ws, out=out)
        b.record()
        lat.append((a, b))
        e = [ev() for _ in range(5)]
        e[0].record()
        _, offsets, eidx, rtok, xq, xs = moe.moe_permute(cfg, x, ids, ws)
        e[1].record()
        hq, hs = moe.moe_grouped_gemm1_swiglu(cfg, xq, xs, rtok, offsets, w, ws)
        e[2].record()
        y = moe.moe_grouped_gemm2(cfg, hq, hs, offsets, w, ws)
        e[3].record()
        moe.moe_combine(cfg, y, eidx, offsets, tw)
        e[4].record()
        st.append(e)
        del y
    torch.cuda.synchronize()
    lat_us = np.array([a.elapsed_time(b) for a, b in lat]) * 1e3
    stg = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(4)] for e in st]) * 1e3
    med = float(np.median(lat_us))
    stages = {n: round(float(np.median(stg[:, i])), 1) for i, n in
              enumerate(["permute_quant", "gemm1_swiglu", "gemm2_fp32y", "combine_fp32y"])}
    R = T * wl.topk
    g1_flops = 2.0 * R * (2 * wl.I) * wl.H
    g1_tf = g1_flops / (stages["gemm1_swiglu"] * 1e-6) / 1e12
    tf = flops / (med * 1e-6) / 1e12
    meas = mfma_rate_tflops(moe, torch, dev, 1)
    # floor of the layer on HBM: every weight byte + x in + out, at the peak
    act_bytes = 2 * 2 * T * wl.H
    hbm_floor_us = (wbytes_all + act_bytes) / (HBM_PEAK_GBS * 1e9) * 1e6
    return {
        "workload": f"{wl.name}: H={wl.H} E={wl.E} top-{wl.topk} I={wl.I} MXFP4 weights, T={T}",
        "layer_us_median": round(med, 1), "layer_us_p10": round(float(np.percentile(lat_us, 10)), 1),
        "layer_us_p90": round(float(np.percentile(lat_us, 90)), 1),
        "TFLOPs": round(tf, 1), "mfma_peak_TFLOPs": MFMA_PEAK_TFLOPS, "mfma_frac": round(tf / MFMA_PEAK_TFLOPS, 4),
        "weight_GBps": round(wbytes_all / (med * 1e-6) / 1e9, 1),
        "stages_us_median": stages,
        "gemm1_TFLOPs": round(g1_tf, 1), "gemm1_mfma_frac": round(g1_tf / MFMA_PEAK_TFLOPS, 4),
        "mfma_measured_TFLOPs": round(meas, 1),
        "mfma_frac_of_measured": round(tf / meas, 4), "gemm1_frac_of_measured": round(g1_tf / meas, 4),
        "fp4_peak_frac": round(tf / FP4_PEAK_TFLOPS, 4),
        "hbm_floor_us": round(hbm_floor_us, 1), "hbm_floor_frac": round(hbm_floor_us / med, 4),
        "reps": reps,
        "note": "stage times use the stage exports (fp32 y); moe_layer keeps y in bf16",
    }


def mfma_rate_tflops(moe, torch, dev, wfmt, iters=4096):
    """Issued rate of the scaled MFMA the prefill GEMMs run (wfmt 1: e2m1
    weights x e4m3 activations), from the library's rate probe: median of
    five timed launches of about a millisecond after one untimed one."""
    sink = torch.empty(8192, dtype=torch.float32, device=dev)
    moe.moe_mfma_rate(wfmt, iters, sink)
    ts, fl = [], 0.0
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fl = moe.moe_mfma_rate(wfmt, iters, sink)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    ts.sort()
    return fl / (ts[len(ts) // 2] * 1e-3) / 1e12


def stream_read_gbs(moe, buf, stream, ev):
    """Achievable HBM read rate on this part: the library's plain read stream
    over the 1 GiB eviction buffer (larger than every cache), median of five
    timed passes after one untimed pass."""
    import torch
    sink = torch.empty(8192, dtype=torch.int32, device=buf.device)
    moe.moe_stream_read(buf, sink)
    ts = []
    for _ in range(5):
        a, b = ev(), ev()
        a.record(stream)
        moe.moe_stream_read(buf, sink)
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    ts.sort()
    return buf.numel() * buf.element_size() / (ts[len(ts) // 2] * 1e-3) / 1e9


def cpu_baseline(wl, w, c, T, budget_s):
    """The CPU oracle, as it stands, on a bounded sample of tokens of the
    roofline-point layer; scaled to effective weight GB/s of the full layer."""
    import oracle
    oracle.build(force=False)
    wc = w.to("cpu")
    x, ids, tw = c["x"].cpu(), c["ids"].cpu(), c["tw"].cpu()
    lay = oracle.layer_for(wl, T, wc)
    n = 1
    t = 0.0
    while True:
        t0 = time.perf_counter()
        lay.layer(x, ids, tw, toks=list(range(n)))
        t = time.perf_counter() - t0
        if t * 2.5 > budget_s or n * 2 > T:
            break
        n *= 2
    if n == T and t < 10.0:
        # the whole layer fits: time whole passes until about 10 s of CPU work
        reps = max(1, int(10.0 / max(t, 1e-3)) + 1)
        t0 = time.perf_counter()
        for _ in range(reps):
            lay.layer(x, ids, tw, toks=list(range(n)))
        tot = time.perf_counter() - t0
        full_s = tot / reps
        sample = f"the whole T={T} layer, {reps} passes ({tot:.1f} s), {full_s:.1f} s per pass"
    else:
        full_s = t * T / n
        sample = f"{n} of {T} tokens of the T={T} layer ({t:.1f} s), scaled by T/{n} to {full_s:.1f} s for the whole layer"
    return {"value": round(c["wbytes"] / full_s / 1e9, 4), "unit": "GB/s", "cores": oracle.threads(),
            "kind": "oracle", "sample": sample}


if __name__ == "__main__":
    main()
