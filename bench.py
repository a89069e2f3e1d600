#!/usr/bin/env python3
"""Benchmark of the MoE layer forward on one MI355X.

One step is one pass of the whole path over one batch: route (logit GEMM +
KeepTopK/softmax), dispatch (histogram, capacity, permute), the SwiGLU
grouped GEMMs (gate/up, then down) and the combine, each through its C-ABI
entry point on one stream.  HIP events recorded on that stream around every
stage give per-stage durations over the timed region; the dominant kernel's
roofline is computed from its algorithmic bytes and flops.  Each stage's
byte rate is also given as a fraction of this device's own streaming-read
rate, measured after the timed steps with moe_stream_read.

For a dropless workload spread over D > 1 ranks, the expert GEMMs are also
timed on one rank's share under D-way expert parallelism (E/D experts, the
rows of D batches), where the grouped GEMM is bound by the matrix cores
rather than by streaming the weights.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, TFLOP/s
METRIC = "MoE layer tokens/s + grouped-GEMM MFMA util, DeepSeek-V3-shaped T=4096"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def stage_traffic(cfg, st, touched):
    """Algorithmic HBM bytes and flops of each stage for one call."""
    T, d, E, k, H = cfg.T, cfg.d, cfg.E, cfg.k, cfg.H
    kept, send_rows = st["kept"], st["send_rows"]
    row = d + 4 if cfg.dispatch_fp8 else d * 2   # a dispatched row: E4M3 + scale, or bf16
    return {
        "route": dict(bytes=T * d * 2 + d * E * 2 + T * k * 8, flops=2 * T * d * E),
        "dispatch": dict(bytes=T * d * 2 + send_rows * row + T * k * 8, flops=0),
        "gate_up": dict(bytes=touched * 2 * H * d * 2 + kept * row + kept * H * 2,
                        flops=4 * kept * d * H),
        "down": dict(bytes=touched * d * H * 2 + kept * H * 2 + kept * d * 2,
                     flops=2 * kept * d * H),
        "combine": dict(bytes=kept * d * 2 + T * d * 2 + T * k * 8
                        + (T * d * 2 if cfg.shared_H else 0), flops=0),
        "shared": dict(bytes=3 * cfg.shared_H * d * 2 + T * d * 2 * 2 + T * cfg.shared_H * 2 * 2,
                       flops=6 * T * d * cfg.shared_H),
    }


def kernel_source_digest():
    h = hashlib.sha256()
    for name in ("ffn.hip", "moe_internal.hpp", "ring.hpp"):
        with open(os.path.join(ROOT, "expert_token_routing_moe_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    ent = rec.get(workload, {}).get(kernel)
    if not ent or ent.get("source_digest") != kernel_source_digest():
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(cfg, inp, budget_s):
    """The oracle as it stands, on the first tokens of the same workload."""
    import numpy as np

    import oracle
    from expert_token_routing_moe_amd.inputs import bf16_bits

    x = bf16_bits(inp["x"])
    wg = bf16_bits(inp["w_gate"])
    bias = None if inp["bias"] is None else inp["bias"].cpu().numpy()
    experts = {}
    shared = (tuple(bf16_bits(inp[n]) for n in ("w1s", "w3s", "w2s")) if cfg.shared_H
              else None)
    batch = 16
    done, spent = 0, 0.0
    while done < cfg.T and spent < budget_s:
        xb = x[done:done + batch]
        tb = xb.shape[0]
        t0 = time.perf_counter()
        lg = oracle.logits(xb, wg, bias)
        idx, w, _ = oracle.topk(lg, cfg.k, cfg.n_groups, cfg.group_limit)
        r = oracle.dispatch(xb, idx, T=tb, d=cfg.d, E=cfg.E, D=cfg.D, cf=cfg.cf,
                            drop_policy=cfg.drop_policy, topk_w=w, min_capacity=cfg.min_capacity,
                            fp8=bool(cfg.dispatch_fp8))
        spent += time.perf_counter() - t0
        need = [e for e in range(cfg.E) if r["expert_kept"][e] and e not in experts]
        for e in need:  # weight copies to the host are not oracle work: not timed
            experts[e] = tuple(bf16_bits(inp[n][e]) for n in ("w1", "w3", "w2"))
        t0 = time.perf_counter()
        # the experts' weights by index (only experts with kept rows are read)
        w1, w3, w2 = ({e: v[i] for e, v in experts.items()} for i in range(3))
        eo = oracle.expert_ffn_all(r["send_buf"], r["expert_offset"], r["expert_kept"],
                                   w1, w3, w2, send_scale=r["send_scale"])
        so = oracle.expert_ffn(xb, *shared) if shared else None
        oracle.combine(eo, r["slot"], w, so)
        spent += time.perf_counter() - t0
        done += tb
        log(f"  cpu oracle: {done} tokens in {spent:.1f} s")
    return dict(value=done / spent, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"first {done} of {cfg.T} tokens of the {cfg.name} workload, in batches "
                       f"of {batch}: route, dispatch, SwiGLU experts and combine in fp64 "
                       f"({spent:.1f} s of oracle compute)")


def pct(v, q):
    v = sorted(v)
    return v[min(len(v) - 1, int(round(q * (len(v) - 1))))]


def rank_local_gemm(cfg, inp, dev, steps, warmup):
    """The expert GEMMs on one rank's share under D-way expert parallelism.

    Every rank's batch (D * T tokens) is routed and dispatched; rank 0's E/D
    experts then hold the rows that the dispatch all-to-all would deliver to
    it (about D * T * k / E rows each), which is the shape one GPU multiplies
    when the layer is spread over D GPUs.  Both grouped GEMMs run on those
    rows through the same entry points with E/D experts.
    """
    import torch

    from expert_token_routing_moe_amd import api
    from expert_token_routing_moe_amd.inputs import make_inputs

    big = cfg.with_(T=cfg.T * cfg.D)
    xin = make_inputs(big, dev, experts=False)
    shape = api.Shape.from_config(big)
    buf = api.LayerBuffers.allocate(shape, dev, keep_logits=False)
    stream = torch.cuda.current_stream()
    api.moe_route(shape, xin["x"], xin["w_gate"], xin["bias"], None, buf.topk_idx, buf.topk_w,
                  buf.workspace, stream)
    api.moe_dispatch(shape, xin["x"], buf.topk_idx, buf.topk_w, buf.send_buf, buf.send_scale,
                     buf.slot, buf.expert_count,
                     buf.expert_kept, buf.expert_offset, buf.rank_rows, buf.stats,
                     buf.workspace, stream)
    el = cfg.E // cfg.D
    loc = api.Shape(big.T, cfg.d, el, cfg.k, cfg.H, 1, 0, big.cf,
                    dispatch_fp8=big.dispatch_fp8)
    rows = int(buf.expert_offset[el].item())
    h = torch.empty(buf.send_buf.shape[0], cfg.H, dtype=torch.bfloat16, device=dev)
    w1, w3, w2 = inp["w1"][:el], inp["w3"][:el], inp["w2"][:el]

    def run(ev=None):
        if ev:
            ev[0].record(stream)
        api.moe_expert_gate_up(loc, buf.send_buf, buf.send_scale, buf.expert_offset,
                               buf.expert_kept, w1, w3, h, stream, workspace=buf.workspace)
        if ev:
            ev[1].record(stream)
        api.moe_expert_down(loc, h, buf.expert_offset, buf.expert_kept, w2, buf.expert_out,
                            stream)
        if ev:
            ev[2].record(stream)

    for _ in range(warmup):
        run()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        run(evs[i])
    torch.cuda.synchronize()
    gu = [e[0].elapsed_time(e[1]) for e in evs]
    dn = [e[1].elapsed_time(e[2]) for e in evs]
    tot = [a + b for a, b in zip(gu, dn)]
    flops = 6 * cfg.d * cfg.H * rows
    wbytes = 3 * el * cfg.d * cfg.H * 2
    t = pct(tot, 0.5) / 1e3
    res = dict(
        experts=el, rows=rows, tokens_routed=big.T,
        gate_up_ms=round(pct(gu, 0.5), 4), down_ms=round(pct(dn, 0.5), 4),
        ms_p10=round(pct(tot, 0.1), 4), ms_p50=round(pct(tot, 0.5), 4),
        ms_p90=round(pct(tot, 0.9), 4),
        tflops=round(flops / t / 1e12, 1),
        mfma_util=round(flops / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        weight_gbs=round(wbytes / t / 1e9, 1))
    del buf, h, xin
    torch.cuda.empty_cache()
    return res


def device_read_rate(dev, stream):
    """Streaming-read rate of this device, GB/s: the best of five reads of a
    2 GiB buffer through moe_stream_read (the expert GEMMs' non-temporal
    16-byte loads), timed with events on the given stream."""
    import torch

    from expert_token_routing_moe_amd import api

    n = 1 << 31
    src = torch.ones(n // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    api.moe_stream_read(src, sink, stream)  # warm-up
    best = float("inf")
    for _ in range(5):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        api.moe_stream_read(src, sink, stream)
        e1.record(stream)
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del src
    return n / (best / 1e3) / 1e9


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3_prefill")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--drop-policy", type=int, default=None, choices=(0, 1),
                    help="capacity overflow: 0 token order, 1 by gate value (default: the workload's)")
    ap.add_argument("--min-capacity", type=int, default=None,
                    help="lower bound on the expert capacity (default: the workload's)")
    ap.add_argument("--dispatch-fp8", action="store_true",
                    help="dispatch payload as E4M3 rows with fp32 row scales (combine stays bf16)")
    ap.add_argument("--groups", type=int, default=None, metavar="G",
                    help="group-limited routing: G expert groups (with --group-limit)")
    ap.add_argument("--group-limit", type=int, default=None, metavar="M",
                    help="group-limited routing: at most M groups per token")
    ap.add_argument("--shared-expert", type=int, default=None, metavar="H",
                    help="add a replicated shared expert of SwiGLU hidden size H")
    ap.add_argument("--no-rank-local", action="store_true",
                    help="skip the expert-parallel rank-local GEMM measurement")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (scale reference for HBM counters)")
    ap.add_argument("--flush-mall", action="store_true",
                    help="read a 512 MiB buffer before every timed step, so the 256 MB "
                         "last-level cache holds nothing of the previous step; the step time "
                         "is then the sum of the stages' event times, without the read")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU's share of the MoE layer; the library has no "
              "multi-GPU path (the expert-parallel exchange is not implemented); use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from expert_token_routing_moe_amd import api
    from expert_token_routing_moe_amd.inputs import CONFIGS, make_inputs

    cfg = CONFIGS[args.workload]
    if args.drop_policy is not None:
        cfg = cfg.with_(drop_policy=args.drop_policy)
    if args.min_capacity is not None:
        cfg = cfg.with_(min_capacity=args.min_capacity)
    if args.dispatch_fp8:
        cfg = cfg.with_(dispatch_fp8=1)
    if args.groups is not None:
        cfg = cfg.with_(n_groups=args.groups, group_limit=args.group_limit or 1)
    if args.shared_expert is not None:
        cfg = cfg.with_(shared_H=args.shared_expert)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"bench: {cfg.name} T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} H={cfg.H} cf={cfg.cf}")
    inp = make_inputs(cfg, dev)
    shape = api.Shape.from_config(cfg)
    buf = api.LayerBuffers.allocate(shape, dev, keep_logits=False)
    h = torch.empty(max(buf.send_buf.shape[0], 0), cfg.H, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    stages = ["route", "dispatch", "gate_up", "down"]
    if cfg.shared_H:
        stages.append("shared")
    stages.append("combine")

    def step(ev=None):
        marks = iter(range(len(stages) + 1))
        rec = (lambda: ev[next(marks)].record(stream)) if ev else (lambda: None)
        rec()
        api.moe_route(shape, inp["x"], inp["w_gate"], inp["bias"], None, buf.topk_idx,
                      buf.topk_w, buf.workspace, stream)
        rec()
        api.moe_dispatch(shape, inp["x"], buf.topk_idx, buf.topk_w, buf.send_buf,
                         buf.send_scale, buf.slot, buf.expert_count, buf.expert_kept, buf.expert_offset, buf.rank_rows,
                         buf.stats, buf.workspace, stream)
        rec()
        api.moe_expert_gate_up(shape, buf.send_buf, buf.send_scale, buf.expert_offset,
                               buf.expert_kept, inp["w1"], inp["w3"], h, stream,
                               workspace=buf.workspace)
        rec()
        api.moe_expert_down(shape, h, buf.expert_offset, buf.expert_kept, inp["w2"],
                            buf.expert_out, stream)
        rec()
        if cfg.shared_H:
            api.moe_shared_expert(shape, inp["x"], inp["w1s"], inp["w3s"], inp["w2s"],
                                  buf.shared_out, buf.workspace, stream)
            rec()
        api.moe_combine(shape, buf.expert_out, buf.slot, buf.topk_w, buf.shared_out, buf.y,
                        stream)
        rec()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"bench: warmup {args.warmup} done")
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    scratch = (torch.ones(128 << 20, dtype=torch.float32, device=dev) if args.flush_mall
               else None)
    t0 = time.perf_counter()
    for i in range(args.steps):
        if scratch is not None:
            scratch.sum()  # reads 512 MiB: clean lines, nothing left to write back
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    if scratch is not None:  # the stages' own time, without the reads between steps
        ms_step = sum(e[j].elapsed_time(e[j + 1]) for e in events
                      for j in range(len(stages))) / args.steps
    samples = {s: [events[i][j].elapsed_time(events[i][j + 1]) for i in range(args.steps)]
               for j, s in enumerate(stages)}
    stage_ms = {s: sum(v) / len(v) for s, v in samples.items()}
    log(f"bench: {args.steps} steps, {ms_step:.3f} ms/step; stages (ms): "
        + ", ".join(f"{s}={v:.4f}" for s, v in stage_ms.items()))

    st = api.stats_dict(buf.stats)
    touched = int((buf.expert_kept > 0).sum().item())
    traffic = stage_traffic(cfg, st, touched)
    read_gbs = device_read_rate(dev, stream)
    log(f"bench: streaming read on this device {read_gbs:.0f} GB/s")
    per_stage = {}
    for s in stages:
        t = stage_ms[s] / 1e3
        per_stage[s] = dict(ms=round(stage_ms[s], 5),
                            p10=round(pct(samples[s], 0.1), 5),
                            p50=round(pct(samples[s], 0.5), 5),
                            p90=round(pct(samples[s], 0.9), 5),
                            gbs=round(traffic[s]["bytes"] / t / 1e9, 1),
                            hbm_frac=round(traffic[s]["bytes"] / t / 1e9 / HBM_PEAK_GBS, 4),
                            read_frac=round(traffic[s]["bytes"] / t / 1e9 / read_gbs, 4),
                            tflops=round(traffic[s]["flops"] / t / 1e12, 2))
    dom = max(("gate_up", "down"), key=lambda s: stage_ms[s])
    t_dom = stage_ms[dom] / 1e3
    intensity = traffic[dom]["flops"] / traffic[dom]["bytes"]
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if intensity < ridge:
        achieved = traffic[dom]["bytes"] / t_dom / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s")
    else:
        achieved = traffic[dom]["flops"] / t_dom / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=MFMA_BF16_PEAK_TFLOPS,
                    unit="TFLOP/s")
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    if roof["bound"] == "hbm":  # against what this device's reads reach
        roof["device_read_gbs"] = round(read_gbs, 1)
        roof["frac_of_device_read"] = round(roof["achieved"] / read_gbs, 4)
    roof["traffic"] = measured_traffic(dom, cfg.name)
    roof["kernel"] = f"grouped_gemm {dom}"
    gemm_flops = traffic["gate_up"]["flops"] + traffic["down"]["flops"]
    gemm_s = (stage_ms["gate_up"] + stage_ms["down"]) / 1e3
    # load imbalance (max - mean) / mean, over experts (routed counts) and over
    # destination ranks (kept rows), from the device counters and rank rows
    counts = {k: st[k] for k in ("kept", "dropped", "padded", "max_expert_count")}
    rank_rows = buf.rank_rows.cpu().tolist()
    mean_e = st["assignments"] / cfg.E
    mean_r = sum(rank_rows) / len(rank_rows)
    counts["imbalance"] = {
        "expert": round((st["max_expert_count"] - mean_e) / mean_e, 4) if mean_e else 0.0,
        "rank": round((max(rank_rows) - mean_r) / mean_r, 4) if mean_r else 0.0,
    }
    out = {
        "metric": METRIC,
        "value": round(cfg.T / (ms_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "E": cfg.E, "k": cfg.k,
                   "H": cfg.H, "capacity_factor": None if cfg.cf == float("inf") else cfg.cf,
                   "drop_policy": cfg.drop_policy, "min_capacity": cfg.min_capacity,
                   "dispatch_fp8": cfg.dispatch_fp8, "n_groups": cfg.n_groups,
                   "group_limit": cfg.group_limit, "shared_H": cfg.shared_H,
                   "D": cfg.D, "parallelism": "single GPU share (EP rank-local layout)",
                   "mall_flush": bool(args.flush_mall)},
        "grouped_gemm": {"tflops": round(gemm_flops / gemm_s / 1e12, 1),
                         "mfma_util": round(gemm_flops / gemm_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                         "touched_experts": touched},
        "stages": per_stage,
        "counts": counts,
        "roofline": roof,
    }
    if cfg.D > 1 and cfg.cf == float("inf") and not args.no_rank_local:
        log(f"bench: rank-local expert GEMMs ({cfg.E // cfg.D} experts, {cfg.D}x tokens routed)")
        out["grouped_gemm_rank_local"] = rank_local_gemm(cfg, inp, dev, args.steps, args.warmup)
    if args.copy_calibration:
        # a plain device copy of known size: its FETCH_SIZE / WRITE_SIZE counter
        # readings give the scale factor for the counters of the kernels above
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = n
        del src, dst
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
