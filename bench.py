#!/usr/bin/env python3
"""Benchmark of the MoE layer forward on one MI355X.

One step is one pass of the whole path over one batch: route (logit GEMM +
KeepTopK/softmax), dispatch (histogram, capacity, permute), the SwiGLU
grouped GEMMs (gate/up, then down) and the combine, each through its C-ABI
entry point on one stream.  HIP events recorded on that stream around every
stage give per-stage durations over the timed region; the dominant kernel's
roofline is computed from its algorithmic bytes and flops.  Each stage's
byte rate is also given as a fraction of this device's own streaming-read
rate (read_frac), and as device_frac: the stage's reads at that rate plus
its writes at the device's streaming-store rate, over the stage's time.
Both rates are measured after the timed steps (moe_stream_read and
moe_stream_write, the non-temporal 16-byte accesses of the kernels), and
the combine is set beside moe_stream_gather, its own access pattern with
none of its arithmetic, on the same expert outputs and slots.

For a dropless workload spread over D > 1 ranks, the expert GEMMs are also
timed on one rank's share under D-way expert parallelism (E/D experts, the
rows of D batches), where the grouped GEMM is bound by the matrix cores
rather than by streaming the weights.

Before every timed step a 512 MiB buffer is read, so the 256 MB last-level
cache holds nothing of the previous step (--no-flush-mall turns that off);
the step time is then the sum of the stages' event times.

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
    """Algorithmic HBM bytes (read and written) and flops of each stage for one call."""
    T, d, E, k, H = cfg.T, cfg.d, cfg.E, cfg.k, cfg.H
    kept, send_rows = st["kept"], st["send_rows"]
    row = d + 4 if cfg.dispatch_fp8 else d * 2   # a dispatched row: E4M3 + scale, or bf16
    sH = cfg.shared_H
    rec = {
        # x and W_g read; top-k indices and weights written
        "route": dict(read=T * d * 2 + d * E * 2, write=T * k * 8, flops=2 * T * d * E),
        # x and the top-k indices read; send rows and slots written
        "dispatch": dict(read=T * d * 2 + T * k * 4, write=send_rows * row + T * k * 4, flops=0),
        "gate_up": dict(read=touched * 2 * H * d * 2 + kept * row, write=kept * H * 2,
                        flops=4 * kept * d * H),
        "down": dict(read=touched * d * H * 2 + kept * H * 2, write=kept * d * 2,
                     flops=2 * kept * d * H),
        # expert outputs, slots and gates (and the shared expert's output) read; y written
        "combine": dict(read=kept * d * 2 + T * k * 8 + (T * d * 2 if sH else 0),
                        write=T * d * 2, flops=0),
        "shared": dict(read=3 * sH * d * 2 + T * d * 2 + T * sH * 2,
                       write=T * sH * 2 + T * d * 2, flops=6 * T * d * sH),
    }
    for v in rec.values():
        v["bytes"] = v["read"] + v["write"]
    return rec


def _code_only(text):
    """Source text without comments and blank space: what the compiler sees."""
    import re

    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_digest():
    """Digest of the grouped GEMM's sources, comments left out, so that the
    stored counter bytes stay valid across comment edits."""
    h = hashlib.sha256()
    for name in ("ffn.hip", "moe_internal.hpp", "ring.hpp"):
        with open(os.path.join(ROOT, "expert_token_routing_moe_amd", "csrc", name)) as f:
            h.update(_code_only(f.read()).encode())
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
    return dict(value=done / spent, unit="tokens/s", cores=oracle.num_threads(),
                cpu_model=cpu_model(), kind="oracle",
                sample=f"first {done} of {cfg.T} tokens of the {cfg.name} workload, in batches "
                       f"of {batch}: route, dispatch, SwiGLU experts and combine in fp64 "
                       f"({spent:.1f} s of oracle compute)")


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def vendor_gemm_reference(cfg, dev, steps):
    """The vendor GEMM library (torch.nn.functional.linear -> hipBLASLt) on one
    expert's two GEMMs, for scale: TFLOP/s and fraction of the bf16
    matrix-core peak.  Rows per expert as in the grouped GEMM it is set
    beside: the expert-parallel rank-local share (D*T*k/E) where bench.py
    times one, else the layer's T*k/E."""
    import torch

    rank_local = cfg.D > 1 and cfg.cf == float("inf")
    rows = max(1, (cfg.D if rank_local else 1) * cfg.T * cfg.k // cfg.E)
    out = {"rows_per_expert": rows}
    for name, (n, kdim) in {"gate_up": (2 * cfg.H, cfg.d), "down": (cfg.d, cfg.H)}.items():
        a = torch.randn(rows, kdim, device=dev).to(torch.bfloat16)
        w = torch.randn(n, kdim, device=dev).to(torch.bfloat16)
        for _ in range(3):
            torch.nn.functional.linear(a, w)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            torch.nn.functional.linear(a, w)
        e1.record()
        e1.synchronize()
        t = e0.elapsed_time(e1) / steps / 1e3
        tf = 2 * rows * n * kdim / t / 1e12
        out[name] = dict(us=round(t * 1e6, 1), tflops=round(tf, 1),
                         mfma_util=round(tf / MFMA_BF16_PEAK_TFLOPS, 4))
    return out


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


def _best_ms(fn, stream, reps=5):
    import torch

    fn()  # warm-up
    best = float("inf")
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1))
    return best


def gather_probe_ms(buf, stream, scratch, reps=5):
    """The combine's access without its arithmetic (moe_stream_gather) on the
    layer's own expert outputs and slots: best of reps, each after the same
    last-level-cache flush as a timed step."""
    import torch

    from expert_token_routing_moe_amd import api

    out = torch.empty_like(buf.y)
    api.moe_stream_gather(buf.expert_out, buf.slot, out, stream)  # warm-up
    best = float("inf")
    for _ in range(reps):
        if scratch is not None:
            scratch.sum()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        api.moe_stream_gather(buf.expert_out, buf.slot, out, stream)
        e1.record(stream)
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del out
    return best


def device_rates(dev, stream):
    """Streaming rates of this device, GB/s: the best of five reads of a 2 GiB
    buffer through moe_stream_read (the expert GEMMs' non-temporal 16-byte
    loads) and the best of five fills of it through moe_stream_write (the
    permute's and the GEMM epilogues' non-temporal 16-byte stores), timed
    with events on the given stream."""
    import torch

    from expert_token_routing_moe_amd import api

    n = 1 << 31
    buf = torch.ones(n // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    rd = _best_ms(lambda: api.moe_stream_read(buf, sink, stream), stream)
    wr = _best_ms(lambda: api.moe_stream_write(buf, 1, stream), stream)
    del buf
    return n / (rd / 1e3) / 1e9, n / (wr / 1e3) / 1e9


# ---------------------------------------------------------------------------
# rocprofv3 summaries: the committed tables under profiles/ are made from the
# CSV output of the commands they list, by the function below.
# ---------------------------------------------------------------------------

def _kernel_label(name):
    name = name.replace("void ", "", 1).replace("(anonymous namespace)::", "")
    depth, out = 0, []
    for ch in name:  # drop the argument list, keep the template arguments
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out).strip()


def _gemm_stage(label):
    """'gate_up' or 'down' for a grouped GEMM kernel label (its DUAL argument:
    the eighth of the ring kernel's template arguments, the second of the
    ping-pong kernel's)."""
    args = label[label.index("<") + 1:label.rindex(">")].split(",")
    dual = args[1] if "grouped_gemm_pp_kernel" in label else args[7]
    return "gate_up" if dual.strip() == "true" else "down"


def _stage_of(label):
    if "route_" in label or "pad_wg" in label or "topk_softmax" in label:
        return "route"
    if "count" in label or "scan_kernel" in label or "permute" in label or "widen" in label:
        return "dispatch"
    if "grouped_gemm" in label:
        return _gemm_stage(label)
    if "combine" in label:
        return "combine"
    return None


def summarize_rocprof(out_dir, workload):
    """Markdown summary of the rocprofv3 runs of one workload (sub-folders
    trace/, fetch/, write/ and mfma/ of out_dir, with the bench JSON lines of
    the traced run in trace.json), and the grouped GEMMs' counter bytes per
    launch for profiles/hbm_traffic.json."""
    import csv
    import statistics as stt

    def rows(sub, name):
        import gzip

        path = os.path.join(out_dir, sub, name)
        if os.path.exists(path):
            return list(csv.DictReader(open(path)))
        if os.path.exists(path + ".gz"):  # the same, compressed
            with gzip.open(path + ".gz", "rt") as f:
                return list(csv.DictReader(f))
        return []

    with open(os.path.join(out_dir, "trace.json")) as f:
        bj = json.loads(f.read().strip().splitlines()[-1])
    # kernel trace: durations per (kernel, grid).  The layer's launches are
    # the groups first dispatched before the device-rate probes, which
    # bench.py runs after the timed steps (the rank-local share comes after)
    groups, first_start = {}, {}
    probe_start = None
    for r in rows("trace", "run_kernel_trace.csv"):
        lab = _kernel_label(r["Kernel_Name"])
        if not lab.startswith("moe::"):
            continue
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        t0 = int(r["Start_Timestamp"])
        if "stream_read" in lab:
            probe_start = t0 if probe_start is None else min(probe_start, t0)
        first_start[(lab, grid)] = min(first_start.get((lab, grid), t0), t0)
        groups.setdefault((lab, grid), []).append((int(r["End_Timestamp"]) - t0) / 1e3)

    def is_layer(key):
        return probe_start is None or first_start.get(key, probe_start) < probe_start

    def counters(sub):
        per = {}
        copies = []
        for r in rows(sub, "run_counter_collection.csv"):
            lab = _kernel_label(r["Kernel_Name"])
            if lab == "__amd_rocclr_copyBuffer":
                copies.append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
                continue
            if not lab.startswith("moe::"):
                continue
            key = (lab, int(r["Grid_Size"]))
            d = per.setdefault(key, {}).setdefault(r["Dispatch_Id"], {})
            d[r["Counter_Name"]] = float(r["Counter_Value"])
            if r.get("Start_Timestamp") and r.get("End_Timestamp"):  # ns, this dispatch
                d["_dur_s"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e9
        # the calibration copies are the run's last three copies
        return per, [v for _, v in sorted(copies)[-3:]]

    fetch, fcopy = counters("fetch")
    write, wcopy = counters("write")
    mfma, _ = counters("mfma")
    cal = bj.get("copy_calibration_bytes", 1 << 30)
    fscale = (cal / 1024) / stt.mean(fcopy) if fcopy else float("nan")
    wscale = (cal / 1024) / stt.mean(wcopy) if wcopy else float("nan")

    def mb(per, key, counter, scale):
        d = per.get(key)
        if not d:
            return float("nan")
        return stt.mean(v[counter] for v in d.values()) * scale * 1024 / 1e6

    cfg = bj["config"]
    dev = bj.get("device") or {"read_gbs": bj["roofline"].get("device_read_gbs"),
                               "write_gbs": bj["roofline"].get("device_write_gbs")}
    lines = [f"| kernel | grid (work-items) | calls | avg us | median us | min us | max us "
             f"| HBM read MB | HBM write MB |", "|---|---|---|---|---|---|---|---|---|"]
    traffic = {}
    stage_counter = {}
    for (lab, grid), ts in groups.items():
        rd = mb(fetch, (lab, grid), "FETCH_SIZE", fscale)
        wr = mb(write, (lab, grid), "WRITE_SIZE", wscale)
        lines.append(f"| `{lab}` | {grid} | {len(ts)} | {stt.mean(ts):.1f} | {stt.median(ts):.1f} "
                     f"| {min(ts):.1f} | {max(ts):.1f} | {rd:.1f} | {wr:.1f} |")
        st = _stage_of(lab)
        layer = is_layer((lab, grid))
        if st and layer:
            acc = stage_counter.setdefault(st, [0.0, 0.0])
            acc[0] += stt.mean(ts)
            acc[1] += rd + wr
        if "grouped_gemm" in lab:
            key = _gemm_stage(lab) + ("" if layer else "_rank_local")
            traffic[key] = dict(kernel=lab, grid=grid, fetch_bytes=round(rd * 1e6),
                                write_bytes=round(wr * 1e6), bytes_per_launch=round((rd + wr) * 1e6),
                                avg_us=round(stt.mean(ts), 2), source_digest=kernel_source_digest())
    stage_lines = ["| stage | event ms (bench) | kernels' avg us (sum) | algorithmic MB "
                   "| counter MB (read + write) | counter / algorithmic |", "|---|---|---|---|---|---|"]
    for st, v in bj["stages"].items():
        alg = v["gbs"] * v["ms"]  # GB/s x ms = MB
        ks, cm = stage_counter.get(st, [float("nan"), float("nan")])
        stage_lines.append(f"| {st} | {v['ms']:.4f} | {ks:.1f} | {alg:.1f} | {cm:.1f} "
                           f"| {cm / alg if alg else float('nan'):.3f} |")
    mf_lines = []
    if mfma:
        mf_lines = ["| kernel | grid | launches | SQ_INSTS_MFMA | algorithmic | ratio "
                    "| MFMA busy cycles | busy fraction | clock GHz | PFLOP/s | of peak at that clock |",
                    "|---|---|---|---|---|---|---|---|---|---|---|"]
        rl = bj.get("grouped_gemm_rank_local")
        for (lab, grid), d in mfma.items():
            if "grouped_gemm" not in lab:
                continue
            st = _gemm_stage(lab)
            layer = is_layer((lab, grid))
            per = 4 if st == "gate_up" else 2
            if layer:
                alg = bj["stages"][st]["tflops"] * bj["stages"][st]["ms"] * 1e9 / 16384
            elif rl:
                alg = per * rl["rows"] * cfg["d"] * cfg["H"] / 16384
            else:
                alg = float("nan")
            inst = stt.mean(v["SQ_INSTS_MFMA"] for v in d.values())
            busy = stt.mean(v["SQ_VALU_MFMA_BUSY_CYCLES"] for v in d.values())
            act = stt.mean(v["GRBM_GUI_ACTIVE"] for v in d.values())
            # the clock the chip held: GPU-active cycles of one XCD over the
            # dispatch's own time; the matrix-core peak at that clock is
            # 1024 SIMDs x 1024 flop per cycle (2.5 PFLOP/s at 2.4 GHz)
            durs = [v["_dur_s"] for v in d.values() if v.get("_dur_s")]
            dur = stt.mean(durs) if durs else float("nan")
            clk = act / 8 / dur if durs else float("nan")
            pf = alg * 16384 / dur / 1e15 if durs else float("nan")
            mf_lines.append(f"| `{lab}`{'' if layer else ' (rank-local share)'} | {grid} | {len(d)} "
                            f"| {inst:.4g} | {alg:.4g} | {inst / alg:.3f} | {busy:.4g} "
                            f"| {busy / (1024 * act / 8):.3f} | {clk / 1e9:.2f} | {pf:.3f} "
                            f"| {pf * 1e15 / (1024 * 1024 * clk):.3f} |")
    R = "$R"
    cmd = f"python3 {R}/bench.py --workload {workload}"
    md = [f"# rocprofv3 summary: MoE layer kernels, {workload} workload", "",
          "Commands (run from /tmp with TMPDIR=/tmp; $R is the repository root, OUT an output folder):", "",
          f"    rocprofv3 --kernel-trace --stats --output-format csv -d OUT/trace -o run -- {cmd} --no-cpu-baseline > OUT/trace.json",
          f"    rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/fetch -o run -- {cmd} --steps 3 --warmup 1 --no-cpu-baseline --copy-calibration",
          f"    rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/write -o run -- {cmd} --steps 3 --warmup 1 --no-cpu-baseline --copy-calibration",
          f"    rocprofv3 --pmc SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE --output-format csv -d OUT/mfma -o run -- {cmd} --steps 3 --warmup 1 --no-cpu-baseline",
          f"    python3 {R}/bench.py --summarize-rocprof OUT --workload {workload}", "",
          "Durations are from the kernel trace (every dispatch of the traced command, warmup",
          "included), grouped by kernel and grid size: the layer's launches come first; other grids",
          "of the same kernels are the rank-local expert-parallel share or the device-rate probes.",
          "",
          f"Counter scale: the counter runs copy a {cal >> 20} MiB device buffer three times "
          f"(`--copy-calibration`); FETCH_SIZE reads {stt.mean(fcopy) if fcopy else float('nan'):.0f} KiB "
          f"per copy (scale x{fscale:.4f}), WRITE_SIZE {stt.mean(wcopy) if wcopy else float('nan'):.0f} KiB "
          f"(scale x{wscale:.4f}); the MB below are scaled, per launch.", "",
          f"Traced bench line: {bj['ms_per_step']} ms/step, {bj['value']} tokens/s; device streaming "
          f"read {dev.get('read_gbs')} GB/s, store {dev.get('write_gbs')} GB/s.",
          "", *lines, "",
          "Per stage (the layer's launches only): HIP-event time of the stage in the traced bench",
          "run, the kernel-trace average of its kernels, its algorithmic bytes, and the counters.", "",
          *stage_lines, ""]
    if mf_lines:
        md += ["Grouped-GEMM matrix-core counters per launch. Algorithmic MFMA instructions = flops / 16384",
               "(one `v_mfma_f32_16x16x32_bf16` is 16x16x32 multiply-adds); busy fraction =",
               "SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs x GRBM_GUI_ACTIVE / 8 (GRBM_GUI_ACTIVE read as",
               "summed over the 8 XCDs); clock = GRBM_GUI_ACTIVE / 8 over the dispatch's own start-to-end",
               "time in the counter run (the clock the chip held under the kernel); PFLOP/s = algorithmic",
               "flops over that time; of peak at that clock = PFLOP/s over 1024 SIMDs x 1024 flop x clock.",
               "", *mf_lines, ""]
    return "\n".join(md), traffic


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the first passes over the 22.5 GB of DeepSeek-V3 expert weights run
    # slower (5.1 -> 4.3 ms over about eight steps): ten untimed steps reach
    # the steady state
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dsv3_prefill")
    ap.add_argument("--tokens", type=int, default=None, metavar="T",
                    help="tokens per layer call instead of the workload's (the same seeded "
                         "inputs, drawn for T tokens)")
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
    ap.add_argument("--no-flush-mall", dest="flush_mall", action="store_false",
                    help="do not read a 512 MiB buffer before every timed step (by default "
                         "the 256 MB last-level cache then holds nothing of the previous "
                         "step, and the step time is the sum of the stages' event times, "
                         "without the read)")
    ap.add_argument("--summarize-rocprof", metavar="OUT", default=None,
                    help="print the markdown summary of the rocprofv3 runs in OUT for --workload "
                         "(no GPU use) and record the grouped GEMMs' counter bytes in "
                         "profiles/hbm_traffic.json")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="also time the vendor GEMM library on one expert's GEMMs at the "
                         "rank-local shape, for scale")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU's share of the MoE layer; the library has no "
              "multi-GPU path (the expert-parallel exchange is not implemented); use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.summarize_rocprof:
        md, traffic = summarize_rocprof(args.summarize_rocprof, args.workload)
        print(md)
        path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
        rec = json.load(open(path)) if os.path.exists(path) else {}
        if traffic:
            rec[args.workload] = traffic
            with open(path, "w") as f:
                json.dump(rec, f, indent=1)
                f.write("\n")
        return

    import torch

    from expert_token_routing_moe_amd import api
    from expert_token_routing_moe_amd.inputs import CONFIGS, make_inputs

    cfg = CONFIGS[args.workload]
    if args.tokens is not None:
        cfg = cfg.with_(T=args.tokens)
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
    read_gbs, write_gbs = device_rates(dev, stream)
    log(f"bench: streaming read on this device {read_gbs:.0f} GB/s, store {write_gbs:.0f} GB/s")
    g_ms = gather_probe_ms(buf, stream, scratch)
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
                            # the stage's reads at the device's streaming-read rate plus
                            # its writes at the streaming-store rate, over its time
                            device_frac=round((traffic[s]["read"] / (read_gbs * 1e9)
                                               + traffic[s]["write"] / (write_gbs * 1e9)) / t, 4),
                            tflops=round(traffic[s]["flops"] / t / 1e12, 2))
    # the whole layer against its roofline: each stage at the larger of its
    # algorithmic bytes at the HBM peak and its flops at the bf16 matrix-core
    # peak, summed over the stages
    bound_ms = sum(max(traffic[s]["bytes"] / (HBM_PEAK_GBS * 1e9),
                       traffic[s]["flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12)) for s in stages) * 1e3
    layer_roof = {"bound_ms": round(bound_ms, 4), "frac": round(bound_ms / ms_step, 4)}
    # the combine against its own access pattern with no arithmetic
    per_stage["combine"]["gather_probe_ms"] = round(g_ms, 5)
    per_stage["combine"]["of_gather_probe"] = round(g_ms / stage_ms["combine"], 4)
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
        roof["device_write_gbs"] = round(write_gbs, 1)
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
        "device": {"read_gbs": round(read_gbs, 1), "write_gbs": round(write_gbs, 1)},
        "counts": counts,
        "roofline": roof,
        "layer_roofline": layer_roof,
    }
    if cfg.D > 1 and cfg.cf == float("inf") and not args.no_rank_local:
        log(f"bench: rank-local expert GEMMs ({cfg.E // cfg.D} experts, {cfg.D}x tokens routed)")
        out["grouped_gemm_rank_local"] = rank_local_gemm(cfg, inp, dev, args.steps, args.warmup)
    if args.vendor_gemm:
        log("bench: vendor GEMM reference at the rank-local expert shape")
        out["vendor_gemm_reference"] = vendor_gemm_reference(cfg, dev, args.steps)
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
