"""bench.py --summarize-rocprof on small synthetic rocprofv3 output (CPU only):
the layer's launches are the kernel groups dispatched before the device-rate
probes, counters are scaled by the calibration copies, and the per-stage
table sets counter bytes against the algorithmic bytes of the bench line."""
import csv
import gzip
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402

GEMM_GU = "void moe::(anonymous namespace)::grouped_gemm_kernel<256, 128, 64, 159744, 1, 2, 4, true, false>(moe::(anonymous namespace)::GemmArgs)"
ROUTE = "void moe::(anonymous namespace)::route_logits_kernel<64, 64, 256, 159744, 1, 2, 4>(moe::(anonymous namespace)::RouteArgs)"
ROUTE_TALL = "void moe::(anonymous namespace)::route_logits_kernel<128, 64, 256, 159744, 1, 2, 4>(moe::(anonymous namespace)::RouteArgs)"
PROBE = "void moe::(anonymous namespace)::stream_read_kernel(uint4 const*, unsigned long, unsigned int*)"
COPY = "__amd_rocclr_copyBuffer"

# (name, grid, start, end) in dispatch order: the layer (two steps), the
# read probe, then a kernel that only the rank-local setup launches
TRACE = [(ROUTE, 1024, 100, 130), (GEMM_GU, 4096, 140, 2140),
         (ROUTE, 1024, 3000, 3032), (GEMM_GU, 4096, 3040, 5040),
         (PROBE, 512, 6000, 6300), (ROUTE_TALL, 1024, 7000, 7200)]


def _write_trace(path):
    os.makedirs(path)
    fields = ["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Start_Timestamp",
              "End_Timestamp"]
    with open(os.path.join(path, "run_kernel_trace.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fields)
        w.writeheader()
        for name, grid, t0, t1 in TRACE:
            w.writerow(dict(Kernel_Name=name, Grid_Size_X=grid, Grid_Size_Y=1, Grid_Size_Z=1,
                            Start_Timestamp=t0 * 1000, End_Timestamp=t1 * 1000))


def _write_counters(path, rows, compress=False):
    """rows: (kernel, grid, counter, value) or (kernel, grid, counter, value,
    dispatch id, start ns, end ns)."""
    os.makedirs(path)
    fields = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value",
              "Start_Timestamp", "End_Timestamp"]
    name = os.path.join(path, "run_counter_collection.csv")
    with (gzip.open(name + ".gz", "wt", newline="") if compress else open(name, "w", newline="")) as f:
        w = csv.DictWriter(f, fields)
        w.writeheader()
        for i, row in enumerate(rows):
            kname, grid, counter, value = row[:4]
            disp, t0, t1 = row[4:] if len(row) > 4 else (i + 1, 0, 0)
            w.writerow(dict(Dispatch_Id=disp, Kernel_Name=kname, Grid_Size=grid,
                            Counter_Name=counter, Counter_Value=value,
                            Start_Timestamp=t0, End_Timestamp=t1))


def test_gemm_stage_of_both_kernels():
    assert bench._gemm_stage(GEMM_GU) == "gate_up"
    assert bench._gemm_stage(GEMM_GU.replace("true, false>", "false, false>")) == "down"
    pp = "void moe::(anonymous namespace)::grouped_gemm_pp_kernel<{}, {}>(moe::(anonymous namespace)::GemmArgs)"
    assert bench._gemm_stage(bench._kernel_label(pp.format(128, "true"))) == "gate_up"
    assert bench._gemm_stage(bench._kernel_label(pp.format(256, "false"))) == "down"
    assert bench._stage_of(bench._kernel_label(pp.format(256, "false"))) == "down"


def test_summary_tables(tmp_path):
    out = tmp_path / "run"
    os.makedirs(out)
    _write_trace(str(out / "trace"))
    copies = [(COPY, 65536, "FETCH_SIZE", 524288.0)] * 3          # half the 1 GiB copied
    _write_counters(str(out / "fetch"),
                    [(ROUTE, 1024, "FETCH_SIZE", 1000.0), (GEMM_GU, 4096, "FETCH_SIZE", 4000.0),
                     (ROUTE_TALL, 1024, "FETCH_SIZE", 9000.0)] + copies, compress=True)
    _write_counters(str(out / "write"),
                    [(ROUTE, 1024, "WRITE_SIZE", 100.0), (GEMM_GU, 4096, "WRITE_SIZE", 200.0)]
                    + [(COPY, 65536, "WRITE_SIZE", 1048576.0)] * 3)
    # matrix-core counters of one gate/up dispatch lasting 2 ms: 8 XCDs x
    # 3.6e6 active cycles -> 1.8 GHz; busy 1024 SIMDs x 1.8e6 cycles -> 0.5
    _write_counters(str(out / "mfma"),
                    [(GEMM_GU, 4096, c, v, 7, 10_000_000, 12_000_000)
                     for c, v in (("SQ_INSTS_MFMA", 1.25e8), ("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 1.8e6),
                                  ("SQ_BUSY_CYCLES", 1.0e7), ("GRBM_GUI_ACTIVE", 8 * 3.6e6))])
    line = {"ms_per_step": 2.0, "value": 2048000.0, "config": {"d": 64, "H": 64},
            "copy_calibration_bytes": 1 << 30,
            "device": {"read_gbs": 7000.0, "write_gbs": 5000.0},
            "roofline": {},
            "stages": {"route": {"ms": 0.03, "gbs": 100.0, "tflops": 0.0},
                       "gate_up": {"ms": 2.0, "gbs": 4.0, "tflops": 1000.0}}}
    (out / "trace.json").write_text("progress line\n" + json.dumps(line) + "\n")
    md, traffic = bench.summarize_rocprof(str(out), "tiny")
    # per-launch scaled megabytes: FETCH x2 (the copies read half), WRITE x1
    assert "| `moe::grouped_gemm_kernel<256, 128, 64, 159744, 1, 2, 4, true, false>` | 4096 | 2 " \
           "| 2000.0 | 2000.0 | 2000.0 | 2000.0 | 8.2 | 0.2 |" in md
    stage = {r.split("|")[1].strip(): r for r in md.splitlines() if r.startswith("| route ")
             or r.startswith("| gate_up ")}
    # route: only the layer's 64-token kernel (31 us mean), not the tall one
    # launched after the probe; algorithmic 100 GB/s x 0.03 ms = 3 MB
    cells = [c.strip() for c in stage["route"].split("|")]
    assert cells[3] == "31.0" and cells[4] == "3.0"
    assert abs(float(cells[5]) - (1000 * 2 + 100) * 1024 / 1e6) < 0.11
    assert traffic["gate_up"]["fetch_bytes"] == 4000 * 2 * 1024    # KiB x scale 2 -> bytes
    assert traffic["gate_up"]["write_bytes"] == 200 * 1024
    assert set(traffic) == {"gate_up"}                              # the router is no GEMM
    assert traffic["gate_up"]["source_digest"] == bench.kernel_source_digest()
    # matrix cores: algorithmic instructions = 1 PFLOP/s x 2 ms / 16384 =
    # 1.2207e8; 1 PFLOP/s over 1024 x 1024 flop x 1.8 GHz = 0.530
    mrow = [r for r in md.splitlines() if r.startswith("| `moe::grouped_gemm") and r.count("|") == 12]
    assert len(mrow) == 1, md
    cells = [c.strip() for c in mrow[0].split("|")][1:-1]
    assert cells[4] == "1.221e+08" and cells[5] == "1.024"
    assert cells[7] == "0.500" and cells[8] == "1.80" and cells[9] == "1.000"
    assert cells[10] == "0.530"


def test_source_digest_ignores_comments():
    code = "int f(int a) { return a + 1; }\n"
    commented = "// what f does\nint f(int a) /* one more */ { return a + 1; } // trailing\n"
    assert bench._code_only(code) == bench._code_only(commented)
    assert bench._code_only(code) != bench._code_only(code.replace("+ 1", "+ 2"))
