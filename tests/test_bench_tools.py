"""bench.py's host-side pieces, without a GPU: the one-GPU guard, the roofline
entry, the kernel label, the traffic figure's source check and the three
profile summarisers (kernel trace, HBM traffic counters, SQ/L1/L2 counters),
each fed small synthetic rocprofv3 CSV files whose expected summaries are
worked out by hand below."""
from __future__ import annotations

import csv
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
    assert r.stdout == ""


def test_roofline_entry():
    # 8 GB in 1 ms against 8 TB/s: HBM bound at exactly the peak
    r = bench.roofline(8_000_000_000, 1_000_000_000, 1.0, 2500.0)
    assert r["bound"] == "hbm" and r["achieved"] == 8000.0 and r["frac"] == 1.0
    assert r["intensity_flop_per_byte"] == 0.1 and r["mfma_frac"] == 0.0004
    # 1.25 PFLOP in 1 s against 2.5 PFLOP/s, 1 GB: MFMA bound at half the peak
    r = bench.roofline(1_000_000_000, 1_250_000_000_000_000, 1000.0, 2500.0)
    assert r["bound"] == "mfma" and r["achieved"] == 1250.0 and r["frac"] == 0.5 and r["unit"] == "TFLOP/s"
    # a forced bound keeps both fractions
    r = bench.roofline(8_000_000_000, 1_000_000_000, 2.0, 2500.0, prefer="mfma")
    assert r["bound"] == "mfma" and r["hbm_frac"] == 0.5


def test_gate_up_kernel_label_thresholds():
    g = 289
    assert "32-row" in bench.gate_up_kernel(24 * g, g, True)
    assert "64-row" in bench.gate_up_kernel(24 * g + 1, g, True)
    assert "64-row" in bench.gate_up_kernel(48 * g - 1, g, True)
    assert "256x256" in bench.gate_up_kernel(48 * g, g, True)
    assert "skipping" in bench.gate_up_kernel(159 * g, g, True)
    assert "skipping" not in bench.gate_up_kernel(160 * g, g, True)
    assert "skipping" not in bench.gate_up_kernel(100 * g, g, False)   # row-major weights never skip


def test_traffic_figure_only_for_the_profiled_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.md"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("prefill") is None                      # no summary
    f.write_text(f"traffic_bytes[prefill]: 7722115456\n\nsource_sha256: {bench.kernel_source_hash()}\n")
    assert bench.measured_traffic("prefill") == 7722115456
    assert bench.measured_traffic("decode") is None                       # workload not in the summary
    f.write_text("traffic_bytes[prefill]: 7722115456\n\nsource_sha256: " + "0" * 64 + "\n")
    assert bench.measured_traffic("prefill") is None                      # kernels changed since


def test_summarize_trace(tmp_path):
    d = tmp_path / "trace"
    rows = []
    for i, (name, dur) in enumerate([("void moe::(anonymous namespace)::combine_kernel<float>(int)", 4000),
                                     ("void moe::(anonymous namespace)::combine_kernel<float>(int)", 6000),
                                     ("void at::native::fill_kernel(int)", 9000)]):
        rows.append(dict(Kernel_Name=name, Start_Timestamp=1000 * i, End_Timestamp=1000 * i + dur,
                         Grid_Size_X=2048, Workgroup_Size_X=256, Grid_Size_Y=4, Workgroup_Size_Y=1))
    write_csv(str(d / "run_kernel_trace.csv"), rows)
    write_csv(str(d / "run_kernel_stats.csv"),
              [dict(Name="moe::(anonymous namespace)::combine_kernel<float>(int)", Calls=2, TotalDurationNs=10000,
                    AverageNs=5000)])
    out = tmp_path / "s.md"
    bench.summarize_trace(str(d), "title", "cmd", str(out))
    text = out.read_text()
    assert "| `moe::combine_kernel<float>` | 8 x 4 | 2 | 5.00 | 4.00 |" in text   # 2048/256 blocks, 4 slices
    assert "fill_kernel" not in text                                               # not the library's
    assert "| `moe::combine_kernel<float>` | 2 | 0.010 | 5.00 |" in text


KERNEL_NAMES = {
    "prefill": ("moe::gemm_bf16_big8<0, true, false, false>(GemmArgs)",
                "moe::gemm_bf16_big8<1, true, false, false>(GemmArgs)"),
    "decode": ("moe::gemm_bf16_mfma<0, 2, 1, 2, 4, true, true, false>(GemmArgs)",
               "moe::gemm_bf16_mfma<1, 2, 1, 2, 4, true, true, false>(GemmArgs)"),
}


@pytest.mark.parametrize("workload", ["prefill", "decode"])
def test_summarize_counters(tmp_path, workload):
    # one dispatch of each expert GEMM; 8 XCDs of 2.0M cycles each in 1 ms: 2 GHz
    gu, dn = KERNEL_NAMES[workload]
    router = "moe::gemm_bf16_mfma<1, 2, 1, 2, 4, true, false, false>(GemmArgs)"   # not an expert GEMM
    cyc = 2.0e6
    vals = {
        "GRBM_GUI_ACTIVE": 8 * cyc, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * cyc * 1024, "SQ_WAVE_CYCLES": 1000.0,
        "SQ_WAIT_ANY": 250.0, "SQ_WAIT_INST_ANY": 400.0, "SQ_LDS_IDX_ACTIVE": 1000.0, "SQ_LDS_BANK_CONFLICT": 5.0,
        "TCC_REQ_sum": 1.0e6, "TCC_HIT_sum": 4.0e5, "SQ_INSTS_MFMA": 2.0e6,
        # 256 compute units, each sending 0.125 reads per cycle with 500 cycles of latency: 62.5 in flight,
        # 16 bytes per cycle
        "TCP_TCC_READ_REQ_sum": 0.125 * 256 * cyc, "TCP_TCC_READ_REQ_LATENCY_sum": 500 * 0.125 * 256 * cyc,
        "TCP_PENDING_STALL_CYCLES_sum": 0.6 * 256 * cyc, "TD_TC_STALL_sum": 0.3 * 256 * cyc,
    }
    for name, counters in bench.COUNTER_PASSES.items():
        rows = []
        for kern in (gu, dn):
            for c in counters.split():
                rows.append(dict(Kernel_Name=kern, Counter_Name=c, Counter_Value=vals.get(c, 0.0)))
        for c in counters.split():   # the router's dispatch must not enter the averages
            rows.append(dict(Kernel_Name=router, Counter_Name=c, Counter_Value=7 * vals.get(c, 1.0)))
        write_csv(str(tmp_path / name / "run_counter_collection.csv"), rows)
    write_csv(str(tmp_path / "trace" / "run_kernel_trace.csv"),
              [dict(Kernel_Name=k, Start_Timestamp=0, End_Timestamp=1_000_000) for k in (gu, dn)])
    out = tmp_path / "c.md"
    bench.summarize_counters(str(tmp_path), str(out), workload)
    text = out.read_text()
    assert f"{workload} (T={32 if workload == 'decode' else 8192})" in text
    line = [l for l in text.splitlines() if l.startswith("- gate/up:")][0]
    for want in ("2.00M cycles per XCD", "1.000 ms", "about 2.00 GHz", "matrix cores busy 50.0%",
                 "waiting on a counter 25%", "to issue 40%", "bank conflicts 0.50%", "hit rate 40.0%",
                 "2.0M MFMA", "average latency 500 cycles", "about 62 reads in flight", "16.0 bytes per cycle",
                 "pending L2 data 60%", "on the cache 30%"):
        assert want in line, (want, line)
    assert "rocprofv3 --pmc TCP_TCC_READ_REQ_sum" in text   # the passes' commands are listed


def test_summarize_pmc(tmp_path):
    # per workload: the 1 GiB copy reads FETCH 524288 KiB (factor 2) and WRITE 1048576 KiB (factor 1);
    # the gate/up kernel fetches 1000 KiB and writes 100 KiB: 2*1000*1024 + 100*1024 bytes
    for w in bench.PMC_WORKLOADS:
        for c, copy_v, kern_v in (("FETCH_SIZE", 524288.0, 1000.0), ("WRITE_SIZE", 1048576.0, 100.0)):
            rows = [dict(Kernel_Name="__amd_rocclr_copyBuffer", Grid_Size=131072, Counter_Name=c, Counter_Value=copy_v),
                    dict(Kernel_Name="moe::gemm_bf16_big8<0, true, false, false>(GemmArgs)", Grid_Size=256,
                         Counter_Name=c, Counter_Value=kern_v)]
            write_csv(str(tmp_path / f"pmc_{w}_{c}" / "run_counter_collection.csv"), rows)
        with open(tmp_path / f"pmc_{w}_FETCH_SIZE" / "bench.log", "w") as f:
            f.write('{"roofline": {"algorithmic_bytes": 1024000}}\n')
    out = tmp_path / "t.md"
    bench.summarize_pmc(str(tmp_path), str(out))
    text = out.read_text()
    want = 2 * 1000 * 1024 + 100 * 1024
    for w in bench.PMC_WORKLOADS:
        assert f"traffic_bytes[{w}]: {want}" in text
        assert f"- {w}: {want / 1e9:.3f} GB measured vs 0.001 GB algorithmic ({want / 1024000:.3f}x)" in text
    assert f"source_sha256: {bench.kernel_source_hash()}" in text
