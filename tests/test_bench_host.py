"""Host-side parts of bench.py (no GPU): the refusal of more than one GPU,
the profile summaries written from rocprofv3's CSV output (kernel trace,
FETCH_SIZE / WRITE_SIZE counters, kernel statistics), the parsing of the
decode kernel's dispatch names and demangled symbols, and the digest that
ties a committed profile to the kernel's sources."""
import csv
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


GATE = "void bl::dot4::decode_dot4_kernel<(bl::Pattern)0, 8, 5, true, 8, 0>(float const*, signed char const*, " \
       "float const*, int const*, long, bl::FusedProjArgs, float*, bl::ActTransform)"
DOWN = "void bl::dot4::decode_dot4_kernel<(bl::Pattern)0, 16, 7, true, 4, 0>(float const*, signed char const*, " \
       "float const*, int const*, long, bl::FusedProjArgs, float*, bl::ActTransform)"
PROBE_KERNEL = "gate+up: fused_decode_dot4_dense_lpr8_u5_p2_w8, down: fused_decode_dot4_dense_lpr16_u7_p1"


def write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        for r in rows:
            w.writerow(r)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_dispatch_names_and_symbols(bench):
    assert bench._dot4_args("fused_decode_dot4_dense_lpr8_u5_p2_w8") == ("dense", 8, 5, True, 8, 0)
    assert bench._dot4_args("fused_decode_dot4_dense_lpr16_u7_p1") == ("dense", 16, 7, True, 4, 0)
    assert bench._dot4_args("decode_dot4_nm68_lpr32_u4_p1") == ("nm68", 32, 4, False, 4, 0)
    assert bench._dot4_args("fused_decode_dot4_dense_lpr8_u5_p2_gate_norm") == ("dense", 8, 5, True, 4, 3)
    assert bench._dot4_args(GATE) == ("dense", 8, 5, True, 8, 0)
    assert bench._dot4_args("void bl::dot4::decode_dot4_kernel<bl::Pattern::NM24, 16, 7, true, 4, 2>(x)") == \
        ("nm24", 16, 7, True, 4, 2)
    assert bench._dot4_args("bl::(anonymous namespace)::gemm_dma_kernel<256, 256, 2, 4, 6, false, 1>(int)") is None
    assert bench._symbol(GATE) == "void bl::dot4::decode_dot4_kernel<(bl::Pattern)0, 8, 5, true, 8, 0>"
    assert bench._symbol("bl::(anonymous namespace)::beta_kernel(double const*, long)") == \
        "bl::(anonymous namespace)::beta_kernel"
    assert bench._symbol("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def test_digest_ignores_the_checkout_location(bench, monkeypatch):
    from ternary_weight_linear_act_amd import build
    d1 = bench.source_digest()
    flags = [f if not os.path.isabs(f) else "/elsewhere/include" for f in build.CFLAGS]
    monkeypatch.setattr(build, "CFLAGS", flags)
    assert bench.source_digest() == d1
    monkeypatch.setattr(build, "CFLAGS", flags + ["-O0"])
    assert bench.source_digest() != d1


def test_trace_summary(bench, tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRACE_FILE", str(tmp_path / "trace.json"))
    tdir = tmp_path / "trace"
    hdr = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id", "Kernel_Name",
           "Correlation_Id", "Start_Timestamp", "End_Timestamp"]
    rows = []
    t = 1000
    for i in range(10):
        rows.append(["KERNEL_DISPATCH", "Agent 1", 1, 0, 1, 2 * i, 1, GATE, 2 * i, t, t + 4000 + 100 * i])
        t += 10000
        rows.append(["KERNEL_DISPATCH", "Agent 1", 1, 0, 1, 2 * i + 1, 2, DOWN, 2 * i + 1, t, t + 3000])
        t += 10000
    rows.append(["KERNEL_DISPATCH", "Agent 1", 1, 0, 1, 99, 3, "__amd_rocclr_copyBuffer", 99, t, t + 500])
    write_csv(str(tdir / "trace_kernel_trace.csv"), hdr, rows)
    write_csv(str(tdir / "trace_kernel_stats.csv"),
              ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"],
              [[GATE, 10, 44500, 4450.0, 50.0, 4000, 4900, 1.0], [DOWN, 10, 30000, 3000.0, 40.0, 3000, 3000, 0.0]])
    probe = tmp_path / "probe.out"
    probe.write_text("noise\n" + json.dumps({"trace_probe": True, "replays": 20, "steps_per_replay": 162,
                                             "us_per_step_events": 9.0, "kernel": PROBE_KERNEL,
                                             "source_digest": "abc"}) + "\n")
    bench.trace_summary(str(tdir), str(probe))
    out = json.load(open(tmp_path / "trace.json"))
    k = out["kernels"]
    assert out["source_digest"] == "abc"
    assert k["fused_decode_dot4_dense_lpr8_u5_p2_w8"]["dispatches"] == 10
    assert k["fused_decode_dot4_dense_lpr8_u5_p2_w8"]["avg_us"] == pytest.approx(4.45)
    assert k["fused_decode_dot4_dense_lpr8_u5_p2_w8"]["stats_avg_us"] == pytest.approx(4.45)
    assert k["fused_decode_dot4_dense_lpr16_u7_p1"]["avg_us"] == pytest.approx(3.0)
    assert k["fused_decode_dot4_dense_lpr16_u7_p1"]["group"] == "down"
    md = open(tmp_path / "trace.md").read()
    assert "--trace-summary" in md and "rocprofv3 --kernel-trace --stats" in md


def test_traffic_summary(bench, tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    hdr = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
           "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
           "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    copy_bytes = 1 << 28

    def rows(counter, gate_kib, down_kib, copy_kib):
        out = []
        for i, (name, v) in enumerate([(GATE, gate_kib), (DOWN, down_kib)] * 3 +
                                      [("__amd_rocclr_copyBuffer", 100.0), ("__amd_rocclr_copyBuffer", copy_kib)]):
            out.append([i, i, "Agent 1", 1, 1, 1, 64, 1, name, 256, 0, 0, 8, 0, 16, counter, v, 0, 1])
        return out
    # FETCH_SIZE reads half the bytes (scale 2), WRITE_SIZE reads them exactly
    write_csv(str(tmp_path / "f" / "p_counter_collection.csv"), hdr,
              rows("FETCH_SIZE", 8800.0, 4400.0, copy_bytes / 1024 / 2))
    write_csv(str(tmp_path / "w" / "p_counter_collection.csv"), hdr,
              rows("WRITE_SIZE", 54.0, 10.0, copy_bytes / 1024))
    probe = tmp_path / "probe.out"
    probe.write_text(json.dumps({"fused_launches": 6, "copy_bytes": copy_bytes, "kernel": PROBE_KERNEL,
                                 "source_digest": "abc"}) + "\n")
    bench.traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"), str(probe))
    out = json.load(open(tmp_path / "traffic.json"))
    assert out["fetch_scale"] == pytest.approx(2.0) and out["write_scale"] == pytest.approx(1.0)
    g = out["per_kernel"]["fused_decode_dot4_dense_lpr8_u5_p2_w8"]
    d = out["per_kernel"]["fused_decode_dot4_dense_lpr16_u7_p1"]
    assert g["dispatches"] == 3
    assert g["fetch_bytes"] == 8800 * 1024 * 2 and g["write_bytes"] == 54 * 1024
    assert d["hbm_bytes"] == 4400 * 1024 * 2 + 10 * 1024
    assert out["hbm_bytes_per_launch"] == round((g["hbm_bytes"] + d["hbm_bytes"]) / 2)


def test_stats_summary(bench, tmp_path):
    write_csv(str(tmp_path / "t" / "b_kernel_stats.csv"),
              ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"],
              [[GATE, 10, 44500, 4450.0, 50.0, 4000, 4900, 1.0],
               ["bl::(anonymous namespace)::gemm_dma_kernel<256, 256, 2, 4, 6, false, 1>(signed char const*)",
                5, 200000, 40000.0, 40.0, 39000, 41000, 1.0],
               ["at::native::vectorized_elementwise_kernel<4>(int)", 3, 10, 3.0, 0.1, 3, 3, 0.0]])
    out = tmp_path / "s.md"
    bench.stats_summary(str(tmp_path / "t"), str(out), "title", "cmd")
    md = out.read_text()
    assert "| `bl::(anonymous namespace)::gemm_dma_kernel<256, 256, 2, 4, 6, false, 1>` | 5 | 40.000 |" in md
    assert "vectorized_elementwise" not in md


def test_gemm_counters_summary(bench, tmp_path):
    hdr = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
           "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
           "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    gemm = "void bl::(anonymous namespace)::gemm_dma_kernel<256, 256, 2, 4, 6, false, 1, false>(signed char const*)"
    M, N, K = 2048, 6912, 2560
    mfmas = M * N * K // 32 ** 3
    rows = []
    for d in range(2):
        for c, v in [("SQ_VALU_MFMA_BUSY_CYCLES", 32.0 * mfmas), ("GRBM_GUI_ACTIVE", 8 * 2.5e3 * 40),
                     ("SQ_WAIT_ANY", 10.0), ("SQ_WAVE_CYCLES", 40.0), ("SQ_LDS_BANK_CONFLICT", 1.0),
                     ("SQ_INSTS_LDS", 4.0)]:
            rows.append([d, d, "Agent 1", 1, 1, 1, 64, 1, gemm, 512, 0, 0, 8, 0, 16, c, v, 0, 40000])
    rows.append([9, 9, "Agent 1", 1, 1, 1, 64, 1, "bl::beta_kernel(double const*)", 64, 0, 0, 8, 0, 16,
                 "SQ_WAVES", 1.0, 0, 5])
    write_csv(str(tmp_path / "p" / "p1_counter_collection.csv"), hdr, rows)
    probe = tmp_path / "probe.out"
    probe.write_text(json.dumps({"gemm_launches": 2, "kernel": "gemm_dense_dma_256x256_w8_s6", "M": M, "N": N,
                                 "K": K}) + "\n")
    out = tmp_path / "c.md"
    bench.gemm_counters_summary(str(tmp_path / "p"), str(probe), str(out), "cmd")
    md = out.read_text()
    assert "32.00 busy cycles per MFMA" in md
    assert "= 2.50 GHz" in md                       # 8 XCDs x 2.5e3 counts per us over 40 us
    assert "25.0% of wave time" in md and "0.25 cycles per LDS instruction" in md
    assert "| dur_us | 40.00 |" in md and "SQ_WAVES" not in md


def test_digest_ignores_comments(bench):
    a = "int f(int x) { // add one\n  return x + 1; /* done */ }\n"
    b = "int f(int x) {\n    return x + 1;\n}\n"
    c = "int f(int x) { return x + 2; }"
    assert bench._code_only(a) == bench._code_only(b) != bench._code_only(c)


def test_block_traffic_summary(bench, tmp_path):
    # two steps of three positions (a quant and two forwards, one of them the
    # same kernel as another position), after a pack dispatch of this library;
    # FETCH_SIZE counts half the bytes (scale 2), WRITE_SIZE all of them
    hdr = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
           "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
           "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    copy_bytes = 1 << 28
    Q = "void bl::(anonymous namespace)::quant_act_reg_kernel<256, 2>(float const*, long)"
    T = "void bl::skinny_direct_tiles::skinny_direct_tiles_kernel<1, 2, 2, false>(signed char const*, long)"
    seq = [("bl::(anonymous namespace)::pack_dense_kernel(float const*)", 1.0)] + \
        [(Q, 10.0), (T, 100.0), (T, 300.0)] * 2

    def rows(counter, copy_kib):
        out = []
        for i, (name, v) in enumerate(seq + [("__amd_rocclr_copyBuffer", copy_kib)]):
            out.append([i, i + 1, "Agent 1", 1, 1, 1, 64, 1, name, 256, 0, 0, 8, 0, 16, counter, v, 0, 1])
        return out[::-1]                                   # the summary orders by dispatch id
    write_csv(str(tmp_path / "f" / "p_counter_collection.csv"), hdr, rows("FETCH_SIZE", copy_bytes / 1024 / 2))
    write_csv(str(tmp_path / "w" / "p_counter_collection.csv"), hdr, rows("WRITE_SIZE", copy_bytes / 1024))
    probe = tmp_path / "probe.out"
    pos = [{"group": "a", "role": "quant_act", "bytes": 40960}, {"group": "a", "role": "forward", "bytes": 409600},
           {"group": "b", "role": "forward", "bytes": 1 << 20}]
    probe.write_text(json.dumps({"block_traffic_probe": 64, "steps": 2, "positions": pos, "copy_bytes": copy_bytes,
                                 "kernels": {}}) + "\n")
    out = tmp_path / "t.md"
    bench.block_traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"), str(probe), str(out), "c1 ;; c2")
    md = out.read_text()
    assert "scale 2.0000 and WRITE_SIZE scale 1.0000" in md
    assert "| a | quant_act | `void bl::(anonymous namespace)::quant_act_reg_kernel<256, 2>` | 20480 | 10240 | " \
           "40960 | 0.750 |" in md
    assert "| b | forward | `void bl::skinny_direct_tiles::skinny_direct_tiles_kernel<1, 2, 2, false>` | 614400 | " \
           "307200 | 1048576 | 0.879 |" in md
    assert "    c1\n    c2\n" in md


def test_block_traffic_summary_refuses_short_runs(bench, tmp_path):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    write_csv(str(tmp_path / "f" / "p_counter_collection.csv"), hdr,
              [[1, "void bl::x<1>(int)", "FETCH_SIZE", 1.0], [2, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 4.0]])
    write_csv(str(tmp_path / "w" / "p_counter_collection.csv"), hdr,
              [[1, "void bl::x<1>(int)", "WRITE_SIZE", 1.0], [2, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 4.0]])
    probe = tmp_path / "probe.out"
    probe.write_text(json.dumps({"block_traffic_probe": 8, "steps": 2, "positions": [{"group": "a", "role": "r",
                                                                                       "bytes": 1}],
                                 "copy_bytes": 4096, "kernels": {}}) + "\n")
    with pytest.raises(SystemExit):
        bench.block_traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"), str(probe), str(tmp_path / "o.md"), "c")
