"""Host-side logic of bench.py (no GPU): the compulsory work per workload, the
roofline arithmetic and the counter-pass summary."""
import csv

import numpy as np
import pytest

import bench
import workloads as W


def _upper_distinct_chunks(cfg):
    """Distinct (batch, kv head, chunk) triples can exceed neither the
    selections nor the chunks a row can see."""
    pos = cfg.q_pos0 + np.arange(cfg.q_len, dtype=np.int64)
    n = np.minimum(pos // 64, cfg.n_chunks)
    sel = int(np.minimum(n, cfg.top_k).sum()) * cfg.batch * cfg.n_kv_heads
    return min(sel, cfg.batch * cfg.n_kv_heads * int(n.max()))


# Hand-computed compulsory work (landmarks and queries read once, every
# selected chunk's K and V read once, out written once; FLOPs 2d per scored
# landmark plus 4*G*64*d per selection):
#   32K prefill: 64 MiB q_attn + 64 MiB out + 8 MiB q_ret + 8 MiB K/V of 511
#     chunks + 128 KiB landmarks = 152 MiB;  8.37 M candidates, 260 K selections -> 70.3 GFLOP
#   128K prefill: 2 GiB + 2 GiB + 256 MiB + 512 MiB + 4 MiB = 4.75 GiB;  1.07 G candidates,
#     16.7 M selections -> 4.65 TFLOP
#   16M decode: 64 MiB landmarks + 16 MiB K/V of 512 chunks + 68 KiB = 80.1 MiB;  1.21 GFLOP
#   1M chunked prefill: 1,032 MiB K/V + 128 MiB q_attn/out + 8 MiB q_ret + 16 MiB landmarks
#     = 2.16 GiB (K/V bound by the 16,511 visible chunks x 4 heads);  413 GFLOP
@pytest.mark.parametrize("i,mib,gflop", [(1, 152.0, 70.3), (2, 4.75 * 1024, 4650.0), (3, 80.1, 1.21),
                                          (4, 2.16 * 1024, 413.0)])
def test_compulsory_work_per_workload(i, mib, gflop):
    cfg = W.CONFIGS[i]
    alg = bench.algorithmic(cfg, _upper_distinct_chunks(cfg))
    assert alg["bytes"] / 2 ** 20 == pytest.approx(mib, rel=0.01)
    assert (alg["scan_flops"] + alg["attend_flops"]) / 1e9 == pytest.approx(gflop, rel=0.01)


def test_step_roofline_takes_the_larger_bound():
    r = bench.step_roofline(8e9, 2.5e12, 2.0)          # 1 ms of HBM, 1 ms of MFMA at peak, 2 ms measured
    assert r["t_hbm_ms"] == pytest.approx(1.0) and r["t_mfma_ms"] == pytest.approx(1.0)
    assert r["frac"] == pytest.approx(0.5)
    r = bench.step_roofline(16e9, 2.5e12, 4.0)
    assert r["bound"] == "hbm" and r["frac"] == pytest.approx(0.5)


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for d, (name, v) in enumerate(rows):
            w.writerow(dict(Dispatch_Id=d, Kernel_Name=name, Counter_Name=counter, Counter_Value=v))


def test_counter_summary_scales_by_the_calibration_copy(tmp_path):
    """FETCH_SIZE reading half of the copy's 1 GiB read gives scale 2; the
    kernel's per-dispatch mean is scaled the same way."""
    f, wcsv = tmp_path / "f.csv", tmp_path / "w.csv"
    copy_kib = bench.COPY_BYTES / 1024
    _counter_csv(f, "FETCH_SIZE", [("void at::native::neg_kernel", copy_kib / 2),
                                   ("void hsa::chunk_attend_kernel<128, 8>(hsa::ChunkArgs)", 1000.0),
                                   ("void hsa::chunk_attend_kernel<128, 8>(hsa::ChunkArgs)", 3000.0)])
    _counter_csv(wcsv, "WRITE_SIZE", [("void at::native::neg_kernel", copy_kib),
                                      ("void hsa::chunk_attend_kernel<128, 8>(hsa::ChunkArgs)", 500.0)])
    text = bench.pmc_summary(str(f), str(wcsv), "prefill_128K", "chunk_attend_kernel<128, 8>", "cmd")
    vals = dict(line.split(": ", 1) for line in text.splitlines() if ": " in line and not line.startswith("#"))
    assert float(vals["fetch_scale"]) == pytest.approx(2.0)
    assert float(vals["write_scale"]) == pytest.approx(1.0)
    assert float(vals["fetch_bytes_per_launch"]) == pytest.approx(2000.0 * 1024 * 2.0)
    assert float(vals["write_bytes_per_launch"]) == pytest.approx(500.0 * 1024)
    assert int(vals["fetch_dispatches"]) == 2


def test_mfma_summary_busy_fraction(tmp_path):
    """A kernel whose 1024 SIMDs are each MFMA-busy for a quarter of the
    dispatch's cycles (GRBM_GUI_ACTIVE arrives summed over the 8 XCDs) reads 25 %;
    the counted bf16 FLOPs are the MOPS counter times 512."""
    path = tmp_path / "m.csv"
    name = "void hsa::(anonymous namespace)::chunk_attend_kernel<128, 8>(hsa::ChunkArgs)"
    cycles = 2_000_000                            # per XCD
    with open(path, "w", newline="") as fh:
        wr = csv.writer(fh)
        wr.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                     "Start_Timestamp", "End_Timestamp"])
        for d in (1, 2):
            for cn, v in (("SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * cycles * bench.N_SIMDS),
                          ("GRBM_GUI_ACTIVE", cycles * bench.N_XCDS),
                          ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e9)):
                wr.writerow([d, name, cn, v, 0, 1_000_000])     # 1 ms
            wr.writerow([3, "void at::native::neg_kernel", "GRBM_GUI_ACTIVE", 5.0, 0, 10])
    text = bench.mfma_summary(str(path), "prefill_128K", "chunk_attend_kernel<128, 8>", "cmd")
    vals = dict(line.split(": ", 1) for line in text.splitlines() if ": " in line and not line.startswith("#"))
    assert int(vals["dispatches"]) == 2
    assert float(vals["mfma_busy_percent"]) == pytest.approx(25.0)
    assert float(vals["mfma_bf16_flop_per_dispatch"]) == pytest.approx(512e9)
    assert float(vals["mfma_bf16_tflops_counted"]) == pytest.approx(512e9 / 1e-3 / 1e12)


def test_counter_summary_refuses_a_run_mixing_workloads(tmp_path):
    """Two workloads that share a kernel (different grid sizes) in one counter
    run would be averaged together: the summary refuses such a CSV."""
    path = tmp_path / "f.csv"
    name = "void hsa::(anonymous namespace)::chunk_attend_kernel<128, 8>(hsa::ChunkArgs)"
    with open(path, "w", newline="") as fh:
        wr = csv.writer(fh)
        wr.writerow(["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value",
                     "Start_Timestamp", "End_Timestamp"])
        wr.writerow([1, 1310720, name, "FETCH_SIZE", 100.0, 0, 10])
        wr.writerow([2, 21102592, name, "FETCH_SIZE", 900.0, 0, 10])
    with pytest.raises(SystemExit, match="grid sizes"):
        bench.pmc_mean_kib(str(path), "FETCH_SIZE", "chunk_attend_kernel")
    with pytest.raises(SystemExit, match="grid sizes"):
        bench.pmc_dispatch_values(str(path), "FETCH_SIZE", "chunk_attend_kernel")


def _trace_csv(path, spans):
    """A rocprofv3 kernel-trace CSV with one row per (start_ns, end_ns, name, grid)."""
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Workgroup_Size_X",
                    "Grid_Size_Y"])
        for st, en, name, grid in spans:
            w.writerow([name, st, en, grid, 256, 1])


def test_trace_summary_groups_workloads_at_host_gaps(tmp_path):
    """Dispatches separated by more than the gap form one workload each; the
    groups before the named workloads are setup; kernels are keyed by name and
    workgroup count."""
    ms = 1_000_000
    spans = [(0, 1 * ms, "void hsa::(anonymous namespace)::fill_u32_kernel(unsigned int*)", 256),
             # workload A after a 1 s gap: two grid sizes of one kernel
             (1000 * ms, 1002 * ms, "void hsa::(anonymous namespace)::chunk_attend_kernel<128, 8>(hsa::ChunkArgs)", 2560),
             (1003 * ms, 1004 * ms, "void hsa::(anonymous namespace)::chunk_attend_kernel<128, 8>(hsa::ChunkArgs)", 5120),
             # workload B after another 1 s gap
             (2000 * ms, 2003 * ms, "void hsa::(anonymous namespace)::scan_wide_kernel<true, 128>(hsa::ScanArgs)", 65536),
             (2003 * ms, 2004 * ms, "void hsa::(anonymous namespace)::scan_wide_kernel<true, 128>(hsa::ScanArgs)", 65536)]
    p = tmp_path / "kt.csv"
    _trace_csv(p, spans)
    text = bench.trace_summary(str(p), ["A", "B"], "cmd")
    sections = text.split("\n## ")[1:]
    assert [s.splitlines()[0] for s in sections] == ["setup 0", "A", "B"]
    a_rows = [l.split() for l in sections[1].splitlines()[2:]]
    assert sorted((r[0] + r[1], int(r[2]), int(r[3])) for r in a_rows) == [
        ("chunk_attend_kernel<128,8>", 10, 1), ("chunk_attend_kernel<128,8>", 20, 1)]
    b_row = sections[2].splitlines()[2].split()
    assert b_row[2] == "256" and b_row[3] == "2" and float(b_row[4]) == pytest.approx(2000.0)
    # with a gap longer than both host gaps everything is one workload
    one = bench.trace_summary(str(p), ["all"], "cmd", gap_s=5.0)
    assert [s.splitlines()[0] for s in one.split("\n## ")[1:]] == ["all"]
