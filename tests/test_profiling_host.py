"""Host tests of the measurement tooling: the code digest that marks stored HBM-traffic counters as stale, and
the scaling of FETCH_SIZE / WRITE_SIZE readings by a copy kernel of known size."""
import csv

from vocabulary_label_bce_amd import profiling as P


def test_code_digest_ignores_comments_but_not_code():
    a = "int f(int x) {\n  // add one\n  return x + 1; /* the\n result */\n}\n"
    b = "int f(int x) {\n  // add one, rephrased\n\n  return x + 1;\n}\n"
    c = "int f(int x) {\n  return x + 2;\n}\n"
    assert P._code_only(a) == P._code_only(b)
    assert P._code_only(a) != P._code_only(c)
    assert "add one" not in P._code_only(a)


def _write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_traffic_scales_by_the_copy_kernel(tmp_path):
    copy_bytes = 1 << 30
    # the copy kernel's counters read half of its fetched bytes and all of its written bytes (in KiB)
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    _write_counters(fetch, [
        dict(Dispatch_Id=1, Kernel_Name="neg_kernel", Counter_Name="FETCH_SIZE", Counter_Value=copy_bytes / 2048),
        # a kernel reported as two records for one dispatch is summed
        dict(Dispatch_Id=2, Kernel_Name="k_rowsI<x>", Counter_Name="FETCH_SIZE", Counter_Value=1000.0),
        dict(Dispatch_Id=2, Kernel_Name="k_rowsI<x>", Counter_Name="FETCH_SIZE", Counter_Value=500.0),
        dict(Dispatch_Id=3, Kernel_Name="k_rowsI<x>", Counter_Name="FETCH_SIZE", Counter_Value=1500.0),
    ])
    _write_counters(write, [
        dict(Dispatch_Id=1, Kernel_Name="neg_kernel", Counter_Name="WRITE_SIZE", Counter_Value=copy_bytes / 1024),
        dict(Dispatch_Id=2, Kernel_Name="k_rowsI<x>", Counter_Name="WRITE_SIZE", Counter_Value=10.0),
        dict(Dispatch_Id=3, Kernel_Name="k_rowsI<x>", Counter_Name="WRITE_SIZE", Counter_Value=10.0),
    ])
    d = P.traffic(str(fetch), str(write), "k_rowsI", "neg_kernel", copy_bytes)
    assert abs(d["scale_fetch"] - 2.0) < 1e-12 and abs(d["scale_write"] - 1.0) < 1e-12
    assert d["fetch_kib_per_dispatch"] == [1500.0, 1500.0]
    assert abs(d["fetch_bytes_per_launch"] - 1500.0 * 1024 * 2.0) < 1e-6
    assert abs(d["bytes_per_launch"] - (1500.0 * 1024 * 2.0 + 10.0 * 1024)) < 1e-6


def test_counter_report_derives_clock_and_mfma_busy(tmp_path):
    # two passes over one kernel: pass 1 carries the MFMA counters, pass 2 GRBM_GUI_ACTIVE, each with its own
    # dispatch duration (1 ms and 2 ms); 1024 SIMDs, 8 XCDs, 2 GHz
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]

    def write(path, rows):
        with open(path, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=fields)
            w.writeheader()
            for r in rows:
                w.writerow(r)

    a, b = tmp_path / "p1.csv", tmp_path / "p2.csv"
    busy = 0.5 * 1024 * 2.0 * 1e6  # half of 1024 SIMDs x 2 GHz x 1 ms
    write(a, [dict(Dispatch_Id=1, Kernel_Name="k_itemsI<x>", Counter_Name="SQ_VALU_MFMA_BUSY_CYCLES",
                   Counter_Value=busy, Start_Timestamp=0, End_Timestamp=1_000_000),
              dict(Dispatch_Id=1, Kernel_Name="k_itemsI<x>", Counter_Name="SQ_INSTS_MFMA", Counter_Value=busy / 32,
                   Start_Timestamp=0, End_Timestamp=1_000_000),
              dict(Dispatch_Id=1, Kernel_Name="k_itemsI<x>", Counter_Name="SQ_INSTS_VALU",
                   Counter_Value=9 * busy / 32, Start_Timestamp=0, End_Timestamp=1_000_000),
              dict(Dispatch_Id=2, Kernel_Name="other", Counter_Name="SQ_INSTS_MFMA", Counter_Value=1.0,
                   Start_Timestamp=0, End_Timestamp=5)])
    write(b, [dict(Dispatch_Id=1, Kernel_Name="k_itemsI<x>", Counter_Name="GRBM_GUI_ACTIVE",
                   Counter_Value=8 * 2.0 * 2e6, Start_Timestamp=0, End_Timestamp=2_000_000)])
    means, durs = P.counter_means([str(a), str(b)], "k_itemsI")
    d = P.counter_report(means, durs)
    clock = [v for k, v in d.items() if k.startswith("shader clock")][0]
    frac = [v for k, v in d.items() if k.startswith("MFMA pipe busy")][0]
    assert abs(clock - 2.0) < 1e-12 and abs(frac - 0.5) < 1e-12
    assert d["MFMA busy cycles per MFMA instruction"] == 32.0
    assert abs(d["VALU instructions per MFMA (SQ_INSTS_VALU counts MFMA too; excluded)"] - 8.0) < 1e-12
