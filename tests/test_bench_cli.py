"""bench.py entry point on the host: the command line parses, a multi-GPU
request is refused with a message, and the rocprof summary mode runs on an
empty directory."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_help():
    r = _run("--help")
    assert r.returncode == 0 and "--steps" in r.stdout


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_rocprof_summary_of_nothing(tmp_path):
    r = _run("--rocprof-summary", str(tmp_path))
    assert r.returncode == 0, r.stderr
    assert "traffic-json: {}" in r.stdout


def test_gemm_counter_summary_of_synthetic_csvs(tmp_path):
    """The GEMM counter summary matches dispatches to cases in launch order
    and derives its columns as documented: a case with 2MNK FLOPs in MOPS
    units, a 1 ms duration, GRBM = 8 x 2e6 cycles (2.0 GHz) and MFMA busy
    cycles of half of 1024 SIMDs x 2e6 reads 1.000, 2.00 GHz and 50.0%."""
    import csv

    sys.path.insert(0, ROOT)
    import bench

    cases = bench.gemm_profile_cases()
    reps = bench.GEMM_PROFILE_REPS
    name = "void fp8bq::(anonymous namespace)::gemm_dense_kernel<Wide, 256, 256>(args)"
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]

    def write_pass(sub, values):
        d = tmp_path / sub
        d.mkdir()
        with open(d / "p_counter_collection.csv", "w", newline="") as fh:
            w = csv.DictWriter(fh, fieldnames=cols)
            w.writeheader()
            w.writerow({"Dispatch_Id": 1, "Kernel_Name": "other_kernel", "Counter_Name": "X", "Counter_Value": 1})
            for i in range(len(cases) * reps):
                m, n, k, _ = cases[i // reps][1:]
                for cname, v in values(m, n, k).items():
                    w.writerow({"Dispatch_Id": 10 + i, "Kernel_Name": name, "Counter_Name": cname,
                                "Counter_Value": v})

    (tmp_path / "kt").mkdir()
    with open(tmp_path / "kt" / "kt_kernel_trace.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for i in range(len(cases) * reps):
            w.writerow({"Dispatch_Id": 10 + i, "Kernel_Name": name, "Start_Timestamp": 1000,
                        "End_Timestamp": 1000 + 1_000_000})
    write_pass("mfma", lambda m, n, k: {"SQ_INSTS_VALU_MFMA_MOPS_F8": 2.0 * m * n * k / 512,
                                        "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * 1024 * 2e6,
                                        "GRBM_GUI_ACTIVE": 8 * 2e6, "SQ_BUSY_CYCLES": 1})
    write_pass("lds", lambda m, n, k: {"SQ_LDS_BANK_CONFLICT": 1, "SQ_LDS_IDX_ACTIVE": 4})
    write_pass("l2", lambda m, n, k: {"TCC_HIT_sum": 3, "TCC_MISS_sum": 1})
    write_pass("wave", lambda m, n, k: {"SQ_WAVE_CYCLES": 100, "SQ_WAIT_ANY": 40, "SQ_WAIT_INST_ANY": 30,
                                        "SQ_WAIT_INST_LDS": 5, "SQ_ACTIVE_INST_ANY": 60, "SQ_ACTIVE_INST_VALU": 20,
                                        "SQ_ACTIVE_INST_LDS": 10, "SQ_ACTIVE_INST_VMEM": 2})
    write_pass("ta", lambda m, n, k: {"TA_BUSY_avr": 1e6, "GRBM_GUI_ACTIVE": 8 * 2e6})
    r = _run("--gemm-counter-summary", str(tmp_path))
    assert r.returncode == 0, r.stderr
    assert "kernel trace %d, mfma %d" % (len(cases) * reps, len(cases) * reps) in r.stdout
    rows = [line for line in r.stdout.splitlines() if line.startswith("| decode qkv (")]
    assert len(rows) == 1
    cells = [c.strip() for c in rows[0].strip("|").split("|")]
    # us, TFLOP/s, % peak, counter ratio, GHz, MFMA busy, LDS conflicts, L2 hit, bytes
    m, n, k = 256, 6144, 4096
    assert cells[2] == "1000.0"
    assert cells[3] == "%.0f" % (2.0 * m * n * k / 1e-3 / 1e12)
    assert cells[5:10] == ["1.000", "2.00", "50.0%", "0.250", "0.750"]
    assert cells[10] == "n/a"  # no fetch / write passes
    wave = [line for line in r.stdout.splitlines() if line.startswith("| decode qkv |")]
    assert len(wave) == 1
    assert [c.strip() for c in wave[0].strip("|").split("|")][1:] == [
        "0.400", "0.300", "0.050", "0.600", "0.200", "0.100", "0.020", "0.500"]


def test_bw_counter_summary_of_synthetic_csvs(tmp_path):
    """The bandwidth-kernel summary matches the library's dispatches to the
    cases in launch order (other kernels skipped), scales the counters by the
    copy calibration and divides by the algorithmic bytes: a case whose
    counters read exactly its algorithmic bytes after a x2 fetch scale, in
    1 ms, reads ratio 1.000 and (bytes / 1 ms) GB/s."""
    import csv

    sys.path.insert(0, ROOT)
    import bench

    cases = bench.bw_profile_cases()
    reps = bench.BW_PROFILE_REPS
    kib = 1 << 30

    def kname(prefix):
        return "void fp8bq::(anonymous namespace)::%s<4>(args)" % prefix

    def write_counter(sub, rows):
        d = tmp_path / sub
        d.mkdir()
        with open(d / "p_counter_collection.csv", "w", newline="") as fh:
            w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writeheader()
            for r in rows:
                w.writerow(r)

    def pass_rows(counter, part):
        rows = [{"Dispatch_Id": 1, "Kernel_Name": "kv_init_kernel", "Counter_Name": counter, "Counter_Value": 5}]
        for i in range(len(cases) * reps):
            label, prefix, algo = cases[i // reps]
            algo = 1_000_000 if algo is None else algo
            v = algo * part / 1024.0
            rows.append({"Dispatch_Id": 10 + i, "Kernel_Name": kname(prefix), "Counter_Name": counter,
                         "Counter_Value": v / 2.0 if counter == "FETCH_SIZE" else v})
        return rows

    write_counter("fetch", pass_rows("FETCH_SIZE", 0.75))
    write_counter("write", pass_rows("WRITE_SIZE", 0.25))
    write_counter("copy_fetch", [{"Dispatch_Id": 1, "Kernel_Name": "copyBuffer", "Counter_Name": "FETCH_SIZE",
                                  "Counter_Value": kib / 1024.0 / 2.0}])
    write_counter("copy_write", [{"Dispatch_Id": 1, "Kernel_Name": "copyBuffer", "Counter_Name": "WRITE_SIZE",
                                  "Counter_Value": kib / 1024.0}])
    (tmp_path / "kt").mkdir()
    with open(tmp_path / "kt" / "kt_kernel_trace.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for i in range(len(cases) * reps):
            w.writerow({"Dispatch_Id": 10 + i, "Kernel_Name": kname(cases[i // reps][1]), "Start_Timestamp": 0,
                        "End_Timestamp": 1_000_000})
    r = _run("--bw-counter-summary", str(tmp_path))
    assert r.returncode == 0, r.stderr
    n = len(cases) * reps
    assert "kernel trace %d, fetch %d, write %d (expected %d)" % (n, n, n, n) in r.stdout
    assert "FETCH_SIZE x2.000, WRITE_SIZE x1.000" in r.stdout
    label, _, algo = cases[0]
    row = [line for line in r.stdout.splitlines() if line.startswith("| %s |" % label)]
    assert len(row) == 1
    cells = [c.strip() for c in row[0].strip("|").split("|")]
    assert cells[2] == "1000.0" and cells[6] == "1.000"
    assert cells[7] == "%.0f" % (algo / 1e6)
