"""CPU checks of bench.py's host logic: the one-GPU refusal, and the counted-traffic record
(rocprofv3 FETCH_SIZE / WRITE_SIZE rows -> HBM bytes per launch through the 1 GiB device copy's
calibration, used only while the source hashes it was taken on still match)."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""  # no bench line


def _counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (kernel, counter, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_record(tmp_path, monkeypatch):
    import bench
    gemm = "void fp4::k_fp4_gemm_wide<2, false>(fp4::TileArgs)"
    esc = "void fp4::k_q16_escapes<1, 1, 1>(fp4::EscArgs)"  # follows the GEMM; not part of it
    comp = "void fp4::k_comp_apply<1, 1, 8>(fp4::CompArgs, int, int)"
    quant = ["fp4::k_zero_u32(unsigned int*, long, unsigned int*, long)",
             "void fp4::k_hist_rowmax<1>(void const*, long, long, unsigned int*, unsigned int*)",
             "void fp4::k_select_colmax<1>(unsigned int const*, fp4::State*, int, float*, unsigned long, fp4::WSide, int)",
             "void fp4::k_quant_rows<1, true, true, true, true>(void const*, long, long)",
             "void fp4::k_coo_qcols<1, true>(fp4::Staging, int const*)"]
    copy = "__amd_rocclr_copyBuffer"
    fetch = [(gemm, "FETCH_SIZE", 1000), (gemm, "FETCH_SIZE", 3000), (esc, "FETCH_SIZE", 99999),
             (comp, "FETCH_SIZE", 500), (comp, "FETCH_SIZE", 700)]
    fetch += [(q, "FETCH_SIZE", 10 * (i + 1)) for i, q in enumerate(quant)]
    write = [(gemm, "WRITE_SIZE", 700), (gemm, "WRITE_SIZE", 900), (esc, "WRITE_SIZE", 88888),
             (comp, "WRITE_SIZE", 400)]
    write += [(q, "WRITE_SIZE", 3) for q in quant]
    _counters(tmp_path / "gf", fetch)
    _counters(tmp_path / "gw", write)
    _counters(tmp_path / "cf", [(copy, "FETCH_SIZE", 524288), (copy, "FETCH_SIZE", 524288)])
    _counters(tmp_path / "cw", [(copy, "WRITE_SIZE", 1048576)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    bench.write_traffic(str(tmp_path / "gf"), str(tmp_path / "gw"), str(tmp_path / "cf"), str(tmp_path / "cw"))
    rec = json.load(open(out))
    # a 1 GiB copy reads 2^30 bytes over 524288 FETCH_SIZE units and writes them over 1048576 WRITE_SIZE units
    assert rec["bytes_per_fetch_unit"] == 2048 and rec["bytes_per_write_unit"] == 1024
    assert rec["gemm_kernel"] == "k_fp4_gemm_wide"
    # means over the GEMM's own dispatches (the escape kernel's rows are not the GEMM's)
    assert rec["hbm_bytes_per_launch"] == 2000 * 2048 + 800 * 1024
    assert rec["comp_hbm_bytes_per_launch"] == 600 * 2048 + 400 * 1024
    # the quantizer stage call: its five launches summed
    assert rec["quant_hbm_bytes_per_call"] == (10 + 20 + 30 + 40 + 50) * 2048 + 5 * 3 * 1024
    assert rec["gemm_src_sha"] == bench.gemm_src_sha() and rec["quant_src_sha"] == bench.quant_src_sha()
    assert bench.load_traffic(0.0, "gemm") == rec["hbm_bytes_per_launch"]
    assert bench.load_traffic(0.0, "comp") == rec["comp_hbm_bytes_per_launch"]
    assert bench.load_traffic(0.0, "quant") == rec["quant_hbm_bytes_per_call"]
    # a record taken on another source of a kernel is not reported for that kernel
    monkeypatch.setattr(bench, "gemm_src_sha", lambda: "0" * 16)
    assert bench.load_traffic(0.0, "gemm") is None
    assert bench.load_traffic(0.0, "comp") == rec["comp_hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.json"))
    assert bench.load_traffic(0.0, "quant") is None

