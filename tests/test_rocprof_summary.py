"""The profile summariser on synthetic rocprofv3 CSV files (CPU only)."""
import csv
import os

from scale_invariant_row_amd import rocprof_summary as R


def test_short_names():
    assert R.short_name("void dsr::l2_rows_kernel<4, 2, true, false>(HIP_vector_type<unsigned "
                        "int, 4u> const*, long, int, float)") == "l2_rows_kernel<4, 2, true, false>"
    assert R.short_name("dsr::rescale_mixed_128<false>(dsr::TaskArgs<dsr::RescaleTask>)") == \
        "rescale_mixed_128<false>"
    assert R.short_name("void at::native::(anonymous namespace)::distribution_elementwise_grid"
                        "_stride_kernel<float, 4>(int, float)").startswith("distribution_")


def test_algorithmic_bytes_of_the_bench_launches():
    t = R.bench_launches()
    assert R.lookup(t, "l2_rows_kernel<4, 2, true, false>", 2097152)[1:3] == (134217728, 67108864)
    assert sum(R.lookup(t, "slerp_rows_kernel<4, 2>", 2097152)[1:3]) == 201342976
    assert sum(R.lookup(t, "swiglu_table_l2_rows_kernel<8, 2>", 393216)[1:3]) == 352378880
    # the 48 linears forward: two launches (768- and 3,072-wide classes) whose
    # bytes add to the whole call's 510,271,488
    fwd = [v for k, v in t.items() if v[0] == "W rownorm, 48 linears"]
    assert len(fwd) == 2 and sum(v[1] + v[2] for v in fwd) == 510271488
    # ResNet-50's 54 weights run in two mixed launches
    res = [k for k, v in t.items() if v[0] == "W rownorm, ResNet-50"]
    assert sorted(k[0] for k in res) == ["rownorm_mixed_128", "rownorm_mixed_256"]


def _write(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_trace_and_traffic(tmp_path):
    kt = tmp_path / "kt" / "host" / "1" / "kt_kernel_trace.csv"
    rows = []
    for i, (name, grid, us) in enumerate([("void dsr::l2_rows_kernel<4, 2, true, false>(int)", 2097152, 32.0),
                                          ("void dsr::l2_rows_kernel<4, 2, true, false>(int)", 2097152, 34.0),
                                          ("__amd_rocclr_copyBuffer", 131072, 30.0)]):
        rows.append({"Kernel_Name": name, "Grid_Size_X": grid, "Grid_Size_Y": 1, "Grid_Size_Z": 1,
                     "Start_Timestamp": 1000 * i, "End_Timestamp": int(1000 * i + us * 1000)})
    _write(str(kt), rows)
    text = R.trace_report(str(tmp_path / "kt"))
    assert "l2_rows_kernel<4, 2, true, false>" in text and "33.00" in text
    # 201,326,592 B / 33 us = 6100.8 GB/s
    assert "6100.8 GB/s = 0.763" in text

    def counters(name, values):
        out = []
        for d, (kn, grid, v) in enumerate(values):
            out.append({"Dispatch_Id": d, "Kernel_Name": kn, "Grid_Size": grid,
                        "Counter_Name": name, "Counter_Value": v})
        return out
    copy_kib = R.COPY_BYTES / 1024
    _write(str(tmp_path / "f" / "a_counter_collection.csv"), counters("FETCH_SIZE", [
        ("__amd_rocclr_copyBuffer", 131072, copy_kib / 2),
        ("l2_rows_kernel<4, 2, true, false>(int)", 2097152, 134217728 / 1024 / 2)]))
    _write(str(tmp_path / "w" / "a_counter_collection.csv"), counters("WRITE_SIZE", [
        ("__amd_rocclr_copyBuffer", 131072, copy_kib),
        ("l2_rows_kernel<4, 2, true, false>(int)", 2097152, 67108864 / 1024)]))
    text = R.traffic_report(str(tmp_path / "f"), str(tmp_path / "w"))
    assert "FETCH_SIZE scale = 2.0000" in text and "WRITE_SIZE scale = 1.0000" in text
    assert "traffic l2_rows_kernel 201326592" in text
    assert "1.0000" in text.split("l2_rows_kernel<4, 2, true, false>")[1].splitlines()[0]
