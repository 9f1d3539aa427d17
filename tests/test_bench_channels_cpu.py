"""The per-L2-channel counter definitions that bench.py writes for rocprofv3:
one derived counter per channel and base counter, each pass within the four
TCC counters one collection pass can hold, and the summary reading a run's
counter CSV back (a synthetic CSV, no GPU)."""
import csv

import bench


def test_channel_yaml_and_passes(tmp_path):
    text = bench.channel_counter_yaml()
    names = bench.channel_counter_names().splitlines()
    assert len(names) == len(bench.CHANNEL_PASSES)
    for line, p in zip(names, bench.CHANNEL_PASSES):
        assert len(p) <= 4  # TCC base counters per pass
        assert len(line.split()) == len(p) * bench.N_L2_CHANNELS
    for tag, base in bench.CHANNEL_COUNTERS:
        for k in range(bench.N_L2_CHANNELS):
            assert f"  - name: {tag}_CH{k}\n" in text
            assert f"reduce(select({base},[DIMENSION_INSTANCE=[{k}]]),sum)" in text


def test_channel_summary_reads_csv(tmp_path):
    d = tmp_path / "run"
    d.mkdir()
    cols = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
            "End_Timestamp"]
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for disp, grid in ((1, 1024), (2, 4096), (3, 4096)):
            for k in range(bench.N_L2_CHANNELS):
                for tag in ("RD", "WR"):
                    w.writerow({"Dispatch_Id": disp, "Grid_Size": grid, "Counter_Name": f"{tag}_CH{k}",
                                "Kernel_Name": "caat::pcr_reduce_f32_runs8_kernel(float const*)",
                                "Counter_Value": (2e6 if k == 3 else 1e6) if tag == "RD" else 1e6,
                                "Start_Timestamp": 0, "End_Timestamp": 700000})
    out = bench.rocprof_channels_summary([str(d)])
    assert "2 launches of 4096 threads" in out and "median 700 us" in out
    rd = next(l for l in out.splitlines() if l.startswith("| TCC_EA0_RDREQ |"))
    # 17 M in total, channel 3 at 2 / (17 / 16) of the mean
    assert rd.split("|")[2].strip() == "17.00" and rd.split("|")[3].strip() == f"{2 / (17 / 16):.3f}"
    wr = next(l for l in out.splitlines() if l.startswith("| TCC_EA0_WRREQ |"))
    assert wr.split("|")[3].strip() == "1.000"
