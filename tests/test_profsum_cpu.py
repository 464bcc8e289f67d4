"""The rocprofv3 CSV condenser behind profiles/ (host only): kernel-name
shortening, the comment-insensitive source hash, the decode split by launch
grid with its GB/s, and the counter calibration of the traffic summary, on
small synthetic CSVs with hand-computed answers."""

import csv
import json

import profsum

TRACE_COLS = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Grid_Size_Y"]


def _write(path, cols, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_short_names():
    n = "void moeq::(anonymous namespace)::decode_kernel<1, true, 4, true>(unsigned short const*, int)"
    assert profsum.short(n) == "decode_kernel<1, true, 4, true>"
    assert profsum.short("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def test_code_only_ignores_comments_and_layout():
    a = "int x = 1; // one\n/* block\n comment */ int y =  2;\n"
    b = "int x = 1;\nint y = 2; // two"
    assert profsum._code_only(a) == profsum._code_only(b)
    assert profsum._code_only(a) != profsum._code_only("int x = 1; int y = 3;")
    assert len(profsum.source_hash()) == 64


def test_decode_split_and_bandwidth(tmp_path, capsys):
    p = tmp_path / "trace.csv"
    g1 = "void moeq::(anonymous namespace)::decode_kernel<1, true, 4, true>(int)"
    g2 = "void moeq::(anonymous namespace)::decode_kernel<3, false, 4, false>(int)"
    rows = [
        {"Kind": "KERNEL_DISPATCH", "Kernel_Name": g1, "Start_Timestamp": 0, "End_Timestamp": 10_000,
         "Grid_Size_X": 2048, "Grid_Size_Y": 32},
        {"Kind": "KERNEL_DISPATCH", "Kernel_Name": g1, "Start_Timestamp": 50_000, "End_Timestamp": 62_000,
         "Grid_Size_X": 2048, "Grid_Size_Y": 32},
        {"Kind": "KERNEL_DISPATCH", "Kernel_Name": g2, "Start_Timestamp": 0, "End_Timestamp": 20_000,
         "Grid_Size_X": 16384, "Grid_Size_Y": 8},
        {"Kind": "KERNEL_DISPATCH", "Kernel_Name": "other_kernel", "Start_Timestamp": 0, "End_Timestamp": 5,
         "Grid_Size_X": 64, "Grid_Size_Y": 1},
    ]
    _write(p, TRACE_COLS, rows)
    profsum.decode(str(p), 2048, 1024, "1=0.5625,3=0.515869140625", "2048=8,16384=63", "cmd")
    out = capsys.readouterr().out
    lines = [l for l in out.splitlines() if l.startswith("| decode_kernel")]
    assert len(lines) == 2 and "other_kernel" not in out
    # gate_up launch: 8 experts x 2I x H x 0.5625 B = 18.874368 MB in 11 us on average
    g1_line = next(l for l in lines if "<1, true" in l)
    cells = [c.strip() for c in g1_line.strip("|").split("|")]
    assert cells[2] == "8" and cells[3] == "2" and cells[4] == "11.00"
    assert cells[7] == "18.9" and cells[8] == f"{8 * 2 * 1024 * 2048 * 0.5625 / 11e-6 / 1e9:.0f}"
    # down launch, double-quantized bytes: 63 experts x H x I x 0.515869 B in 20 us
    g2_line = next(l for l in lines if "<3, false" in l)
    cells = [c.strip() for c in g2_line.strip("|").split("|")]
    assert cells[8] == f"{63 * 2048 * 1024 * 0.515869140625 / 20e-6 / 1e9:.0f}"


def test_traffic_calibration(tmp_path, capsys):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    fdir, wdir = tmp_path / "f", tmp_path / "w"
    fdir.mkdir()
    wdir.mkdir()
    copy = 1 << 20  # a 1 MiB copy
    # FETCH_SIZE reads 0.5 counter bytes per copied byte, WRITE_SIZE 1.0; the
    # kernel's counters are split over two rows of one dispatch
    _write(fdir / "a_counter_collection.csv", cols, [
        {"Dispatch_Id": 1, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "FETCH_SIZE",
         "Counter_Value": copy * 0.5 / 1024},
        {"Dispatch_Id": 2, "Kernel_Name": "k<1>", "Counter_Name": "FETCH_SIZE", "Counter_Value": 100.0},
        {"Dispatch_Id": 2, "Kernel_Name": "k<1>", "Counter_Name": "FETCH_SIZE", "Counter_Value": 156.0},
    ])
    _write(wdir / "a_counter_collection.csv", cols, [
        {"Dispatch_Id": 1, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "WRITE_SIZE",
         "Counter_Value": copy / 1024},
        {"Dispatch_Id": 2, "Kernel_Name": "k<1>", "Counter_Name": "WRITE_SIZE", "Counter_Value": 64.0},
    ])
    profsum.traffic(str(fdir), str(wdir), "k<1>", copy, 1000.0, "f", "w")
    out = capsys.readouterr().out
    block = json.loads(out.split("```json\n")[1].split("\n```")[0])
    assert block["hbm_read_bytes"] == 256.0 * 1024 / 0.5
    assert block["hbm_write_bytes"] == 64.0 * 1024
    assert block["traffic_bytes"] == block["hbm_read_bytes"] + block["hbm_write_bytes"]
    assert block["source_sha256"] == profsum.source_hash()


def test_counters_mfma_busy_and_clock(tmp_path, capsys):
    # 2 XCDs, 8 SIMDs: GRBM_GUI_ACTIVE arrives summed over the XCDs (2 x 1000
    # busy cycles over a 500 ns dispatch: 2 GHz); the SIMDs were MFMA-busy for
    # 4000 of their 8 x 1000 cycles (50 %); 10 MFMA op units of 512 flops
    d = tmp_path / "c"
    d.mkdir()
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    rows = []
    for disp in (1, 2):
        for name, v in (("GRBM_GUI_ACTIVE", 2000.0), ("SQ_VALU_MFMA_BUSY_CYCLES", 4000.0),
                        ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 10.0)):
            rows.append({"Dispatch_Id": disp, "Kernel_Name": "void moeq::(anonymous namespace)::g<1>(int)",
                         "Counter_Name": name, "Counter_Value": v, "Start_Timestamp": 1000,
                         "End_Timestamp": 1500})
    _write(d / "7_counter_collection.csv", cols, rows)
    _write(d / "7_agent_info.csv", ["Name", "Num_Xcc", "Simd_Count"],
           [{"Name": "cpu", "Num_Xcc": 0, "Simd_Count": 0}, {"Name": "gfx950", "Num_Xcc": 2, "Simd_Count": 8}])
    profsum.counters(str(d), "g<1>@w", 0, 5120.0, "cmd")
    out = capsys.readouterr().out
    block = json.loads(out.split("```json\n")[1].split("\n```")[0])
    assert block["kernel"] == "g<1>@w" and block["dispatches"] == 2
    assert abs(block["mfma_util"] - 0.5) < 1e-12
    assert abs(block["shader_clock_GHz"] - 2.0) < 1e-12
    assert block["counter_flops"] == 5120.0 and block["algorithmic_flops"] == 5120.0


def test_kernels_table(tmp_path, capsys):
    # two library kernels and a foreign one; 1 XCD, 4 SIMDs
    d = tmp_path / "k"
    d.mkdir()
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    rows = []
    for disp, name, ctr in ((1, "moeq::(anonymous namespace)::a_kernel(int)",
                             {"GRBM_GUI_ACTIVE": 1000.0, "SQ_VALU_MFMA_BUSY_CYCLES": 1000.0,
                              "SQ_WAVE_CYCLES": 200.0, "SQ_WAIT_INST_ANY": 50.0, "SQ_WAIT_ANY": 20.0,
                              "SQ_ACTIVE_INST_VALU": 100.0, "SQ_ACTIVE_INST_LDS": 10.0}),
                            (2, "void moeq::(anonymous namespace)::b_kernel<2>(int)", {"SQ_WAVE_CYCLES": 100.0,
                                                                                    "SQ_WAIT_INST_ANY": 10.0,
                                                                                    "SQ_WAVES": 8.0,
                                                                                    "SQ_INSTS_VALU": 400.0,
                                                                                    "SQ_INSTS_VMEM_RD": 24.0}),
                            (3, "void at::native::fill(int)", {"SQ_WAVE_CYCLES": 5.0})):
        for n, v in ctr.items():
            rows.append({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": n, "Counter_Value": v,
                         "Start_Timestamp": 0, "End_Timestamp": 2000})
    _write(d / "1_counter_collection.csv", cols, rows)
    _write(d / "1_agent_info.csv", ["Name", "Num_Xcc", "Simd_Count"], [{"Name": "gfx950", "Num_Xcc": 1, "Simd_Count": 4}])
    got = profsum.kernels(str(d), "cmd")
    capsys.readouterr()
    assert set(got) == {"a_kernel", "b_kernel<2>"}
    a = got["a_kernel"]
    assert abs(a["mfma_busy"] - 0.25) < 1e-12 and abs(a["clock_GHz"] - 0.5) < 1e-12
    assert (a["wait_counter"], a["wait_any"], a["valu"], a["lds"]) == (0.25, 0.1, 0.5, 0.05)
    assert got["b_kernel<2>"]["wait_counter"] == 0.1 and "mfma_busy" not in got["b_kernel<2>"]
    b = got["b_kernel<2>"]
    assert (b["valu_per_wave"], b["vmem_rd_per_wave"]) == (50.0, 3.0) and "mfma_per_wave" not in b
    assert "valu_per_wave" not in a  # no SQ_WAVES in its run
    assert a["mean_us"] == 2.0
