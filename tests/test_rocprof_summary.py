"""CPU checks of decoder_block_amd/rocprof_summary.py on small hand-made CSVs:
kernel-name parsing, warm-up skipping, grouping by grid size, and the clock
and MFMA-busy arithmetic."""
import csv

from decoder_block_amd import rocprof_summary as R


def test_short_names():
    assert R.short_name("void llk::(anonymous namespace)::gemm_big_kernel<2, 256>(llk::GemmArgs)") == \
        "gemm_big_kernel<2, 256>"
    assert R.short_name("_ZN3llk12_GLOBAL__N_119rms_rowscale_kernelIDF16bEEvPKT_PfPS2_iifNS_6UploadE") == \
        "rms_rowscale_kernel<bf16>"
    assert R.short_name("_ZN3llk12_GLOBAL__N_126attn_decode_combine_kernelIDF16bLi128EEEvPKfPT_iiNS_9BatchViewE") == \
        "attn_decode_combine_kernel<bf16, 128>"


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_trace_skips_warmups_and_splits_grids(tmp_path, capsys):
    p = tmp_path / "kt.csv"
    hdr = ["Kernel_Name", "Dispatch_Id", "Grid_Size_X", "Start_Timestamp", "End_Timestamp"]
    rows = []
    # kernel A at two grid sizes: 2 warm-ups of 100 us, then 10 us and 20 us; small grid 5 us each
    for i, dur in enumerate([100_000, 100_000, 10_000, 20_000]):
        rows.append(["void k_a(int)", 2 * i, 1024, 0, dur])
        rows.append(["void k_a(int)", 2 * i + 1, 64, 0, 5_000])
    _write(p, hdr, rows)
    R.trace(str(p), skip=2, regex=None, merge=None)
    out = capsys.readouterr().out
    assert "| k_a grid=1024 | 2 | 15.0 | 15.0 |" in out
    assert "| k_a grid=64 | 2 | 5.0 | 5.0 |" in out
    R.trace(str(p), skip=2, regex=None, merge="k_a")
    out = capsys.readouterr().out
    assert "| k_a | 6 |" in out  # 8 dispatches of one name, the first 2 skipped


def test_pmc_clock_and_mfma_busy(tmp_path, capsys):
    p = tmp_path / "pmc.csv"
    hdr = ["Kernel_Name", "Dispatch_Id", "Grid_Size", "Counter_Name", "Counter_Value", "Start_Timestamp",
           "End_Timestamp"]
    # 1 ms dispatch; 8 XCDs x 2e6 busy cycles -> 2 GHz; half of 1024 SIMDs busy all the time -> 50%
    rows = []
    for d in (1, 2):
        rows.append(["void g(int)", d, 256, "GRBM_GUI_ACTIVE", 8 * 2e6, 0, 1_000_000])
        rows.append(["void g(int)", d, 256, "SQ_VALU_MFMA_BUSY_CYCLES", 512 * 2e6, 0, 1_000_000])
    _write(p, hdr, rows)
    R.pmc(str(p), skip=1, regex=None, merge=None)
    out = capsys.readouterr().out
    assert "n=1 mean 1000.0 us" in out and "clock 2.00 GHz" in out and "MFMA busy 50.0%" in out
