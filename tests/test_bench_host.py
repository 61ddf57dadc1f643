"""Host logic of bench.py (no GPU): the one-GPU contract, the step's byte
count, kernel-name mapping, and the rocprofv3 summaries that --write-profiles
writes and the bench reads back (on synthetic CSVs, into a temporary
profiles directory)."""

import csv
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
from causal_flash_attention_amd.workloads import HEADLINE  # noqa: E402

FWD = "_ZN5cattn12_GLOBAL__N_120attn_fwd_bf16_kernelEPKDF16bPDF16bPfiiiif"
DKDV = "_ZN5cattn12_GLOBAL__N_125attn_bwd_dkdv_bf16_kernelEPKDF16bS2_PKfPDF16biiiiiff"
DQP = "_ZN5cattn12_GLOBAL__N_123attn_bwd_dq_bf16_kernelILb1EEEvPKDF16bS3_S3_PKfPfPDF16biiiiiff"
DQ = "_ZN5cattn12_GLOBAL__N_123attn_bwd_dq_bf16_kernelILb0EEEvPKDF16bS3_S3_PKfPfPDF16biiiiiff"
COPY = "__amd_rocclr_copyBuffer"


def _write_csv(path, fields, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=fields)
        wr.writeheader()
        wr.writerows(rows)


def _counters(path, rows):
    _write_csv(path, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"],
               [{"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v}
                for d, k, c, v in rows])


def test_more_than_one_gpu_exits(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_defaults_are_one_gpu_and_short():
    a = bench.parse_args([])
    assert a.gpus == 1 and 0 < a.steps <= 1000 and 0 <= a.warmup <= 1000


def test_step_hbm_bytes_headline():
    # X = 16*12*1024*64 elements, R = 16*12*1024 rows: 32 X + 80 R bytes.
    X, R = 16 * 12 * 1024 * 64, 16 * 12 * 1024
    assert bench.step_hbm_bytes(HEADLINE) == 32 * X + 80 * R == 418381824


def test_kernel_names():
    assert bench._kernel_of(FWD) == "attn_fwd"
    assert bench._kernel_of(DKDV) == "attn_bwd_dkdv"
    assert bench._kernel_of(DQP) == "attn_bwd_dq_preprocess"
    assert bench._kernel_of(DQ) == "attn_bwd_dq"
    assert bench._kernel_of("void cattn::(anonymous namespace)::gemm_bf16_kernel<0, 1, 192, "
                            "false>(cattn::(anonymous namespace)::Operand)") == "gemm_rt192_bf16"
    assert bench._kernel_of("gemm_bf16_kernel<1, 1, 128, true>(x)") == "gemm_tt128_f32"
    assert bench._kernel_of(COPY) == "copy"
    assert bench._kernel_of("some_other_kernel") is None


@pytest.fixture
def profiles(tmp_path, monkeypatch):
    out = tmp_path / "profiles"
    out.mkdir()
    monkeypatch.setattr(bench, "PROFILE_DIR", str(out))
    return tmp_path


def test_write_and_read_back_profiles(profiles):
    t = profiles
    # Trace: three dKdV dispatches back to back (10, 12, 14 us), one forward alone (5 us).
    _write_csv(str(t / "trace" / "x_kernel_stats.csv"),
               ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
               [{"Name": DKDV, "Calls": 3, "AverageNs": 12000, "MinNs": 10000, "MaxNs": 14000,
                 "Percentage": 87.8},
                {"Name": FWD, "Calls": 1, "AverageNs": 5000, "MinNs": 5000, "MaxNs": 5000,
                 "Percentage": 12.2}])
    _write_csv(str(t / "trace" / "x_kernel_trace.csv"),
               ["Start_Timestamp", "End_Timestamp", "Kernel_Name"],
               [{"Start_Timestamp": 0, "End_Timestamp": 5000, "Kernel_Name": FWD},
                {"Start_Timestamp": 10000, "End_Timestamp": 20000, "Kernel_Name": DKDV},
                {"Start_Timestamp": 20000, "End_Timestamp": 32000, "Kernel_Name": DKDV},
                {"Start_Timestamp": 32000, "End_Timestamp": 46000, "Kernel_Name": DKDV}])
    # Counters: the 256 MiB copy reads FETCH = half its bytes and WRITE = all of them.
    copy_kib = bench.COPY_BYTES / 1024.0
    _counters(str(t / "fetch" / "f_counter_collection.csv"),
              [(1, DKDV, "FETCH_SIZE", 100.0), (2, DKDV, "FETCH_SIZE", 300.0),
               (3, COPY, "FETCH_SIZE", copy_kib / 2)])
    _counters(str(t / "write" / "w_counter_collection.csv"),
              [(1, DKDV, "WRITE_SIZE", 50.0), (2, DKDV, "WRITE_SIZE", 50.0),
               (3, COPY, "WRITE_SIZE", copy_kib)])
    _counters(str(t / "mfma" / "m_counter_collection.csv"),
              [(1, DKDV, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 300.0),
               (1, DKDV, "GRBM_GUI_ACTIVE", 8 * 1000.0),
               (1, DKDV, "SQ_LDS_IDX_ACTIVE", 400.0), (1, DKDV, "SQ_LDS_BANK_CONFLICT", 20.0)])
    wave = {"SQ_WAVE_CYCLES": 1000.0, "SQ_ACTIVE_INST_ANY": 340.0, "SQ_ACTIVE_INST_VALU": 200.0,
            "SQ_ACTIVE_INST_SCA": 80.0, "SQ_ACTIVE_INST_LDS": 40.0, "SQ_ACTIVE_INST_VMEM": 10.0,
            "SQ_ACTIVE_INST_MISC": 10.0, "SQ_WAIT_ANY": 240.0, "SQ_WAIT_INST_ANY": 420.0,
            "SQ_WAVES": 10.0, "SQ_INSTS_VALU": 20000.0, "SQ_INSTS_MFMA": 3000.0,
            "SQ_INSTS_SALU": 9000.0, "SQ_INSTS_LDS": 4000.0}
    names = sorted(wave)
    # Split over two passes, and each value over two rows of one dispatch (summed).
    _counters(str(t / "w1" / "a_counter_collection.csv"),
              [(7, DKDV, c, wave[c] / 2) for c in names[:7]] * 2)
    _counters(str(t / "w2" / "b_counter_collection.csv"),
              [(9, DKDV, c, wave[c] / 2) for c in names[7:]] * 2)

    args = bench.parse_args([
        "--write-profiles", "--trace-dir", str(t / "trace"), "--fetch-dir", str(t / "fetch"),
        "--write-dir", str(t / "write"), "--mfma-dir", str(t / "mfma"),
        "--wave-dirs", str(t / "w1"), str(t / "w2"), "--profile-command", "CMD",
        "--mfma-command", "MCMD", "--wave-command", "WCMD"])
    assert bench.write_profiles(args, HEADLINE) == 0
    p = t / "profiles"

    stats = (p / f"kernel_stats_{HEADLINE.name}.txt").read_text()
    assert "# command: CMD" in stats
    assert "attn_bwd_dkdv, 3, 12.00, 12.00, 10.00, 14.00, 87.80, 3, 12.00" in stats
    assert "attn_fwd, 1, 5.00, 5.00, 5.00, 5.00, 12.20, 0, -" in stats

    mfma = (p / f"mfma_util_{HEADLINE.name}.txt").read_text()
    assert "# command: MCMD" in mfma
    assert "attn_bwd_dkdv, 1, 300, 1000, 30.0, 5.0" in mfma

    waves = (p / f"wave_cycles_{HEADLINE.name}.txt").read_text()
    assert "# command: WCMD" in waves
    assert ("attn_bwd_dkdv, 1, 0.340, 0.200, 0.080, 0.040, 0.010, 0.010, 0.240, 0.420, "
            "2000, 300, 900, 400") in waves

    # Traffic: mean FETCH 200 KiB x 2 + mean WRITE 50 KiB x 1 per dispatch.
    want = 200.0 * 1024 * 2 + 50.0 * 1024
    assert bench.traffic_from_profile("attn_bwd_dkdv", HEADLINE.name) == pytest.approx(want)
    # A profile taken on other sources is not used.
    f = p / f"attn_bwd_dkdv_{HEADLINE.name}_hbm_traffic.txt"
    text = f.read_text()
    # the digest covers the kernel's source file and its generated program
    digest = bench.source_digest(os.path.join(bench.CSRC, "attn_bwd_bf16.hip"),
                                 [os.path.join(bench.CSRC, "attn_dkdv_asm.inc")])
    assert digest == bench.kernel_digest("attn_bwd_dkdv")
    assert digest != bench.source_digest(os.path.join(bench.CSRC, "attn_bwd_bf16.hip"))
    assert f"source_sha256_16: {digest}" in text
    f.write_text(text.replace(digest, "0" * 16))
    assert bench.traffic_from_profile("attn_bwd_dkdv", HEADLINE.name) is None
    assert bench.traffic_from_profile("attn_fwd", HEADLINE.name) is None  # no counters for it


def test_traffic_needs_the_copy_calibration(profiles):
    t = profiles
    _counters(str(t / "fetch" / "f_counter_collection.csv"), [(1, DKDV, "FETCH_SIZE", 1.0)])
    _counters(str(t / "write" / "w_counter_collection.csv"), [(1, DKDV, "WRITE_SIZE", 1.0)])
    args = bench.parse_args(["--write-profiles", "--fetch-dir", str(t / "fetch"),
                             "--write-dir", str(t / "write")])
    with pytest.raises(SystemExit, match="copy-calibration"):
        bench.write_profiles(args, HEADLINE)
