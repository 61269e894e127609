"""Host logic of the counter summaries (nvfp4_weight_only_moe_amd.pmc): the
copy calibration, the per-launch averages and the traffic entries bench.py
reads back."""
import json
import os

from nvfp4_weight_only_moe_amd import pmc

HEADER = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id","Grid_Size",'
          '"Kernel_Id","Kernel_Name","Workgroup_Size","LDS_Block_Size","Scratch_Size","VGPR_Count",'
          '"Accum_VGPR_Count","SGPR_Count","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"\n')


def _csv(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "x_counter_collection.csv"), "w") as fh:
        fh.write(HEADER)
        for did, name, val in rows:
            fh.write(f'{did},{did},"Agent 1",1,1,1,64,1,"{name}",64,0,0,8,0,16,"{counter}",{val},0,1\n')


def test_calibrated_traffic_entries(tmp_path):
    # the counter reads half the copy's bytes for FETCH and all of them for WRITE
    kib = 268435456 / 1024
    fetch = [(1, "__amd_rocclr_copyBuffer", 3.0),               # an earlier small copy: ignored
             (2, "k_dec_down<3, 1, false>", 1000.0), (3, "k_dec_down<3, 1, false>", 3000.0),
             (4, "k_other", 5.0),
             (5, "__amd_rocclr_copyBuffer", kib / 2), (6, "__amd_rocclr_copyBuffer", kib / 2),
             (7, "__amd_rocclr_copyBuffer", kib / 2)]
    write = [(2, "k_dec_down<3, 1, false>", 16.0), (3, "k_dec_down<3, 1, false>", 16.0),
             (5, "__amd_rocclr_copyBuffer", kib), (6, "__amd_rocclr_copyBuffer", kib),
             (7, "__amd_rocclr_copyBuffer", kib)]
    _csv(tmp_path / "f", "FETCH_SIZE", fetch)
    _csv(tmp_path / "w", "WRITE_SIZE", write)
    out = tmp_path / "traffic.json"
    out.write_text(json.dumps({"keep@me": {"hbm_bytes_per_launch": 1}}))
    assert pmc.main(["--fetch", str(tmp_path / "f"), "--write", str(tmp_path / "w"), "--workload", "wl",
                     "--kernel", "dec_down=k_dec_down<", "--update", str(out)]) == 0
    data = json.loads(out.read_text())
    assert data["keep@me"] == {"hbm_bytes_per_launch": 1}
    rec = data["dec_down@wl"]
    assert rec["fetch_bytes"] == 2000 * 1024 * 2          # mean 2000 KiB, scale 2
    assert rec["write_bytes"] == 16 * 1024
    assert rec["hbm_bytes_per_launch"] == rec["fetch_bytes"] + rec["write_bytes"]
    assert rec["copy_scale_fetch"] == 2.0 and rec["copy_scale_write"] == 1.0
    assert rec["source_sha256"] == pmc.kernel_source_hash("dec_down")


def test_missing_calibration_is_refused(tmp_path):
    _csv(tmp_path / "f", "FETCH_SIZE", [(1, "k_dec_down<3, 1, false>", 10.0)])
    _csv(tmp_path / "w", "WRITE_SIZE", [(1, "k_dec_down<3, 1, false>", 10.0)])
    try:
        pmc.main(["--fetch", str(tmp_path / "f"), "--write", str(tmp_path / "w"), "--workload", "wl",
                  "--kernel", "dec_down=k_dec_down<"])
    except SystemExit as e:
        assert "copy-calibration" in str(e)
    else:
        raise AssertionError("a run without calibration copies must be refused")
