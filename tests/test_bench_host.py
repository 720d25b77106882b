"""Host-side checks of bench.py that need no GPU: the one-GPU guard and the rule that
counter-based traffic is reported only for the kernel source it was measured on."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_committed_traffic_follows_the_kernel_source():
    """profiles/traffic.json carries the sha256 of the kernel sources each record was
    measured on; the bench reports its bytes while they are unchanged and null after a
    change."""
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    for key, field in (("decode_gemv_nf4dq_m1", "traffic_bytes_per_launch"),
                       ("encoder_nvfp4_m1500", "traffic_bytes_per_step")):
        if key not in rec:
            assert bench.measured_traffic(key, field) is None
            continue
        v = bench.measured_traffic(key, field)
        if bench.source_digest(rec[key]["sources"]) == rec[key]["sources_sha256"]:
            # counters never read fewer bytes than the kernel must move
            assert v == rec[key][field] and v > rec[key]["algorithmic_bytes_per_" + field.split("_per_")[1]]
        else:
            assert v is None


def test_traffic_is_withheld_for_another_source(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    src = "block_quantized_bit_amd/csrc/gemv.hip"
    (prof / "traffic.json").write_text(json.dumps({"decode_gemv_nf4dq_m1": {
        "traffic_bytes_per_launch": 123, "algorithmic_bytes_per_launch": 100, "sources": [src],
        "sources_sha256": "0" * 64}}))
    csrc = tmp_path / "block_quantized_bit_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "gemv.hip").write_text("// some other kernel source\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("decode_gemv_nf4dq_m1") is None
    # the same record with the right digest is reported
    rec = json.loads((prof / "traffic.json").read_text())
    rec["decode_gemv_nf4dq_m1"]["sources_sha256"] = bench.source_digest([src])
    (prof / "traffic.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("decode_gemv_nf4dq_m1") == 123
