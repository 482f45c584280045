"""bench.py's HBM-traffic bookkeeping on the host: counter CSVs in, bytes
per launch per workload out, looked up per workload (no GPU needed)."""
import csv
import io
import json
import os
import sys
from contextlib import redirect_stdout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FIELDS = ["Kernel_Name", "Counter_Name", "Counter_Value"]


def _csv(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(FIELDS, r)))


def test_write_traffic_scales_by_the_copy_calibration(tmp_path):
    gib_kib = (1 << 30) // 1024
    _csv(tmp_path / "copy_fetch.csv", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", gib_kib / 2)])
    _csv(tmp_path / "copy_write.csv", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", gib_kib)])
    # two dispatches of one kernel (averaged), one of another; prefill145 only
    _csv(tmp_path / "prefill145_fetch.csv", [
        ("void moe::k_expert_gateup_p<true, 4>(int)", "FETCH_SIZE", 1000.0),
        ("void moe::k_expert_gateup_p<true, 4>(int)", "FETCH_SIZE", 3000.0),
        ("void moe::k_combine<10>(int)", "FETCH_SIZE", 50.0),
        ("at::native::something", "FETCH_SIZE", 7.0)])
    _csv(tmp_path / "prefill145_write.csv", [
        ("void moe::k_expert_gateup_p<true, 4>(int)", "WRITE_SIZE", 100.0),
        ("void moe::k_expert_gateup_p<true, 4>(int)", "WRITE_SIZE", 300.0),
        ("void moe::k_combine<10>(int)", "WRITE_SIZE", 10.0)])
    buf = io.StringIO()
    with redirect_stdout(buf):
        bench.write_traffic(str(tmp_path))
    t = json.loads(buf.getvalue())
    assert t["source_digest"] == bench.source_digest()
    assert abs(t["calibration"]["fetch_counter_per_byte"] - 0.5) < 1e-12
    assert set(t["workloads"]) == {"prefill145"}          # no decode / 120B files given
    k = t["workloads"]["prefill145"]
    assert set(k) == {"k_expert_gateup_p<true, 4>", "k_combine<10>"}  # library kernels only
    g = k["k_expert_gateup_p<true, 4>"]
    assert g["dispatches"] == 2
    assert g["hbm_bytes_per_launch"] == round((2000.0 / 0.5 + 200.0) * 1024)


def test_stage_kernel_names_are_current():
    # every stage's kernel base name is a kernel the library defines
    src = ""
    csrc = os.path.join(ROOT, "latent_sparse_moe_amd", "csrc")
    for f in os.listdir(csrc):
        if f.endswith(".hip"):
            src += open(os.path.join(csrc, f)).read()
    for table in (bench.DECODE_STAGE_KERNELS, bench.GROUPED_STAGE_KERNELS):
        for names in table.values():
            assert any(f" {n}(" in src for n in names), names
