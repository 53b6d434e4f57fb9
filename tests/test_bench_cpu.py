"""bench.py host logic without a GPU: the multi-GPU refusal and the source-checked HBM traffic figure."""
import hashlib
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def write_profile(tmp_path, src_rel, digest, workload="multihot-bf16-zipf"):
    rec = {"workload": workload, "kernels": {"seg_reduce_adagrad": {
        "dispatches": 3, "read_bytes": 1000, "write_bytes": 24, "sources": [src_rel], "source_sha256": digest}}}
    p = tmp_path / "hbm.md"
    p.write_text("# summary\n\n```\ntraffic-json: " + json.dumps(rec) + "\n```\n")
    return str(p)


def digest_of(rel, data):
    h = hashlib.sha256()
    h.update(rel.encode())
    h.update(b"\0")
    h.update(data)
    return h.hexdigest()


def test_traffic_used_only_for_unchanged_sources(tmp_path):
    src = tmp_path / "k.hip"
    src.write_bytes(b"kernel v1\n")
    prof = write_profile(tmp_path, "k.hip", digest_of("k.hip", b"kernel v1\n"))
    got = bench.measured_traffic("seg_reduce_adagrad", "multihot-bf16-zipf", prof, str(tmp_path))
    assert got == {"bytes": 1024, "read": 1000, "write": 24}
    # another workload, another kernel: no figure
    assert bench.measured_traffic("seg_reduce_adagrad", "multihot-bf16-uniform", prof, str(tmp_path)) is None
    assert bench.measured_traffic("pool_wave_per_bag", "multihot-bf16-zipf", prof, str(tmp_path)) is None
    # the kernel changed since the counters were taken: no figure
    src.write_bytes(b"kernel v2\n")
    assert bench.measured_traffic("seg_reduce_adagrad", "multihot-bf16-zipf", prof, str(tmp_path)) is None
    # no summary at all
    assert bench.measured_traffic("seg_reduce_adagrad", "multihot-bf16-zipf", str(tmp_path / "none.md"),
                                  str(tmp_path)) is None


def test_committed_profile_is_well_formed():
    line = next(l for l in open(bench.TRAFFIC_PROFILE) if l.startswith("traffic-json: "))
    rec = json.loads(line[len("traffic-json: "):])
    assert rec["workload"] == "multihot-bf16-zipf"
    for name, e in rec["kernels"].items():
        assert e["read_bytes"] >= 0 and e["write_bytes"] >= 0 and e["dispatches"] > 0
        for f in e["sources"]:
            assert os.path.exists(os.path.join(ROOT, f)), f


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_read_ceiling_fraction():
    gather = {"zipf": {"hbm_GBps": 3000.0}, "uniform": {"hbm_GBps": None}, "cold": {}}
    bench.add_read_ceiling(gather, {"random_row_gather": {"random_row_read_GBps": 6000.0}})
    assert gather["zipf"]["hbm_frac_of_random_row_read_ceiling"] == 0.5
    assert "hbm_frac_of_random_row_read_ceiling" not in gather["uniform"]
    assert "hbm_frac_of_random_row_read_ceiling" not in gather["cold"]
    # no probe measured: nothing added
    g2 = {"zipf": {"hbm_GBps": 3000.0}}
    bench.add_read_ceiling(g2, {})
    assert g2 == {"zipf": {"hbm_GBps": 3000.0}}


def test_inference_summary_bytes_and_rates():
    class WL:
        D, T, B, N, P, elem_size = 128, 26, 16384, 27, 351, 2
    nnz = 1000000
    out = bench.inference_summary({"fused": 0.25, "two_call": 0.30}, WL, nnz)
    alg = nnz * (128 * 2 + 8) + (26 * 16384 + 1) * 8 + 16384 * 128 * 4 + 16384 * (351 + 128) * 4
    assert out["fused_algorithmic_bytes"] == alg
    assert abs(out["fused_GBps"] - alg / 0.25e-3 / 1e9) < 1e-6
    assert abs(out["speedup"] - 1.2) < 1e-12
    assert abs(out["fused_samples_per_s"] - 16384 / 0.25e-3) < 1e-3
    assert out["fused_frac_hbm_peak"] == out["fused_GBps"] / bench.HBM_PEAK_GBPS
