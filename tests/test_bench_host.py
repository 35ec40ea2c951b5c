"""Host logic of bench.py, without a GPU: the one-GPU refusal, the kernel classes of
rocprofv3 names, and the HBM-traffic summary (counter units scaled by a copy kernel of known
size, kept only while the GEMM source is unchanged)."""
import argparse
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_several_gpus_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("name,cls", [
    ("_ZN3dit12_GLOBAL__N_16k_gemmIDF16_Li1EEEvNS_8GemmArgsENS0_10TileBoundsEiii", "linear1"),
    ("_ZN3dit12_GLOBAL__N_16k_gemmIDF16_Li2EEEvNS_8GemmArgsENS0_10TileBoundsEiii", "linear2"),
    ("_ZN3dit12_GLOBAL__N_16k_gemmIDF16_Li0EEEvNS_8GemmArgsENS0_10TileBoundsEiii", "final/embed"),
    ("void dit::(anonymous namespace)::k_gemm8<1>(dit::GemmArgs, dit::TileBounds, int)", "linear1"),
    ("void dit::(anonymous namespace)::k_gemm8<2>(dit::GemmArgs, dit::TileBounds, int)", "linear2"),
    # tile height after the epilogue (16-bit and FP8 GEMMs), token blocks (fp32 MFMA GEMM)
    ("_ZN3dit12_GLOBAL__N_16k_gemmIDF16_Li1ELi256EEEvNS_8GemmArgsENS0_10TileBoundsEiii", "linear1"),
    ("_ZN3dit12_GLOBAL__N_16k_gemmIDF16bLi2ELi224EEEvNS_8GemmArgsENS0_10TileBoundsEiii", "linear2"),
    ("void dit::(anonymous namespace)::k_gemm8<1, 256>(dit::GemmArgs, dit::(anonymous", "linear1"),
    ("void dit::(anonymous namespace)::k_gemm8<2, 224>(dit::GemmArgs, dit::(anonymous", "linear2"),
    ("void dit::(anonymous namespace)::k_gemm_reduce<2, 224>(dit::GemmArgs, dit::(anon", "linear2"),
    ("_ZN3dit12_GLOBAL__N_113k_gemm_reduceILi0ELi256EEEvNS_8GemmArgsENS0_10TileBoundsEiii",
     "final/embed"),
    ("_ZN3dit12_GLOBAL__N_111k_gemm_f32mILi1ELi3EEEvNS_8GemmArgsENS0_10TileStartsEii", "linear1"),
    ("_ZN3dit12_GLOBAL__N_111k_gemm_f32mILi2ELi4EEEvNS_8GemmArgsENS0_10TileStartsEii", "linear2"),
    ("_ZN3dit12_GLOBAL__N_113k_gemm_simpleIDF16bLi0EEEvNS_8GemmArgsENS0_10TileStartsEii",
     "final/embed"),
    ("_ZN3dit12_GLOBAL__N_19k_attn_ppIDF16_EEvNS_8AttnArgsENS0_8AttnPlanE", "attention"),
    ("_ZN3dit6k_gemvIDF16_Lb1EEEvPfPKT_iiPKfii", "conditioning"),
    ("__amd_rocclr_fillBufferAligned", None),
])
def test_kernel_classes_of_rocprof_names(name, cls):
    assert bench._kernel_class(name) == cls


def _counter_csv(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, c, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_traffic_summary_scales_counters_by_the_copy_kernel(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    lin1 = "_ZN3dit12_GLOBAL__N_16k_gemmIDF16_Li1EEEvNS_8GemmArgsENS0_10TileBoundsEiii"
    lin2 = "_ZN3dit12_GLOBAL__N_16k_gemmIDF16_Li2EEEvNS_8GemmArgsENS0_10TileBoundsEiii"
    # copy kernel: 1 GiB read reads as 2^19 fetch units, 1 GiB written as 2^20 write units
    _counter_csv(tmp_path / "cf", [("vectorized_elementwise_kernel<MulFunctor>", "FETCH_SIZE", 2 ** 19)] * 3)
    _counter_csv(tmp_path / "cw", [("vectorized_elementwise_kernel<MulFunctor>", "WRITE_SIZE", 2 ** 20)] * 3)
    _counter_csv(tmp_path / "f", [(lin1, "FETCH_SIZE", 1000.0), (lin1, "FETCH_SIZE", 3000.0),
                                  (lin2, "FETCH_SIZE", 50.0)])
    _counter_csv(tmp_path / "w", [(lin1, "WRITE_SIZE", 100.0), (lin1, "WRITE_SIZE", 300.0),
                                  (lin2, "WRITE_SIZE", 5.0)])
    args = argparse.Namespace(workload="wl", compute="f16", trace_dir=None, mfma_dir=None,
                              fetch_dir=str(tmp_path / "f"), write_dir=str(tmp_path / "w"),
                              copy_fetch_dir=str(tmp_path / "cf"), copy_write_dir=str(tmp_path / "cw"),
                              pmc_cmd=["cmd"], traffic_kernel="linear1")
    bench.summarize_rocprof(args)
    d = bench.load_traffic("linear1", "wl", "f16")
    assert d is not None
    assert d["fetch_bytes_per_launch"] == pytest.approx(2000.0 * 2048)   # mean units x 2 KiB
    assert d["write_bytes_per_launch"] == pytest.approx(200.0 * 1024)    # mean units x 1 KiB
    assert d["bytes_per_launch"] == pytest.approx(2000.0 * 2048 + 200.0 * 1024)
    # a changed GEMM source voids the figure
    monkeypatch.setattr(bench, "source_sha256", lambda compute="f16": "0" * 16)
    assert bench.load_traffic("linear1", "wl", "f16") is None


def test_committed_traffic_summaries_parse():
    """Every committed counter summary carries a machine-readable figure with its source hash;
    bench.py uses it only while that hash matches the GEMM sources in the tree (else the
    bench line's traffic is null, as test_traffic_summary_scales_counters_by_the_copy_kernel checks)."""
    import glob
    import json
    import re
    paths = glob.glob(os.path.join(bench.PROFILES, "traffic_*.md"))
    assert paths
    for path in paths:
        m = re.search(r"^traffic_json: (\{.*\})$", open(path).read(), re.M)
        assert m, path
        d = json.loads(m.group(1))
        assert d["bytes_per_launch"] > 0 and len(d["source_sha256"]) == 16, path
