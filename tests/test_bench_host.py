"""CPU checks of bench.py's host logic: one GPU only, and the kernel-source hash that
guards the committed counter summaries."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_summaries_match_kernel_sources():
    # the committed counter summaries name the kernel sources they were taken on; bench.py
    # reports their traffic only while that hash matches the current sources
    sys.path.insert(0, ROOT)
    import bench
    h = bench.kernel_hash()
    found = 0
    for f in os.listdir(os.path.join(ROOT, "profiles")):
        if f.endswith("_pmc.txt"):
            found += 1
            text = open(os.path.join(ROOT, "profiles", f)).read()
            assert f"kernel_sources_sha256_16: {h}" in text, f
            if not f.startswith("conv_kernel_"):
                continue   # the backward's counter summaries: no bench.py field reads them
            wl = f[len("conv_kernel_"):-len("_pmc.txt")]
            dtype = "f32"
            if wl.endswith("_f64"):
                wl, dtype = wl[:-4], "f64"
            assert bench.read_traffic(wl, dtype) is not None, f
    assert found >= 1
