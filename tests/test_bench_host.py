"""Host-side checks of bench.py's tables and argument handling (no GPU needed)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_every_workload_names_its_stage_kernels_and_sources():
    for wl in bench.WORKLOADS:
        assert bench.TRAFFIC_KERNELS[wl], wl
        for src in bench.TRAFFIC_SOURCES[wl]:
            assert os.path.exists(os.path.join(ROOT, "quantized_moe_expert_fp32_amd", "csrc", src)), (wl, src)


@pytest.mark.parametrize("wl,tokens", [("prefill512", 512), ("prefill4096", 4096), ("prefill512_8bit", 512),
                                       ("prefill512_fp8", 512), ("prefill4096_fp8", 4096)])
def test_count_launch_listed_only_above_the_self_count_limit(wl, tokens):
    # the scatter counts the picks itself up to 8192 of them (top-8, so 1024 tokens)
    listed = "prefill_count_kernel" in bench.TRAFFIC_KERNELS[wl]
    assert listed == (tokens * 8 > 8192)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0
    assert "--gpus 1" in r.stderr
