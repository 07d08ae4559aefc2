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


def test_traffic_hash_ignores_comments_only():
    a = 'int a = 1; // note\n/* block\n note */ const char* s = "x // kept /* kept */";\nchar q = \'"\';  int b;'
    b = 'int a = 1;\n const char* s = "x // kept /* kept */"; /* another note */\nchar q = \'"\'; // more\n int b;'
    assert bench.code_only(a) == bench.code_only(b)
    assert "// kept /* kept */" in bench.code_only(a)
    assert bench.code_only(a) != bench.code_only(a.replace("int b;", "int c;"))
    assert bench.code_only('s = "esc\\"aped // x"; t') == 's = "esc\\"aped // x"; t'


def test_every_workload_has_a_source_hash():
    hashes = {wl: bench.source_hash(wl) for wl in bench.WORKLOADS}
    assert all(len(h) == 16 for h in hashes.values())
    assert hashes["decode"] == hashes["stack1"] and hashes["decode"] != hashes["prefill512"]
