"""CPU: bench.py's contract that needs no GPU (argument checks, the byte
accounting behind the headline, the traffic bookkeeping, stacking groups)."""
import importlib.util
import os
import subprocess
import sys

import pytest

from weight_only_block_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr


def test_matrix_core_rows_out_of_range_are_refused():
    r = run_bench("--workload", "lm_head_mma", "--m", "17")
    assert r.returncode == 2 and "2..16" in r.stderr


def test_lm_head_algorithmic_bytes(bench):
    # int8 codes + one fp16 scale per 64 codes + bf16 x + fp32 y.
    _, _, N, K = synth.LM_HEAD
    assert synth.bytes_q8g64(N, K) == N * K + 2 * N * (K // 64) == 401_111_040
    assert synth.bytes_q8g64(N, K) + 2 * K + 4 * N == 401_723_904


def test_q4g32_and_moe_bytes_per_call():
    # Codes at half a byte, scale and min (fp16 each) per 32 codes.
    assert synth.bytes_q4g32(9216, 2560) == 9216 * 2560 // 2 + 4 * 9216 * (2560 // 32) == 14_745_600
    N, K = synth.MOE["gate"]
    assert synth.MOE["n_slots"] * synth.bytes_q4g32(N, K) == 31_457_280


def test_traffic_entries_name_known_workloads_and_sources(bench):
    for name, entry in bench.TRAFFIC.items():
        assert name in bench.KERNEL_SOURCES
        assert len(entry["source_digest"]) == 16 and entry["bytes_per_launch"] > 0
    for files in bench.KERNEL_SOURCES.values():
        for f in files:
            assert os.path.exists(os.path.join(ROOT, "weight_only_block_amd", "csrc", f)), f
    # The digest is a function of the listed sources only.
    assert bench.kernel_source_digest("lm_head") == bench.kernel_source_digest("lm_head")
    assert bench.kernel_source_digest("lm_head") != bench.kernel_source_digest("moe_experts")


def test_stacking_groups_follow_the_layer_order(bench):
    def stacked(name, mats):
        out = []
        for label, *_ in mats:
            g = bench._stack_group(name, label)
            if out and g is not None and bench._stack_group(name, out[-1].split("+")[0]) is g:
                out[-1] += "+" + label
            else:
                out.append(label)
        return out

    assert stacked("qwen3_0.6b", synth.QWEN3_06B_LAYER) == ["q+k+v", "o", "gate+up", "down"]
    assert stacked("q4_k2560", synth.Q4_K2560) == ["gate+up", "down"]
    assert stacked("w8a16_qwen3_14b_tp4", synth.W8A16_QWEN3_14B_TP4) == ["qkv", "o", "gate+up", "down"]
    # Members of a group read the same activation (same K).
    for name, mats in (("qwen3_0.6b", synth.QWEN3_06B_LAYER), ("q4_k2560", synth.Q4_K2560),
                       ("w8a16_qwen3_14b_tp4", synth.W8A16_QWEN3_14B_TP4)):
        for group in bench.STACK_GROUPS[name]:
            ks = {K for label, _, _, K in mats if label in group}
            assert len(ks) == 1, (name, group)
