"""Host-side logic of bench.py, without a GPU."""
import os
import subprocess
import sys

import bench
from synth.workloads import get_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_stream_plan_longest_first_least_loaded():
    wl = get_workload("llama3_8b_proj_m2048")
    work = [2.0 * wl.M * sum(p.N for p in wl.group(inp)) * K for inp, K in wl.inputs]
    plan = bench.plan_streams(work, 3)
    names = [wl.inputs[gi][0] for gi, _ in plan]
    assert names == ["mlp_in", "down_in", "attn_in", "o_in"]
    assert [si for _, si in plan] == [0, 1, 2, 2]          # QKV and O share the third stream
    # every group once; never more streams than groups
    assert sorted(gi for gi, _ in bench.plan_streams([5.0, 1.0], 3)) == [0, 1]
    assert max(si for _, si in bench.plan_streams([5.0, 1.0], 3)) == 1
    # equal work: input order, round robin
    assert bench.plan_streams([1.0] * 4, 2) == [(0, 0), (1, 1), (2, 0), (3, 1)]


def test_gemm_tile_rule_covers_the_workload():
    wl = get_workload("llama3_8b_proj_m2048")
    tiles = {inp: bench.gemm_tile(wl.M, sum(p.N for p in wl.group(inp)), K) for inp, K in wl.inputs}
    assert set(tiles.values()) <= {"256x256", "256x192", "128x128", "skinny", "generic"}
    # M = 2048: 256x192 tiles fill the chip for QKV (N = 6144: 256 tiles, 192 at
    # 256x256); gate+up keeps 256x256 (a near-tie, and less data per op); the
    # N = 4096 groups take 128x128
    assert tiles == {"attn_in": "256x192", "o_in": "128x128", "mlp_in": "256x256", "down_in": "128x128"}


def test_gemm_tile_rule_prefers_whole_rounds():
    assert bench.gemm_tile(2048, 24576, 4096) == "256x256"    # 768 tiles: 3 whole rounds
    assert bench.gemm_tile(4096, 6144, 4096) == "256x192"     # 512 tiles instead of 384
    assert bench.gemm_tile(2048, 4096, 14336) == "128x128"
    assert bench.gemm_tile(2048, 4096, 4100) == "generic"
    assert bench.gemm_tile(64, 5120, 20480) == "decode"          # decode, no LoRA epilogue
    assert bench.gemm_tile(64, 15360, 5120) == "decode"          # 240 blocks of 64 columns
    assert bench.gemm_tile(64, 20480, 5120) == "decode128"       # 320 of 64: 160 of 128
    assert bench.gemm_tile(65, 5120, 20480) == "128x128"
    assert bench.gemm_tile(64, 5120, 20480, lora=True) == "skinny"
    assert bench.gemm_tile(64, 15360, 5120, lora=True) == "128x128"   # wide: 120 column tiles


def test_cpu_baseline_on_the_tiny_workload():
    cb = bench.cpu_baseline(get_workload("tiny_m16_k256_n256"), 8, 64)
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert cb["nproc"] >= 1 and set(cb["stages_s"]) >= {"fold_quant", "quant", "gemm_dequant",
                                                         "lora_shrink", "lora_expand"}
    assert cb["full_step_tops"] < cb["value"]


def test_cpu_baseline_on_segmented_adapters():
    """The multi-tenant workload's oracle leg, on a tiny sample (rows and weight rows)."""
    cb = bench.cpu_baseline(get_workload("multitenant_lora_m8192"), 4, 32)
    assert cb["value"] > 0 and cb["stages_s"]["lora_expand"] > 0


def test_tile_dims_known_for_every_rule():
    for t in ("256x256", "256x192", "128x128", "generic", "skinny", "decode", "decode128"):
        assert len(bench.tile_dims(t)) == 2
