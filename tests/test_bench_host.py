"""Host logic of bench.py, on the CPU: the algorithmic byte counts that the
roofline divides by, against the figures the workload definitions fix, and the
committed rocprofv3 counter summaries, which bench.py only reports while they
match the kernel sources they were taken on."""
import glob
import os
import subprocess
import sys
import types

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from hybrid_linear_attention_amd.workloads import FULL_DIMS, GqaDims  # noqa: E402


def test_decode_step_bytes():
    # state read and written once: 2 x 64 requests x 48 heads x 128 x 128 x 4 B
    assert 2 * 64 * 48 * 128 * 128 * 4 == 402_653_184
    # plus conv inputs, history read and written, z, gates and y (bf16)
    assert bench.fused_decode_bytes(FULL_DIMS, 64) == 413_413_376
    assert bench.fused_decode_bytes(FULL_DIMS, 64, state_bytes=2) == 212_086_784


def test_prefill_bytes_per_token():
    # x 20,480 + z 12,288 + a, b 192 + y 12,288 bytes per token
    base = bench.fused_prefill_bytes(FULL_DIMS, 0, 0, 0)
    assert bench.fused_prefill_bytes(FULL_DIMS, 1, 0, 0) - base == 45_248
    # one request's state written (and read with an initial state), history r+w
    state = 48 * 128 * 128 * 4
    hist = 2 * 10240 * 3 * 2
    assert bench.fused_prefill_bytes(FULL_DIMS, 0, 1, 1) == 2 * state + hist


def test_spec_verify_bytes():
    state, total = bench.spec_bytes(FULL_DIMS, 64, 4)
    assert state == 64 * 5 * 48 * 128 * 128 * 4
    assert total == 1_037_877_248


def test_gqa_decode_bytes():
    # 64 requests over 129,633 cached positions, 24 query / 4 key-value heads x 256
    c = types.SimpleNamespace(
        dims=GqaDims(24, 4, 256, 64), num_reqs=64,
        context_lens=torch.tensor([129_633 - 63 * 2000] + [2000] * 63),
        k_cache=torch.empty(0, dtype=torch.bfloat16))
    kv, total = bench.gqa_bytes(c)
    assert kv == 530_976_768
    assert total == 530_976_768 + 2_883_584
    c.k_cache = torch.empty(0, dtype=torch.float8_e4m3fn)
    kv, total = bench.gqa_bytes(c)
    assert (kv, total) == (265_488_384, 268_240_896)


def test_counter_summaries_match_the_sources():
    """Every committed counter summary was taken on the kernel source now in
    the tree (bench.py reports its traffic only then)."""
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.txt")))
    assert paths
    for path in paths:
        kernel = os.path.basename(path)[:-len("_traffic.txt")]
        source = None
        with open(path) as f:
            for line in f:
                if line.startswith("source:"):
                    source = line.split(":", 1)[1].strip()
        assert source, path
        assert bench.measured_traffic(kernel, source) is not None, path
    for name in ("prefill_4096", "prefill_varlen16"):
        cnt = bench.step_counters(name)
        assert cnt is not None, name
        assert cnt["kernels"] and cnt["hbm_bytes_per_step"] > 0
    gemm = bench.gemm_counters()
    assert gemm is not None and gemm["in_proj_hbm_bytes"] > 0 and gemm["out_proj_hbm_bytes"] > 0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stdout
