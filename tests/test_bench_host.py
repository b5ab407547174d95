"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the CPU
baseline's sampling, and the key under which stored HBM traffic is valid."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and not res.stdout.strip()


def test_cpu_baseline_cycles_until_its_budget():
    wl = synth.WORKLOADS["dsa_decode_b32_128k"].replace(B=2, N=2048, q_pos0=2047, K=128)
    x = synth.make_inputs(wl, 0)
    res = bench.cpu_baseline(wl, x, 0.3)
    done = int(res["sample"].split()[0])
    assert res["kind"] == "oracle" and res["unit"] == "queries/s" and res["value"] > 0
    assert done > 2, "two queries take far less than the budget: the sample must repeat them"
    assert "cycling" in res["sample"]


def test_traffic_digest_follows_sources_and_flags(monkeypatch):
    from long_context_sparse_14_amd import build
    base = bench.kernel_sources_digest("indexer_dma_bf16")
    assert base == bench.kernel_sources_digest("indexer_tiled_bf16")  # same source file, same flags
    assert base != bench.kernel_sources_digest("sparse_mla_bf16_kernel")
    monkeypatch.setitem(build.EXTRA_FLAGS, "indexer.hip", ["-O2"])
    assert bench.kernel_sources_digest("indexer_dma_bf16") != base, "a compile flag changes the kernel"
