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


def test_traffic_digest_ignores_comments_not_code():
    src = 'int f(int x) {  // doubles x\n  return 2 * x; /* no overflow check */\n}\nconst char* s = "a // b";\n'
    same = 'int f(int x) {\n  return 2 * x;\n}\n// a note\nconst char* s = "a // b";\n'
    assert bench.code_only(src) == bench.code_only(same)
    assert bench.code_only(src) != bench.code_only(src.replace("2 * x", "3 * x")), "a code change is seen"
    assert bench.code_only(src) != bench.code_only(src.replace('"a // b"', '"a b"')), "string literals are code"
    assert '"a // b"' in bench.code_only(src)


def _write_csv(path, header, rows):
    import csv
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(header)
        wr.writerows(rows)


def test_record_mfma_derives_rates_from_counters(tmp_path, monkeypatch):
    """Counted flops are MOPS x 512; rates use the median kernel duration of the trace; other kernels
    (a differently named one sharing a prefix) are ignored; the record carries the sources' digest."""
    wl = synth.WORKLOADS["dsa_prefill_16k"]
    algo = bench.kernel_flops(wl, "sparse_mla_bf16_kernel")
    assert algo == 2 * 128 * (576 + 512) * sum(min(t + 1, 2048) for t in range(16384))
    name = "void dsa::(anonymous namespace)::sparse_mla_bf16_kernel<false>(unsigned short const*)"
    other = "void dsa::(anonymous namespace)::sparse_mla_bf16_kernel_extra(float)"
    mops = algo * 1.25 / 512
    raw = {"SQ_INSTS_VALU_MFMA_MOPS_BF16": mops, "SQ_VALU_MFMA_BUSY_CYCLES": 1e9, "SQ_BUSY_CYCLES": 5e8,
           "SQ_LDS_BANK_CONFLICT": 1e6, "SQ_LDS_IDX_ACTIVE": 3e6, "GRBM_GUI_ACTIVE": 8e7}
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    _write_csv(tmp_path / "m.csv", hdr, [[n, c, v * (3 if n == other else 1)] for n in (name, other) for c, v in raw.items()])
    _write_csv(tmp_path / "u.csv", hdr, [[name, "MfmaUtil", 51.5], [name, "LdsBankConflict", 0.2],
                                         [other, "MfmaUtil", 99.0], [other, "LdsBankConflict", 9.0]])
    # three dispatches of 8, 10 and 12 ms: the median is 10 ms
    _write_csv(tmp_path / "t.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
               [[name, 0, 8_000_000], [name, 0, 10_000_000], [name, 0, 12_000_000], [other, 0, 1]])
    profiles = tmp_path / "profiles"
    profiles.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    args = type("A", (), dict(workload="dsa_prefill_16k", kernel="sparse_mla_bf16_kernel", pmc_mfma=str(tmp_path / "m.csv"),
                              pmc_util=str(tmp_path / "u.csv"), ktrace=str(tmp_path / "t.csv"), commands="cmd"))()
    monkeypatch.setattr(bench, "kernel_sources_digest", lambda k: "d1")
    bench.record_mfma(args)
    import json
    rec = json.load(open(profiles / "sparse_mla_bf16_kernel_dsa_prefill_16k_mfma.json"))
    assert rec["kernel_us_median"] == 10000.0
    assert rec["counted_over_algorithmic"] == 1.25
    assert abs(rec["frac_algorithmic"] - algo / 1e-2 / 1e12 / bench.BF16_PEAK_TFLOPS) < 1e-4
    assert abs(rec["frac_counted"] - 1.25 * rec["frac_algorithmic"]) < 2e-4
    assert rec["mfma_util_pct"] == 51.5 and rec["lds_bank_conflict_pct"] == 0.2
    assert rec["lds_conflicts_per_access"] == 0.5
    assert bench.stored_mfma("dsa_prefill_16k", "sparse_mla_bf16_kernel")["frac_counted"] == rec["frac_counted"]
    monkeypatch.setattr(bench, "kernel_sources_digest", lambda k: "d2")
    assert bench.stored_mfma("dsa_prefill_16k", "sparse_mla_bf16_kernel") is None, "a changed source voids the record"
