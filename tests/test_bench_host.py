"""Host logic of bench.py (CPU only): the one-GPU refusal, the algorithmic work
per launch that the roofline divides by, the lookup of committed HBM-traffic
records by kernel-source hash (and that profiles/ holds records for the
kernel sources as committed), and the kernel-name mapping.

The weight sizes are pinned to the parameter counts of the layers the pages
describe: E experts of three F x d matrices (gate, up, down), at the weight
type's bytes per value, with fp8's one f32 scale per weight row."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from mixture_experts_sparse_amd import workloads as W  # noqa: E402


def _weight_bytes(work, sh, kept):
    """Weight bytes of a step's expert GEMMs: each pass's bytes less its activation terms."""
    a = W.nbytes_of(sh.act_dtype)
    hb = 4 if sh.w_dtype == W.DT_F32 else 2
    gu = work["gemm_gate_up"]["bytes"] - kept * sh.d * a - kept * sh.F * hb
    dn = work["gemm_down"]["bytes"] - kept * sh.F * hb - kept * sh.d * 4
    return gu, dn


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_mixtral_expert_weights_are_2_82_GB():
    # 8 experts x 3 x 14336 x 4096 bf16 values = 2.82 GB resident
    sh = W.WORKLOADS["mixtral_bf16"]
    work = bench.algorithmic_work(sh, kept_rows=sh.T * sh.k, touched=sh.E)
    gu, dn = _weight_bytes(work, sh, sh.T * sh.k)
    assert gu + dn == 8 * 3 * 14336 * 4096 * 2
    assert abs((gu + dn) / 1e9 - 2.82) < 0.005
    assert gu == 2 * dn  # gate and up against down
    # 4 N d F for the gated pass, 2 N F d for the down pass (N = 8192 kept rows)
    assert work["gemm_gate_up"]["flop"] == pytest.approx(1.9241e12, rel=1e-4)
    assert work["gemm_down"]["flop"] == pytest.approx(work["gemm_gate_up"]["flop"] / 2)


def test_fine_grained_weights_are_22_6_GB_with_the_shared_expert():
    # 256 routed + 1 shared expert of 3 x 2048 x 7168 bf16 values
    sh = W.WORKLOADS["fine_shared_bf16"]
    kept = sh.T * sh.k
    work = bench.algorithmic_work(sh, kept_rows=kept, touched=sh.E)
    gu, dn = _weight_bytes(work, sh, kept)
    a = W.nbytes_of(sh.act_dtype)
    shared = (work["shared_gate_up"]["bytes"] - sh.T * sh.d * a - sh.T * sh.F * 2
              + work["shared_down"]["bytes"] - sh.T * sh.F * 2 - sh.T * sh.d * 4)
    total = gu + dn + shared
    assert sh.E == 256 and sh.n_shared == 1
    assert abs(total / 1e9 - 22.6) < 0.05


def test_fp8_weights_are_2_42_GB_plus_3_7_MB_of_scales():
    sh = W.WORKLOADS["skewed_fp8"]
    work = bench.algorithmic_work(sh, kept_rows=0, touched=sh.E)
    gu, dn = _weight_bytes(work, sh, 0)
    codes = 128 * 3 * 1536 * 4096  # one byte per e4m3 value
    scales = 128 * (2 * 1536 + 4096) * 4  # one f32 per weight row
    assert gu + dn == codes + scales
    assert abs(codes / 1e9 - 2.42) < 0.005 and abs(scales / 1e6 - 3.7) < 0.05


def test_combine_reads_kept_rows_once_and_writes_the_output_once():
    sh = W.WORKLOADS["mixtral_bf16"]
    N = 8000
    c = bench.algorithmic_work(sh, kept_rows=N, touched=sh.E)["combine"]["bytes"]
    out_b = 4 if sh.out_dtype == W.DT_F32 else 2
    assert c == N * sh.d * 4 + sh.T * sh.d * out_b + sh.T * sh.k * 8


def test_kernel_key_drops_dtype_tags():
    assert bench.kernel_key("gemm_gate_up_bf16") == "gemm_gate_up"
    assert bench.kernel_key("gemm_down_int4") == "gemm_down"
    assert bench.kernel_key("gemm_f32_down") == "gemm_down"
    assert bench.kernel_key("combine") == "combine"


def test_traffic_record_is_used_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    csrc = tmp_path / "mixture_experts_sparse_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("kernel source one\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h = bench.kernel_source_hash()

    def rec(kernel, workload, sha, b):
        return "traffic_record: " + json.dumps({"kernel": kernel, "workload": workload,
                                                "source_sha256": sha, "bytes_per_launch": b})

    (tmp_path / "profiles" / "x.md").write_text("\n".join([
        "# summary", rec("gemm_gate_up_bf16", "mixtral_bf16", "0" * 64, 1),
        rec("gemm_down_bf16", "mixtral_bf16", h, 2), rec("gemm_gate_up_bf16", "mixtral_bf16", h, 3),
        rec("gemm_gate_up_bf16", "gumbel_bf16", h, 4)]) + "\n")
    assert bench.recorded_traffic("gemm_gate_up_bf16", "mixtral_bf16")["bytes_per_launch"] == 3
    assert bench.recorded_traffic("gemm_gate_up_bf16", "gumbel_bf16")["bytes_per_launch"] == 4
    assert bench.recorded_traffic("combine", "mixtral_bf16") is None
    # any change to a kernel source retires the records
    (csrc / "k.hip").write_text("kernel source two\n")
    assert bench.kernel_source_hash() != h
    assert bench.recorded_traffic("gemm_gate_up_bf16", "mixtral_bf16") is None
    # a header counts as a kernel source too
    (csrc / "k.hip").write_text("kernel source one\n")
    assert bench.kernel_source_hash() == h
    (csrc / "k.h").write_text("#pragma once\n")
    assert bench.recorded_traffic("gemm_gate_up_bf16", "mixtral_bf16") is None


# the workloads whose HBM traffic profiles/ records, and the weight type of each
PROFILED = {"mixtral_bf16": "bf16", "gumbel_bf16": "bf16", "fine_shared_bf16": "bf16",
            "fine_grouped_bf16": "bf16", "skewed_fp8": "fp8", "skewed_fp8_reroute": "fp8",
            "skewed_fp8_decode": "fp8", "skewed_int4_decode": "int4"}


@pytest.mark.parametrize("workload", sorted(PROFILED))
def test_committed_traffic_records_describe_the_committed_kernels(workload):
    """Every profiled workload has copy-calibrated FETCH/WRITE records of both expert
    passes taken on exactly these kernel sources (a kernel edit without a new
    profile leaves bench.py's `traffic` null, and this test names the workload)."""
    wt = PROFILED[workload]
    for kernel in (f"gemm_gate_up_{wt}", f"gemm_down_{wt}"):
        rec = bench.recorded_traffic(kernel, workload)
        assert rec is not None, f"profiles/ holds no traffic record of {kernel} at {workload} for these sources"
        assert rec["bytes_per_launch"] > 0
