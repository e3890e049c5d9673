"""Host-side helpers on the CPU: the seeded input generators (any block of rows can be
regenerated on its own, draws are repeatable, distributions have the stated scale) and
bench.py's reading of the committed HBM-counter summary (reported only for the kernel
sources and configuration it was taken on)."""
import os

import numpy as np
import pytest
import torch

import bench
from gemm_epilogues_epilog_amd import inputs


def test_row_ranges_regenerate_the_same_values():
    full = inputs.normal(700, 24, 0.5, "f16", seed=3, tag=1)
    for r0, r1 in ((0, 1), (255, 257), (256, 512), (300, 700), (699, 700)):
        part = inputs.normal(700, 24, 0.5, "f16", seed=3, tag=1, r0=r0, r1=r1)
        assert torch.equal(part, full[r0:r1])


def test_draws_repeat_and_depend_on_seed_and_tag():
    a = inputs.normal(300, 16, 1.0, "bf16", seed=0, tag=1)
    assert torch.equal(a, inputs.normal(300, 16, 1.0, "bf16", seed=0, tag=1))
    assert not torch.equal(a, inputs.normal(300, 16, 1.0, "bf16", seed=1, tag=1))
    assert not torch.equal(a, inputs.normal(300, 16, 1.0, "bf16", seed=0, tag=2))


def test_scale_is_the_standard_deviation():
    x = inputs.normal(4096, 256, 1.0 / 64, "f32", seed=0, tag=1).double().numpy()
    assert abs(x.std() * 64 - 1.0) < 0.01 and abs(x.mean()) < 1e-3


def test_workload_shapes_follow_their_names():
    for name, W in inputs.WORKLOADS.items():
        dims = [int(t) for t in name.replace("_", "x").split("x") if t.isdigit()]
        assert W.m in dims or name.startswith("mlp_bf16_8192") and W.m == 8192, name
        assert W.flops() == 2 * W.m * W.n * W.k


def test_mlp_case_shapes():
    X, W1, b1, W2, dY = inputs.mlp_case(72, 136, 40, 264, "bf16")
    assert X.shape == (72, 264) and W1.shape == (136, 72) and b1.shape == (136,)
    assert W2.shape == (40, 136) and dY.shape == (40, 264)


def test_traffic_summary_is_keyed_to_sources_and_configuration(tmp_path, monkeypatch):
    desc = "f16 RELU_BIAS tile 256x256 test configuration"
    f = tmp_path / "traffic.txt"
    f.write_text("# comment: not a key\n"
                 f"kernel_source_sha: {bench.kernel_source_hash()}\n"
                 f"kernel: {desc}\n"
                 "hbm_bytes_per_launch: 12345\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.read_traffic(desc) == 12345
    assert bench.read_traffic(desc + " other") is None
    f.write_text(f"kernel_source_sha: 0000000000000000\nkernel: {desc}\nhbm_bytes_per_launch: 12345\n")
    assert bench.read_traffic(desc) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.read_traffic(desc) is None


def test_committed_traffic_summary_matches_the_sources():
    # the summary under profiles/ counts for the current headline kernel sources only; a
    # stale one is reported as traffic null by the benchmark (and skipped here, by name)
    kv = {}
    for line in open(bench.TRAFFIC_FILE):
        if ":" in line and not line.startswith(("#", " ")):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv["kernel_source_sha"] != bench.kernel_source_hash():
        pytest.skip("HBM counter summary taken on other kernel sources: the benchmark reports traffic null")
    assert int(kv["hbm_bytes_per_launch"]) > int(kv["algorithmic_bytes_per_launch"])
