"""Host logic of bench.py (no GPU): the one-GPU refusal, the roofline arithmetic of the
dominant kernel, and the HBM traffic figure being withdrawn once the GEMM sources no longer
match the hash its counter summary records."""
import os
import subprocess
import sys

import pytest

import bench
import flux_synth as fs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_dominant_roofline_arithmetic():
    wl = fs.workload("klein9b_step_1024")
    m, n, k = bench.dominant_shape(wl)
    assert (m, n, k) == (4608, 24576, 4096)  # single-block linear1, MLP part (gate | up)
    line = bench.dominant_roofline(wl, launches=240, mean_us=742.0)
    flops = 2.0 * 4608 * 24576 * 4096
    assert line["algorithmic_flops_per_launch"] == flops
    assert line["achieved"] == pytest.approx(flops / 742e-6 / 1e12, abs=0.05)
    assert line["peak"] == 2500.0 and line["unit"] == "TFLOP/s" and line["bound"] == "mfma"
    assert line["frac"] == pytest.approx(line["achieved"] / 2500.0, abs=1e-4)
    # A and W read once, the SwiGLU output (half the columns) written once, all bf16
    assert line["algorithmic_bytes_per_launch"] == 2 * (4608 * 4096 + 24576 * 4096 + 4608 * 12288)
    assert line["launches_timed"] == 240 and line["avg_launch_us"] == 742.0


def test_traffic_figure_follows_the_kernel_sources(monkeypatch, tmp_path):
    # a summary recording the hash of the current sources is read
    summary = tmp_path / "summary.md"
    summary.write_text("notes\n\ntraffic_bytes_per_launch: 1616541886\n"
                       f"kernel_source_sha256: {bench.kernel_source_hash()}\n")
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(summary))
    assert bench.measured_traffic() == 1616541886
    # another source set hashes differently: the recorded figure no longer applies
    other = tmp_path / "gemm.hip"
    other.write_text("// a changed kernel\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", (str(other),))
    assert bench.measured_traffic() is None
    # a summary without the figure
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(tmp_path / "missing.md"))
    assert bench.measured_traffic() is None


def test_committed_traffic_summary_is_well_formed():
    with open(bench.TRAFFIC_SUMMARY) as f:
        text = f.read()
    assert "traffic_bytes_per_launch:" in text and "kernel_source_sha256:" in text


def test_site_table_and_split_flops():
    from diffusion_transformer_mmdit_amd import flux as F
    wl = fs.workload("klein9b_step_1024")
    rows = {r[0]: r for r in bench.site_table(F, wl)}
    assert len(rows) == 9
    # (name, site, what, launches per step, flops, shape)
    assert rows["single_mlp_in"][4] == 2.0 * 4608 * 24576 * 4096 and rows["single_mlp_in"][3] == 24
    assert rows["single_linear2"][5] == [4608, 4096, 16384]
    # the double block's sites time one launch over both streams' rows
    assert rows["double_mlp_out"][5] == [4608, 4096, 12288] and rows["double_qkv"][3] == 8
    assert rows["single_attention"][4] == 4.0 * 4608 * 4608 * 4096
    # split precision: the LN-fed and SwiGLU-fed products twice, the head's projection twice
    extra = 8 * 2.0 * 4608 * (3 * 4096 ** 2 + 2 * 12288 * 4096 + 12288 * 4096) + \
        24 * 2.0 * 4608 * ((3 * 4096 + 2 * 12288) * 4096 + 12288 * 4096) + 2.0 * 4096 * 4096 * 128
    assert bench.split_mfma_flops(wl) == pytest.approx(bench.step_flops(wl) + extra)


def test_headline_precision_converts_exactly_the_block_linears():
    """The benchmark's FLUX_PRECISION_F16 weight set: the block linears in binary16 (the same
    values as the bf16 weights), everything else untouched (the same tensors)."""
    import torch
    from diffusion_transformer_mmdit_amd import flux as F
    wl = fs.workload("tiny_single_f32", kind="step", dtype="bf16", dim=256, heads=2,
                     mlp_hidden=768, in_channels=64, context_dim=32, n_double=1, n_single=1)
    g = torch.Generator().manual_seed(3)
    w = {name: (0.02 * torch.randn(shape, generator=g)).to(torch.bfloat16) if kind == "w"
         else torch.ones(shape) for name, (shape, kind) in fs.step_weight_specs(wl).items()}
    w16 = bench.to_headline_precision(F, w)
    assert set(w16) == set(w)
    for name, v in w.items():
        if F.is_block_linear(name):
            assert w16[name].dtype == torch.float16, name
            # bf16 values in binary16's normal range convert exactly; below 2^-14 (its
            # subnormals) the error is at most half the subnormal spacing, 2^-25
            a, b = w16[name].double(), v.double()
            nrm = b.abs() >= 2.0 ** -14
            assert torch.equal(a[nrm], b[nrm]), name
            assert (a - b).abs().max().item() <= 2.0 ** -25, name
        else:
            assert w16[name] is v, name
    # one double block (4 linears per stream, 2 streams) and one single block (2 linears)
    assert sum(F.is_block_linear(n) for n in w) == 8 + 2
