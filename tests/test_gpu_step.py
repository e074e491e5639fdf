"""Denoiser-step parity with the fp64 oracle through the C ABI."""
import os

import numpy as np
import pytest

import flux_synth as fs
from oracle import flux_oracle as O
from tests import flux_gpu as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_transformer_mmdit_amd import flux as F
    F.lib()


def small_step(dtype, batch=1, n_txt=16, n_img=64, nd=2, ns=2, dim=256, heads=2):
    return fs.workload("tiny_single_f32", kind="step", dtype=dtype, batch=batch, n_txt=n_txt,
                       n_img=n_img, dim=dim, heads=heads, mlp_hidden=3 * dim, in_channels=128,
                       context_dim=384, n_double=nd, n_single=ns, t_fixed=None,
                       seed=3000 + n_img + batch)


@pytest.mark.parametrize("dtype,batch,n_txt,n_img", [("f32", 1, 16, 64), ("bf16", 1, 16, 64),
                                                     ("bf16", 2, 7, 36), ("bf16", 1, 0, 64)])
def test_small_step(dtype, batch, n_txt, n_img):
    wl = small_step(dtype, batch, n_txt, n_img)
    inp = fs.step_inputs(wl)
    out = G.run_step(wl, inp)
    ref = O.denoiser_step(inp["x"], inp["ctx"], inp["t"], inp["weights"], inp["img_ids"],
                          inp["txt_ids"], wl.n_double, wl.n_single)
    G.assert_close(G.host(out), ref, dtype, f"step {dtype} B={batch} Nt={n_txt} Ni={n_img}")


def test_step_d512_more_blocks():
    wl = small_step("bf16", 1, 32, 256, nd=3, ns=5, dim=512, heads=4)
    inp = fs.step_inputs(wl)
    out = G.run_step(wl, inp)
    ref = O.denoiser_step(inp["x"], inp["ctx"], inp["t"], inp["weights"], inp["img_ids"],
                          inp["txt_ids"], wl.n_double, wl.n_single)
    G.assert_close(G.host(out), ref, "bf16", "step D=512 3+5 blocks")


@pytest.mark.parametrize("precision", [0, 1, 2])
@pytest.mark.parametrize("dim", [1024, 2048])
def test_full_depth_step_narrow(dim, precision):
    """The Klein-9B depth (8 double + 24 single blocks) at D 1024 / 2048 with 128 + 1024
    tokens against the fp64 oracle, whole output, in every operand precision."""
    wl = fs.workload("klein9b_step_1024", dim=dim, heads=dim // 128, mlp_hidden=3 * dim,
                     n_img=1024, n_txt=128, context_dim=1536)
    inp = fs.step_inputs(wl)
    out = G.run_step(wl, inp, precision=precision)
    ref = O.denoiser_step(inp["x"], inp["ctx"], inp["t"], inp["weights"], inp["img_ids"],
                          inp["txt_ids"], wl.n_double, wl.n_single)
    ma, nl = G.assert_close(G.host(out), ref, "bf16",
                            f"step 8+24 blocks D={dim} precision {precision}")
    if precision in (1, 2):
        # hi / lo or binary16 operands shrink the dominant roundings: well inside the bar
        assert nl <= 2.5e-3, nl


# ------------------------------------------------------------------------------------
# the full Klein-9B 1024² step against the stored fp64 oracle output
# ------------------------------------------------------------------------------------
GOLDEN_DIR = os.path.join(os.path.dirname(__file__), "golden")
GOLDEN_9B = os.path.join(GOLDEN_DIR, "klein9b_step_1024.npy")


@pytest.fixture(scope="module")
def klein9b_step():
    """The seeded weights and inputs of tests/golden/make_step_golden.py (9.08B parameters,
    generated here block by block and uploaded in bf16), and a runner of the whole step
    (8 double + 24 single blocks) through flux_denoiser_step with the workspace and launches
    bench.py times.  The runner returns the host copy of the output [1, 4096, 128]."""
    if not os.path.exists(GOLDEN_9B):
        pytest.skip("golden output not generated")
    wl = fs.workload("klein9b_step_1024")
    inp = fs.step_inputs(wl, with_weights=False)
    lw = fs.LazyWeights(fs.step_weight_specs(wl), wl.seed, wl.dtype, threads=16)
    w_dev = {}
    for grp in lw.groups():
        for name in lw.group_names(grp):
            w_dev[name] = G.dev(lw[name], "f32" if name.endswith("_norm") else wl.dtype)

    def run(precision):
        out = G.host(G.run_step(wl, inp, w_dev, precision=precision))
        G.torch().cuda.empty_cache()  # the binary16 copy of the block weights
        assert np.isfinite(out).all()
        return out[0]

    yield run
    w_dev.clear()


def golden_9b():
    ref = np.load(GOLDEN_9B, allow_pickle=False)
    assert ref.shape == (4096, 128) and ref.dtype == np.float64
    return ref


def test_klein9b_step_1024_split_precision_vs_fp64(klein9b_step):
    """North-star parity of the headline workload: the whole output of the Klein-9B 1024^2
    step (4096 x 128 values) against the exact fp64 step, max-abs 3e-2 and nL2 1e-2, with the
    LayerNorm and SwiGLU outputs carried as bf16 hi + lo pairs (FLUX_PRECISION_SPLIT)."""
    from diffusion_transformer_mmdit_amd import flux as F
    got = klein9b_step(F.FLUX_PRECISION_SPLIT)
    G.assert_close(got, golden_9b(), "bf16", "Klein-9B 1024^2 step (split precision) vs fp64")


def test_klein9b_step_1024_f16_precision_vs_fp64(klein9b_step):
    """The same whole-output parity with the block linears' operands in binary16
    (FLUX_PRECISION_F16: LayerNorm, attention and SwiGLU outputs and the block weights),
    which keeps bf16's MFMA rate; the oracle's storage study with these rounding points
    (128 + 1024 tokens at D 4096) predicts max-abs 1.16e-2 / nL2 1.76e-3."""
    from diffusion_transformer_mmdit_amd import flux as F
    got = klein9b_step(F.FLUX_PRECISION_F16)
    G.assert_close(got, golden_9b(), "bf16", "Klein-9B 1024^2 step (binary16 precision) vs fp64")


@pytest.mark.xfail(strict=True, reason=(
    "with every GEMM operand stored in bf16, the roundings of the LayerNorm and SwiGLU "
    "outputs are amplified through the 32 blocks at D 4096 beyond the bars (measured on the "
    "GPU: max-abs 8.1e-2, nL2 1.17e-2 over the whole output; the oracle's bf16 storage mode "
    "with the same rounding points: 7.3e-2 / 1.18e-2 at 128 + 1024 tokens); "
    "FLUX_PRECISION_SPLIT meets them (7.1e-3 / 1.0e-3)"))
def test_klein9b_step_1024_bf16_precision_vs_fp64(klein9b_step):
    from diffusion_transformer_mmdit_amd import flux as F
    got = klein9b_step(F.FLUX_PRECISION_BF16)
    G.assert_close(got, golden_9b(), "bf16", "Klein-9B 1024^2 step (bf16 precision) vs fp64")
