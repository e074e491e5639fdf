"""Denoiser-step parity with the fp64 oracle through the C ABI."""
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
