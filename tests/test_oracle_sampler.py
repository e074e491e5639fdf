"""Pins of the oracle's sampling loop (CPU): latent packing against an independent library
routine, the ids against the pages' tiny example, the noise schedule's closed form, and the
Euler / guidance structure through identities a wrong time index, sign, state hand-over or
combination would break."""
import einops
import numpy as np
import pytest

import flux_synth as fs
from oracle import flux_oracle as O


def tiny(nd=1, ns=1, **kw):
    return fs.workload("tiny_single_f32", kind="step", in_channels=32, context_dim=48,
                       n_double=nd, n_single=ns, n_img=16, n_txt=5, **kw)


@pytest.mark.parametrize("shape", [(1, 32, 16, 16), (2, 8, 6, 10), (1, 3, 2, 2)])
def test_pack_matches_einops_rearrange(shape):
    z = np.random.default_rng(1).standard_normal(shape)
    ref = einops.rearrange(z, "b c (h ph) (w pw) -> b (h w) (c ph pw)", ph=2, pw=2)
    assert np.array_equal(O.pack_latents(z), ref)
    assert np.array_equal(O.unpack_latents(ref, shape[2], shape[3]), z)


def test_pack_literal_patch():
    # one 2x2 patch of two channels: token channels (c0: a b c d | c1: e f g h)
    z = np.array([[[[1, 2], [3, 4]], [[5, 6], [7, 8]]]], dtype=np.float64)
    assert np.array_equal(O.pack_latents(z), [[[1, 2, 3, 4, 5, 6, 7, 8]]])
    with pytest.raises(ValueError):
        O.pack_latents(np.zeros((1, 1, 3, 4)))


def test_generation_ids_follow_the_tiny_example():
    # the shape trace's tiny case: 64 image tokens (0, row, col, 0) on an 8 x 8 grid and
    # 16 text tokens (0, 0, 0, i) -- the same ids the seeded inputs use
    img, txt = O.generation_ids(8, 8, 16)
    assert np.array_equal(img, fs.image_ids(64)) and np.array_equal(txt, fs.text_ids(16))
    img, txt = O.generation_ids(2, 3, 0)
    assert img.tolist() == [[0, 0, 0, 0], [0, 0, 1, 0], [0, 0, 2, 0],
                            [0, 1, 0, 0], [0, 1, 1, 0], [0, 1, 2, 0]]
    assert txt.shape == (0, 4)


def test_uniform_sigmas_closed_form():
    s = O.uniform_sigmas(4)
    assert s.dtype == np.float32 and s.tolist() == [1.0, 0.75, 0.5, 0.25, 0.0]
    s = O.uniform_sigmas(50)
    assert len(s) == 51 and s[0] == 1 and s[-1] == 0 and np.all(np.diff(s) < 0)
    np.testing.assert_allclose(np.diff(s.astype(np.float64)), -1 / 50, rtol=0, atol=1e-7)


def _run(wl, inp, sigmas, **kw):
    return O.denoise(inp["noise"], inp["ctx"], inp["weights"], sigmas, wl.n_double,
                     wl.n_single, **kw)


def test_zero_velocity_is_identity():
    wl = tiny()
    inp = fs.sample_inputs(wl, 8, 8)
    w = dict(inp["weights"])
    w["proj_out"] = np.zeros_like(w["proj_out"])
    out = O.denoise(inp["noise"], inp["ctx"], w, O.uniform_sigmas(3), 1, 1)
    assert np.array_equal(out, inp["noise"].astype(np.float64))


def test_one_step_is_euler_from_the_first_level():
    # velocity taken at sigma_0, step of (sigma_1 - sigma_0): a velocity read at sigma_1,
    # or a flipped sign, fails
    wl = tiny()
    inp = fs.sample_inputs(wl, 8, 8)
    sig = np.array([0.8, 0.3], dtype=np.float32)
    out = _run(wl, inp, sig)
    x = O.pack_latents(inp["noise"])
    img_ids, txt_ids = O.generation_ids(4, 4, wl.n_txt)
    def v_at(t):
        return O.denoiser_step(x, inp["ctx"], np.float32([t]), inp["weights"], img_ids, txt_ids,
                               1, 1)
    d = float(sig[1]) - float(sig[0])
    ref = O.unpack_latents(x + d * v_at(sig[0]), 8, 8)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13)
    wrong = O.unpack_latents(x + d * v_at(sig[1]), 8, 8)
    assert np.abs(out - wrong).max() > 1e-3


def test_steps_compose():
    # sampling over [s0, s1, s2] = sampling [s0, s1], then [s1, s2] from that result
    wl = tiny()
    inp = fs.sample_inputs(wl, 6, 10)
    full = _run(wl, inp, [1.0, 0.625, 0.25])
    half = _run(wl, inp, [1.0, 0.625])
    inp2 = dict(inp, noise=half)
    np.testing.assert_allclose(full, _run(wl, inp2, [0.625, 0.25]), rtol=0, atol=1e-13)


def test_guidance_scale_one_and_zero_select_one_branch():
    wl = tiny(batch=2)
    inp = fs.sample_inputs(wl, 8, 8, with_uncond=True)
    sig = O.uniform_sigmas(2)
    cond = _run(wl, inp, sig)
    unc = O.denoise(inp["noise"], inp["ctx_uncond"], inp["weights"], sig, 1, 1)
    np.testing.assert_allclose(_run(wl, inp, sig, ctx_uncond=inp["ctx_uncond"], guidance=1.0),
                               cond, rtol=0, atol=1e-12)
    np.testing.assert_allclose(_run(wl, inp, sig, ctx_uncond=inp["ctx_uncond"], guidance=0.0),
                               unc, rtol=0, atol=1e-12)
    # equal conditions: guidance has nothing to amplify
    assert np.array_equal(_run(wl, inp, sig, ctx_uncond=inp["ctx"], guidance=4.0), cond)
    # one guided step extrapolates from the unconditional result through the conditional
    # one (the state after one step is affine in the velocity)
    one = O.uniform_sigmas(1)
    c1, u1 = _run(wl, inp, one), O.denoise(inp["noise"], inp["ctx_uncond"], inp["weights"], one, 1, 1)
    g1 = _run(wl, inp, one, ctx_uncond=inp["ctx_uncond"], guidance=3.0)
    np.testing.assert_allclose(g1, u1 + 3.0 * (c1 - u1), rtol=0, atol=1e-12)
    assert np.abs(g1 - c1).max() > 1e-3
    np.testing.assert_allclose(O.cfg_combine(np.float64([2.0]), np.float64([1.0]), 3.0), [4.0])
