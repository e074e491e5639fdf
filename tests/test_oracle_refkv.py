"""Pins of the oracle's reference-image K/V cache (CPU): the masked attention against brute
force, the cache's exactness (cached mode reproduces extract mode), the reduction to the
plain step without references, the cache's independence of the image, text and timestep
(reference tokens attend only to references, at a fixed timestep), and a duplicate-token
identity that ties the reference path to the plain (pinned) blocks."""
import math

import numpy as np
import pytest

import flux_synth as fs
from oracle import flux_oracle as O


def tiny(nd=1, ns=2, n_txt=5, **kw):
    return fs.workload("tiny_single_f32", kind="step", in_channels=32, context_dim=48,
                       n_double=nd, n_single=ns, n_img=16, n_txt=n_txt, **kw)


def refs_for(wl, R=1, gh=3, gw=4, seed=5):
    ref = fs.normal(seed, "ref", (wl.batch, R * gh * gw, wl.in_channels), dtype="f32")
    return ref, O.reference_ids(R, gh, gw)


def extract(wl, inp, ref, rid, **kw):
    return O.step_extract(inp["x"], ref, inp["ctx"], inp["t"], inp["weights"], inp["img_ids"],
                          rid, inp["txt_ids"], wl.n_double, wl.n_single, **kw)


def cached(wl, inp, cache):
    return O.step_cached(inp["x"], inp["ctx"], inp["t"], inp["weights"], inp["img_ids"],
                         inp["txt_ids"], cache, wl.n_double, wl.n_single)


def test_masked_attention_matches_brute_force():
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((1, n, 1, 4)) for n in (3, 5, 5))
    allowed = np.array([[1, 1, 0, 0, 1], [0, 0, 1, 1, 0], [1, 1, 1, 1, 1]], dtype=bool)
    got = O.attention_masked(q, k, v, allowed)
    for i in range(3):
        keys = [j for j in range(5) if allowed[i, j]]
        s = [sum(q[0, i, 0, c] * k[0, j, 0, c] for c in range(4)) / 2.0 for j in keys]
        e = [math.exp(x) for x in s]
        ref = [sum(e[a] * v[0, j, 0, c] for a, j in enumerate(keys)) / sum(e) for c in range(4)]
        np.testing.assert_allclose(got[0, i], ref, rtol=1e-13, atol=1e-13)
    # no mask: the unmasked attention
    q2 = rng.standard_normal((1, 5, 1, 4))
    np.testing.assert_allclose(O.attention_masked(q2, k, v), O.attention(q2, k, v), rtol=1e-13,
                               atol=1e-13)


def test_reference_ids_literal():
    ids = O.reference_ids(2, 1, 2)
    assert ids.tolist() == [[1, 0, 0, 0], [1, 0, 1, 0], [2, 0, 0, 0], [2, 0, 1, 0]]
    assert O.reference_ids(0, 3, 3).shape == (0, 4)


def test_cached_mode_reproduces_extract_mode():
    wl = tiny(batch=2)
    inp = fs.step_inputs(wl)
    ref, rid = refs_for(wl, R=2, gh=2, gw=3)
    out, cache = extract(wl, inp, ref, rid)
    assert len(cache) == wl.n_double + wl.n_single
    assert cache[0][0].shape == (2, 12, wl.heads, 128)
    np.testing.assert_allclose(cached(wl, inp, cache), out, rtol=0, atol=1e-12)
    # and the references matter: another reference changes the output
    ref2 = ref + 0.5
    out2, _ = extract(wl, inp, ref2, rid)
    assert np.abs(out2 - out).max() > 1e-4


def test_without_references_both_modes_are_the_plain_step():
    wl = tiny()
    inp = fs.step_inputs(wl)
    plain = O.denoiser_step(inp["x"], inp["ctx"], inp["t"], inp["weights"], inp["img_ids"],
                            inp["txt_ids"], wl.n_double, wl.n_single)
    out, cache = extract(wl, inp, np.zeros((1, 0, wl.in_channels)), np.zeros((0, 4), np.int32))
    np.testing.assert_allclose(out, plain, rtol=0, atol=1e-13)
    np.testing.assert_allclose(cached(wl, inp, cache), plain, rtol=0, atol=1e-13)


def test_cache_does_not_depend_on_image_text_or_timestep():
    wl = tiny()
    inp = fs.step_inputs(wl)
    ref, rid = refs_for(wl)
    _, c1 = extract(wl, inp, ref, rid)
    other = dict(inp, x=inp["x"] * -0.7 + 0.3, ctx=inp["ctx"] + 1.0,
                 t=np.float32([0.91]))
    _, c2 = extract(wl, other, ref, rid)
    for (k1, v1), (k2, v2) in zip(c1, c2):
        np.testing.assert_allclose(k1, k2, rtol=0, atol=1e-13)
        np.testing.assert_allclose(v1, v2, rtol=0, atol=1e-13)
    # the fixed timestep does matter
    _, c3 = extract(wl, inp, ref, rid, t_ref=0.4)
    assert np.abs(c3[-1][0] - c1[-1][0]).max() > 1e-6


def test_duplicate_image_tokens_reproduce_the_plain_step():
    # image tokens identical to the reference tokens (same values, same ids) at t = t_ref,
    # no text: every image key has an identical reference twin, which leaves each image
    # query's attention output unchanged, so the image rows follow the plain step on the
    # reference tokens (this ties the reference rows to the image-stream weights, norms,
    # positions and the fixed-timestep modulation)
    wl = tiny(n_txt=0)
    inp = fs.step_inputs(wl)
    ref = inp["x"]
    plain = O.denoiser_step(ref, inp["ctx"], np.float32([0.0]), inp["weights"], inp["img_ids"],
                            inp["txt_ids"], wl.n_double, wl.n_single)
    out, _ = O.step_extract(ref, ref, inp["ctx"], np.float32([0.0]), inp["weights"],
                            inp["img_ids"], inp["img_ids"], inp["txt_ids"], wl.n_double,
                            wl.n_single, t_ref=0.0)
    np.testing.assert_allclose(out, plain, rtol=0, atol=1e-12)


def test_sampling_with_cache_equals_recomputing_references():
    wl = tiny()
    inp = fs.sample_inputs(wl, 8, 8)
    refs = fs.normal(9, "refs", (1, 2, 8, 4, 6), dtype="f32")
    sig = O.uniform_sigmas(3)
    a = O.denoise_with_refs(inp["noise"], refs, inp["ctx"], inp["weights"], sig, 1, 2)
    b = O.denoise_with_refs(inp["noise"], refs, inp["ctx"], inp["weights"], sig, 1, 2,
                            use_cache=False)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    plain = O.denoise(inp["noise"], inp["ctx"], inp["weights"], sig, 1, 2)
    assert np.abs(a - plain).max() > 1e-4
