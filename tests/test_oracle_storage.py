"""Pins of the oracle's bf16 storage mode (the definition with values rounded where a
bf16 pipeline stores them): the rounding itself against an independent conversion, worked
ties, identities that survive it, and the size of its effect."""
import numpy as np
import pytest

import flux_synth as fs
from oracle import flux_oracle as O


def test_bf16_storage_matches_torch_conversion():
    import torch
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(200_000) * np.exp(rng.uniform(-12, 12, 200_000))).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.bf16_storage(x), ref)


@pytest.mark.parametrize("x,want", [
    (1.0, 1.0),
    (1.0 + 2.0 ** -8, 1.0),                     # halfway, ties to the even neighbour 1.0
    (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),     # halfway, ties to the even 1 + 2^-6
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 1.0),        # rounded to fp32 first: becomes a tie
    (-1.5, -1.5),
    (1.0 / 3.0, 0.333984375),
    (65504.0, 65536.0),
])
def test_bf16_storage_worked_values(x, want):
    assert O.bf16_storage(np.array([x]))[0] == want


@pytest.mark.parametrize("kind", ["double", "single"])
def test_zero_gate_identity_survives_storage_rounding(kind):
    wl = fs.workload("tiny_single_f32", dtype="bf16", t_fixed=None)
    inp = fs.block_inputs(wl, kind=kind)
    D = wl.dim
    w = dict(inp["weights"])
    if kind == "double":
        for s in ("img", "txt"):
            m = w[f"mod_{s}"].copy()
            m[2 * D:3 * D] = 0.0
            m[5 * D:6 * D] = 0.0
            w[f"mod_{s}"] = m
        img, txt = O.double_block(inp["img"], inp["txt"], inp["t"], w, inp["img_ids"],
                                  inp["txt_ids"], storage=O.bf16_storage)
    else:
        m = w["mod"].copy()
        m[2 * D:3 * D] = 0.0
        w["mod"] = m
        img, txt = O.single_block(inp["img"], inp["txt"], inp["t"], w, inp["img_ids"],
                                  inp["txt_ids"], storage=O.bf16_storage)
    np.testing.assert_array_equal(img, inp["img"].astype(np.float64))
    np.testing.assert_array_equal(txt, inp["txt"].astype(np.float64))


@pytest.mark.parametrize("kind", ["double", "single"])
def test_storage_rounding_effect_is_bf16_sized(kind):
    wl = fs.workload("tiny_single_f32", dtype="bf16", t_fixed=None)
    inp = fs.block_inputs(wl, kind=kind)
    fn = O.double_block if kind == "double" else O.single_block
    args = (inp["img"], inp["txt"], inp["t"], inp["weights"], inp["img_ids"], inp["txt_ids"])
    exact, _ = fn(*args)
    rounded, _ = fn(*args, storage=O.bf16_storage)
    upd = exact - inp["img"].astype(np.float64)
    rel = np.linalg.norm(rounded - exact) / np.linalg.norm(upd)
    # a few bf16 roundings (relative 2^-9 each) in the update's inputs
    assert 1e-4 < rel < 2e-2, rel


def test_f16_storage_matches_torch_conversion():
    import torch
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(200_000) * np.exp(rng.uniform(-20, 10, 200_000))).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.f16_storage(x), ref)


@pytest.mark.parametrize("x,want", [
    (1.0, 1.0),
    (1.0 + 2.0 ** -11, 1.0),                     # halfway, ties to the even neighbour 1.0
    (1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -9),     # halfway, ties to the even 1 + 2^-9
    (1.0 / 3.0, 0.333251953125),
    (65504.0, 65504.0),                          # the largest finite value
    (65519.0, 65504.0),                          # below the halfway point to 2^16
    (65520.0, np.inf),                           # halfway: overflows
    (2.0 ** -25, 0.0),                           # half the subnormal spacing: ties to 0
    (3 * 2.0 ** -25, 2.0 ** -23),                # ties to the even subnormal 2 * 2^-24
])
def test_f16_storage_worked_values(x, want):
    assert O.f16_storage(np.array([x]))[0] == want


def test_f16_storage_is_eight_times_finer_than_bf16():
    """Relative rounding error of N(0, 1) values: unit roundoff 2^-11 for binary16 against
    2^-8 for bf16, so the rms error ratio is close to 8."""
    x = np.random.default_rng(7).standard_normal(400_000)
    e16 = np.sqrt(np.mean(((O.f16_storage(x) - x) / x) ** 2))
    eb = np.sqrt(np.mean(((O.bf16_storage(x) - x) / x) ** 2))
    assert 7.0 < eb / e16 < 9.0, eb / e16
    # in binary16's normal range the relative error is at most the unit roundoff (plus the
    # fp32 step's 2^-24)
    nrm = np.abs(x) >= 2.0 ** -14
    assert np.abs((O.f16_storage(x[nrm]) - x[nrm]) / x[nrm]).max() <= 2.0 ** -11 + 2.0 ** -24
