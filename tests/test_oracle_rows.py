"""The oracle's row-sampled blocks equal the full blocks at the sampled rows.

double_block_rows / single_block_rows evaluate the same definition as double_block /
single_block for a subset of output rows (keys and values from every token, the rest per
row); this pins them to the full evaluation on small inputs, so the large-workload GPU
tests that use them compare against the definition itself.
"""
import numpy as np
import pytest

import flux_synth as fs
from oracle import flux_oracle as O


def _inputs(kind, batch=2):
    wl = fs.workload("tiny_single_f32", batch=batch, n_txt=16, n_img=64)
    return fs.block_inputs(wl, kind=kind)


@pytest.mark.parametrize("kind", ["double", "single"])
def test_rows_equal_full_block(kind):
    inp = _inputs(kind)
    full_fn = O.double_block if kind == "double" else O.single_block
    rows_fn = O.double_block_rows if kind == "double" else O.single_block_rows
    img_full, txt_full = full_fn(inp["img"], inp["txt"], inp["t"], inp["weights"],
                                 inp["img_ids"], inp["txt_ids"])
    rng = np.random.default_rng(3)
    ri = np.sort(rng.choice(64, 9, replace=False))
    rt = np.array([0, 5, 15])
    img_r, txt_r = rows_fn(inp["img"], inp["txt"], inp["t"], inp["weights"], inp["img_ids"],
                           inp["txt_ids"], ri, rt)
    np.testing.assert_allclose(img_r, img_full[:, ri], rtol=0, atol=1e-12)
    np.testing.assert_allclose(txt_r, txt_full[:, rt], rtol=0, atol=1e-12)


@pytest.mark.parametrize("kind", ["double", "single"])
def test_rows_with_no_text_rows(kind):
    inp = _inputs(kind, batch=1)
    full_fn = O.double_block if kind == "double" else O.single_block
    rows_fn = O.double_block_rows if kind == "double" else O.single_block_rows
    img_full, _ = full_fn(inp["img"], inp["txt"], inp["t"], inp["weights"], inp["img_ids"],
                          inp["txt_ids"])
    ri = np.array([0, 63])
    img_r, txt_r = rows_fn(inp["img"], inp["txt"], inp["t"], inp["weights"], inp["img_ids"],
                           inp["txt_ids"], ri, np.array([], dtype=np.int64))
    assert txt_r.shape[1] == 0
    np.testing.assert_allclose(img_r, img_full[:, ri], rtol=0, atol=1e-12)
