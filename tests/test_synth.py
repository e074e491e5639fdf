"""The seeded input generator: determinism, bf16 rounding and id layout (CPU only)."""
import numpy as np

import flux_synth as fs


def test_bf16_round_to_nearest_even():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even mantissa (1.0);
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6 -> even (1 + 2^-6)
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -2.5, 0.0],
                 dtype=np.float32)
    r = fs.round_to_bf16(x)
    assert r[0] == 1.0
    assert r[1] == 1 + 2 ** -6
    assert r[2] == 1 + 2 ** -7
    assert r[3] == -2.5 and r[4] == 0.0
    bits = fs.to_bf16_bits(np.array([1.0, -2.0], dtype=np.float32))
    assert bits.tolist() == [0x3F80, 0xC000]


def test_rounded_values_are_bf16_representable():
    x = fs.normal(7, "w", (1000,), std=0.02)
    u = x.view(np.uint32)
    assert not (u & 0xFFFF).any()


def test_streams_are_deterministic_and_keyed_by_name():
    a = fs.normal(1, "a", (64,))
    assert np.array_equal(a, fs.normal(1, "a", (64,)))
    assert not np.array_equal(a, fs.normal(1, "b", (64,)))
    assert not np.array_equal(a, fs.normal(2, "a", (64,)))


def test_weight_generation_order_independent():
    specs = fs.single_block_weight_specs(256, 768)
    all_w = fs.make_weights(specs, 5, "bf16")
    one = fs.make_weights(specs, 5, "bf16", names=["linear2"], threads=1)
    assert np.array_equal(all_w["linear2"], one["linear2"])
    g = all_w["q_norm"]
    assert g.dtype == np.float32 and abs(g.mean() - 1) < 0.01


def test_ids():
    img = fs.image_ids(64)
    assert img.shape == (64, 4) and img.dtype == np.int32
    assert img[9].tolist() == [0, 1, 1, 0]
    assert img[63].tolist() == [0, 7, 7, 0]
    txt = fs.text_ids(16)
    assert txt[5].tolist() == [0, 0, 0, 5]


def test_workload_shapes():
    w = fs.workload("klein9b_double_1024")
    assert (w.dim, w.heads, w.mlp_hidden, w.n_img, w.n_txt, w.seq) == (4096, 32, 12288, 4096, 512, 4608)
    assert w.dim == w.heads * 128 and w.mlp_hidden == 3 * w.dim
    d = fs.workload("dev_pair_2048")
    assert d.seq == 16896 and d.grid == 128
