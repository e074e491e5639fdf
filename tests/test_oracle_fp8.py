"""Pins of the oracle's FP8 (E4M3) linear layer (CPU): the encoder against torch's
independent float8_e4m3fn conversion and the format's closed forms, the rounding bound and
ties, saturation, the per-row quantizer's scale and error bound, and the product against
brute force."""
import numpy as np
import pytest

from oracle import flux_oracle as O


def test_every_code_round_trips():
    codes = np.arange(256, dtype=np.uint8)
    d = O.fp8_decode(codes)
    ok = ~np.isnan(d)
    assert ok.sum() == 254          # S.1111.111 are the two NaNs
    assert np.array_equal(O.fp8_encode(d[ok]), codes[ok])


def test_decode_closed_forms():
    d = O.fp8_decode([0x38, 0x7E, 0x01, 0x07, 0x08, 0x80, 0xB8, 0x3F])
    assert d[0] == 1.0 and d[1] == 448.0 and d[2] == 2.0 ** -9 and d[3] == 7 * 2.0 ** -9
    assert d[4] == 2.0 ** -6 and d[5] == 0.0 and np.signbit(d[5]) and d[6] == -1.0
    assert d[7] == 1.875


def test_encoder_matches_torch_float8_e4m3fn():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.standard_normal(4000) * 30.0, rng.standard_normal(2000) * 1e-2,
                        rng.uniform(-448, 448, 2000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.fp8_encode(x.astype(np.float64)), ref)


def test_rounding_bound_ties_and_saturation():
    rng = np.random.default_rng(5)
    x = rng.uniform(-440, 440, 3000)
    err = np.abs(O.fp8_decode(O.fp8_encode(x)) - x)
    # half a spacing: 2^-4 of the binade's lower end for normals, 2^-10 for subnormals
    binade = np.exp2(np.maximum(np.floor(np.log2(np.abs(x))), -6))
    assert np.all(err <= binade * 2.0 ** -4 + 1e-300)
    # exact midpoints go to the even mantissa
    assert O.fp8_encode([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10]).tolist() == [0x38, 0x3A, 0x00,
                                                                                   0x02]
    assert O.fp8_encode([1e6, -1e6, np.nan]).tolist() == [0x7E, 0xFE, 0x7F]
    # monotone
    y = np.sort(rng.uniform(-448, 448, 500))
    assert np.all(np.diff(O.fp8_decode(O.fp8_encode(y))) >= 0)


def test_row_quantizer_scale_and_error():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((5, 300)) * rng.uniform(0.01, 50, (5, 1))).astype(np.float32)
    x[3] = 0.0
    q, s = O.quantize_rows_fp8(x)
    assert s.dtype == np.float32 and s[3] == 1.0 and not q[3].any()
    dq = O.fp8_decode(q)
    for m in (0, 1, 2, 4):
        assert s[m] == np.float32(np.abs(x[m]).max() / np.float32(448.0))
        assert np.abs(dq[m]).max() == 448.0           # the row maximum maps to 448
        # half a code spacing (2^-4 relative, 2^-10 s below 2^-6 s) plus the fp32
        # rounding of the multiplier and of s
        err = np.abs(dq[m] * s[m] - x[m])
        assert np.all(err <= np.abs(x[m]) * (2.0 ** -4 + 2.0 ** -20) + s[m] * 2.0 ** -10)


def test_linear_matches_brute_force():
    rng = np.random.default_rng(7)
    qa = rng.integers(0, 256, (3, 7)).astype(np.uint8)
    qw = rng.integers(0, 256, (4, 7)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x11
    qw[(qw & 0x7F) == 0x7F] = 0x22
    sa = np.float32([0.5, 2.0, 0.25])
    sw = np.float32([1.0, 0.125, 4.0, 3.0])
    y = O.linear_fp8(qa, sa, qw, sw)
    for m in range(3):
        for n in range(4):
            ref = sum(float(O.fp8_decode(qa[m, k])) * float(O.fp8_decode(qw[n, k]))
                      for k in range(7)) * float(sa[m]) * float(sw[n])
            assert abs(y[m, n] - ref) <= 1e-12 * max(1.0, abs(ref))
