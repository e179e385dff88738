"""Pins of the oracle's fp8 e4m3 codec (CPU only): values the OCP format
fixes, round trips, ties to even, saturation and the tensorwise scale."""

import numpy as np

from oracle import fp8


def test_known_codes():
    t = fp8.e4m3_decode_table()
    assert t[0x38] == 1.0 and t[0x40] == 2.0 and t[0x3C] == 1.5 and t[0x30] == 0.5
    assert t[0x7E] == 448.0 and np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x01] == 2.0 ** -9 and t[0x08] == 2.0 ** -6 and t[0x07] == 7 * 2.0 ** -9
    assert t[0xB8] == -1.0 and t[0x00] == 0.0
    finite = t[:0x7F]
    assert np.all(np.diff(finite) > 0)                 # codes 0..126 increase
    assert len(np.unique(finite)) == 127


def test_round_trip_of_every_finite_value():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)], np.uint8)
    np.testing.assert_array_equal(fp8.e4m3_encode(fp8.e4m3_decode(codes)), codes)


def test_ties_go_to_the_even_code_and_large_values_saturate():
    enc = fp8.e4m3_encode
    assert enc(1.0625) == 0x38          # halfway 1.0 (0x38) / 1.125 (0x39)
    assert enc(1.1875) == 0x3A          # halfway 1.125 (0x39) / 1.25 (0x3A)
    assert enc(7.5 * 2.0 ** -9) == 0x08  # halfway 7 * 2^-9 / 2^-6: the normal code is even
    assert enc(0.5 * 2.0 ** -9) == 0x00  # halfway 0 / 2^-9
    assert enc(1.07) == 0x39 and enc(1.05) == 0x38
    assert enc(460.0) == 0x7E and enc(1e9) == 0x7E and enc(-1e9) == 0xFE
    # between two neighbours the nearest wins, on a grid of every interval
    t = fp8.e4m3_decode_table()[:0x7F]
    mid = (t[:-1] + t[1:]) / 2
    below, above = mid - 1e-6 * (t[1:] - t[:-1]), mid + 1e-6 * (t[1:] - t[:-1])
    np.testing.assert_array_equal(fp8.e4m3_encode(below), np.arange(0, 0x7E))
    np.testing.assert_array_equal(fp8.e4m3_encode(above), np.arange(1, 0x7F))


def test_tensorwise_scale_maps_amax_to_448():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(1000).astype(np.float32) * 3
    codes, amax, scale = fp8.quantize_tensorwise(x)
    assert amax == np.max(np.abs(x)) and scale == np.float32(448.0) / np.float32(amax)
    assert np.max(fp8.e4m3_decode(codes) * np.sign(x)) == 448.0 or \
        np.min(fp8.e4m3_decode(codes)) == -448.0
    # relative error of the representation is at most 2^-4 above the subnormal range
    v = fp8.e4m3_decode(codes) / scale
    big = np.abs(x * scale) >= 2.0 ** -6
    assert np.max(np.abs(v[big] - x[big]) / np.abs(x[big])) <= 2.0 ** -4
    zero_codes, a0, s0 = fp8.quantize_tensorwise(np.zeros(5))
    assert a0 == 0.0 and s0 == 1.0 and not zero_codes.any()


def test_nan_is_code_0x7f_and_poisons_the_tensor_scale():
    """OCP e4m3 has one NaN pattern per sign (exponent 15, mantissa 7) and
    no infinities: a NaN value is stored as 0x7F, and one NaN in a tensor
    makes its amax and scale NaN, so every code of that tensor is 0x7F."""
    assert fp8.e4m3_encode(np.nan) == 0x7F and fp8.e4m3_encode(-np.nan) == 0x7F
    assert np.isnan(fp8.e4m3_decode(0x7F))
    x = np.linspace(-3, 3, 11).astype(np.float32)
    x[4] = np.nan
    codes, amax, scale = fp8.quantize_tensorwise(x)
    assert np.isnan(amax) and np.isnan(scale)
    assert np.all(codes == 0x7F)
    # finite values beside a NaN are not what decides the codes
    assert fp8.e4m3_encode(np.array([1.0, np.nan, -2.0])).tolist() == [0x38, 0x7F, 0xC0]


def test_fp8_matmul_is_the_product_of_decoded_values():
    rng = np.random.default_rng(1)
    a = rng.integers(0, 256, (3, 16)).astype(np.uint8)
    b = rng.integers(0, 256, (4, 16)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x38
    b[(b & 0x7F) == 0x7F] = 0x38
    ref = np.array([[sum(fp8.e4m3_decode(a[i, k]) * fp8.e4m3_decode(b[j, k]) for k in range(16))
                     for j in range(4)] for i in range(3)]) * 0.5
    np.testing.assert_allclose(fp8.fp8_matmul(a, b, 0.5), ref, rtol=1e-15)


def test_fp8_linear_is_exact_for_representable_operands():
    # entries in {0, +-1, +-2}: amax 2, scale 224, scaled values 0, +-224, +-448 are
    # e4m3 values, so the fp8 product is the exact product
    from oracle.model import _fp8_linear
    rng = np.random.default_rng(3)
    x = rng.choice([-2.0, -1.0, 0.0, 1.0, 2.0], size=(2, 5, 16))
    W = rng.choice([-2.0, -1.0, 1.0, 2.0], size=(7, 16))
    np.testing.assert_array_equal(_fp8_linear(x, W), x @ W.T)


def test_fp8_forward_model_stays_close_to_the_exact_one():
    # e4m3 keeps 3 mantissa bits: the loss moves by well under its own size, and
    # the straight-through gradients keep their direction
    import oracle
    from oracle.model import param_shapes
    from gpt_pretraining_step_gemms_amd import synthetic
    cfg = dict(n_layer=2, d_model=32, n_head=2, head_dim=16, d_ff=128, vocab=64, seq_len=8,
               rope_base=10000.0, norm_eps=1e-6)
    params = {k: v.astype(np.float64) for k, v in
              synthetic.normal_params(0, param_shapes(cfg), 0.3).items()}
    tok, tgt = synthetic.token_rows(1, 2, 8, 64, "uniform")
    l0, g0 = oracle.loss_and_grads(params, tok, tgt, cfg)
    l8, g8 = oracle.loss_and_grads(params, tok, tgt, dict(cfg, fp8_forward=True))
    assert l8 != l0 and abs(l8 - l0) / l0 < 0.05
    for n in g0:
        a, b = g0[n].ravel(), g8[n].ravel()
        assert a @ b / (np.linalg.norm(a) * np.linalg.norm(b)) > 0.95, n


def test_bf16_round_known_values_and_ties():
    r = fp8.bf16_round
    assert r(1.0) == 1.0 and r(-2.5) == -2.5
    assert r(1.0 + 2.0 ** -8) == 1.0               # halfway to 1 + 2^-7: ties to even (1.0)
    assert r(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6   # halfway 1+2^-7 / 1+2^-6: even is 1+2^-6
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -12) == 1.0 + 2.0 ** -7
    x = np.random.default_rng(0).standard_normal(1000)
    y = r(x)
    assert np.all(np.abs(y - x) <= 2.0 ** -8 * np.abs(x) * (1 + 1e-6))   # unit roundoff 2^-8
    assert np.all(np.ascontiguousarray(y.astype(np.float32)).view(np.uint32) & 0xFFFF == 0)
