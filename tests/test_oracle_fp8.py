"""Pins of the fp8 weight-cache oracle (model card, Help wanted: decode once into
a resident fp8 copy).  Each pin compares the oracle with something other than
itself: torch's float8_e4m3fn type (a library definition of OCP e4m3), closed
forms for the power-of-two scale, exact round trips, explicit loops, and the
card's size figure."""

import numpy as np
import torch

import oracle as O
from block_diffusion_lm_tq4_amd import inputs as I

SB = I.sign_bits()


def test_e4m3_table_matches_torch_float8():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = ref.to(torch.float32).numpy().astype(np.float64)
    mine = O.e4m3_values()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.nanmax(mine) == 448.0 and mine[0x01] == 2.0 ** -9


def _torch_codes(v):
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_e4m3_round_matches_torch_cast():
    rng = np.random.default_rng(0)
    pos = np.unique(np.abs(O.e4m3_values()[~np.isnan(O.e4m3_values())]))
    mids = (pos[:-1] + pos[1:]) / 2                # exact ties, all of them
    v = np.concatenate([
        pos, -pos, mids, -mids,
        rng.uniform(-448, 448, 4000),
        rng.standard_normal(4000) * 2.0 ** rng.integers(-12, 8, 4000),
        [0.0, -0.0, 2.0 ** -10, -2.0 ** -10, 3 * 2.0 ** -11, 447.99, 448.0],
    ]).astype(np.float32)
    v = v[np.abs(v) <= 448]
    assert np.array_equal(O.e4m3_round(v.astype(np.float64)), _torch_codes(v))


def test_e4m3_round_rejects_out_of_range():
    import pytest
    with pytest.raises(ValueError):
        O.e4m3_round(np.array([448.5]))


def test_e8m0_exponent_closed_forms():
    rng = np.random.default_rng(1)
    a = np.abs(rng.standard_normal(2000)) * 2.0 ** rng.integers(-60, 60, 2000)
    e = O.e8m0_exponent(a)
    assert np.all(a <= 448.0 * 2.0 ** e)
    assert np.all(a > 448.0 * 2.0 ** (e - 1))
    assert list(O.e8m0_exponent(np.array([448.0, np.nextafter(448.0, 1e9), 224.0, 1.0, 0.0,
                                          448.0 * 2.0 ** 20, 1e-300, 1e300]))) == \
        [0, 1, -1, -8, -127, 20, -127, 127]


def test_mx_quantize_round_trip_bounds_and_exact_values():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((7, 96)) * 2.0 ** rng.integers(-20, 20, (7, 1))
    codes, scales = O.mx_quantize(v)
    back = O.mx_dequant(codes, scales)
    e = np.repeat(scales.astype(np.int64) - 127, 32, axis=1)
    # half a unit in the last place: 2^-4 relative in the normal range, 2^(e-10) below it
    assert np.all(np.abs(back - v) <= np.maximum(2.0 ** -4 * np.abs(v), 2.0 ** (e - 10)))
    # every block's largest magnitude lands in (224, 448] before rounding
    amax = np.max(np.abs(v.reshape(7, 3, 32)), axis=-1)
    scaled = amax / 2.0 ** (scales.astype(np.int64) - 127)
    assert np.all((scaled > 224) & (scaled <= 448))
    # values on the e4m3 grid times the block's scale come back exactly
    grid = O.e4m3_values()[rng.integers(0, 0x7F, (4, 64))] * np.where(rng.random((4, 64)) < .5, -1, 1)
    grid[:, 0] = 448.0
    grid[:, 32] = -448.0
    exact = grid * 2.0 ** 5
    c2, s2 = O.mx_quantize(exact)
    assert np.all(s2 == 127 + 5) and np.array_equal(O.mx_dequant(c2, s2), exact)
    # an all-zero block stores scale byte 0 and zero codes; -0.0 keeps its sign
    c3, s3 = O.mx_quantize(np.array([[0.0] * 31 + [-0.0]]))
    assert s3[0, 0] == 0 and np.all(c3[0, :31] == 0) and c3[0, 31] == 0x80


def test_linear_fp8_brute_force_elements():
    w = I.weights(12, 64)
    x = I.activations_bf16(3, 64)
    codes, scales = O.fp8_cache(O.pack(w, SB), SB)
    y = O.linear_fp8(x, codes, scales)
    xq, xs = O.act_mxfp8(x)
    vals = O.e4m3_values()
    for m in range(3):
        for n in range(12):
            acc = 0.0
            for k in range(64):
                xv = vals[xq[m, k]] * 2.0 ** (int(xs[m, k // 32]) - 127)
                wv = vals[codes[n, k]] * 2.0 ** (int(scales[n, k // 32]) - 127)
                acc += xv * wv
            assert abs(acc - y[m, n]) <= 1e-12 * max(1.0, abs(acc))


def test_fp8_cache_is_the_decoded_weights_rounded():
    w = I.weights(40, 128, "student_t3")
    p = O.pack(w, SB)
    codes, scales = O.fp8_cache(p, SB)
    assert codes.shape == (40, 128) and scales.shape == (40, 4)
    wh = O.dequant(p, SB)
    back = O.mx_dequant(codes, scales)
    e = np.repeat(scales.astype(np.int64) - 127, 32, axis=1)
    assert np.all(np.abs(back - wh) <= np.maximum(2.0 ** -4 * np.abs(wh), 2.0 ** (e - 10)))


def test_linear_fp8_error_against_the_exact_layer():
    """Both operands carry e4m3 rounding (at most 2^-4 relative each); on
    Gaussian data the product's relative Frobenius error is a few percent."""
    w = I.weights(256, 512)
    x = I.activations_bf16(16, 512)
    p = O.pack(w, SB)
    y = O.linear_fp8(x, *O.fp8_cache(p, SB))
    ref = O.linear(x, p, SB)
    relf = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert 0.005 < relf < 0.06, relf


def test_cache_size_matches_the_card():
    # one byte per weight plus one scale byte per 32 weights, for the 59e9
    # weights of both towers: the card quotes about 63 GB
    size_gb = 59e9 * (1 + 1 / 32) / 1e9
    assert 55 < size_gb < 66


def _exact_cache(w):
    """Cache of an integer matrix whose 32-blocks quantize exactly."""
    c, sc = O.mx_quantize(np.asarray(w, np.float64))
    assert np.array_equal(O.mx_dequant(c, sc), w)
    return c, sc


def test_moe_fp8_exact_case_equals_integer_moe():
    # one-hot tokens pick a column of W1, so u = W1[:, a] in {-1..3} and
    # h = relu(u)^2 in {0, 1, 4, 9}: every quantization on the way is exact
    # (9 * 2^5 = 288 = 1.125 * 2^8), and the layer reduces to integer
    # arithmetic with power-of-two gates
    rng = np.random.default_rng(5)
    e_n, n1, k, t, topk = 5, 64, 96, 7, 2
    w1 = rng.integers(-1, 4, size=(e_n, n1, k)).astype(np.float64)
    w2 = rng.integers(-3, 4, size=(e_n, k, n1)).astype(np.float64)
    cols = rng.integers(0, k, size=t)
    x = np.zeros((t, k), np.float32)
    x[np.arange(t), cols] = 1.0
    ids = np.array([[0, 3], [1, 2], [4, 0], [2, 2], [3, -1], [0, 5], [1, 4]], np.int32)
    g = np.array([[0.5, 0.25], [1, 2], [0.125, 4], [1, 1], [8, 1], [0.5, 1], [2, 0.5]])
    want = np.zeros((t, k))
    for ti in range(t):
        for j in range(topk):
            e = ids[ti, j]
            if 0 <= e < e_n:
                h = np.maximum(w1[e][:, cols[ti]], 0) ** 2
                want[ti] += g[ti, j] * (w2[e] @ h)
    got = O.moe_fp8(O.bf16_bits_from_f32(x), ids, g,
                    [_exact_cache(w) for w in w1], [_exact_cache(w) for w in w2])
    assert np.array_equal(got, want)


def test_moe_fp8_rounds_the_hidden_activations():
    # hand-derived roundings of h in one 32-block of the hidden layer:
    #   u = 5, 1: h = 25 is the block's largest, e = -4 (25 <= 448/16 = 28 but
    #   not <= 14); 25 * 16 = 400 lies halfway between 384 and 416 (spacing
    #   32 in [256, 512)), the tie goes to the even code 384 -> h_q = 24.
    #   u = 7 in another row: h = 49, e = -3, 49 * 8 = 392 -> 384 -> h_q = 48.
    n1, k = 32, 32
    w1 = np.zeros((n1, k))
    w1[0, 0], w1[1, 0], w1[2, 0] = 5, 1, 3
    w1[0, 1] = 7
    w2 = np.eye(k, n1)                                # o = h_q itself
    x = np.zeros((2, k), np.float32)
    x[0, 0], x[1, 1] = 1.0, 1.0
    ids = np.zeros((2, 1), np.int32)
    g = np.ones((2, 1))
    got = O.moe_fp8(O.bf16_bits_from_f32(x), ids, g, [_exact_cache(w1)], [_exact_cache(w2)])
    assert got[0, 0] == 24.0 and got[0, 1] == 1.0 and got[0, 2] == 9.0
    assert got[1, 0] == 48.0 and not got[1, 1:].any()
    assert not got[0, 3:].any()
