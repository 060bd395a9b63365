"""Pins of the oracle's TQ4_1S encoder and decoder.

* brute force: the threshold rule equals nearest-level search (ties -> lower);
* special cases: zero block, one-hot block, constructed ties;
* the model card's measured reconstruction cosine ~0.997, uniform across
  tensor types (section *What "Config-I" means*), which singles out the
  absmax scale reading;
* the card's ~5 bits/weight and its 118 GB -> 38 GB sizes (same section and
  its size table), as closed forms.
"""

import numpy as np
import pytest

import oracle as O
from block_diffusion_lm_tq4_amd import inputs as I

SB = I.sign_bits()


def _cos(a, b):
    a = a.astype(np.float64).ravel()
    b = b.astype(np.float64).ravel()
    return float(a @ b / np.linalg.norm(a) / np.linalg.norm(b))


def test_threshold_rule_is_nearest_level():
    w = I.weights(512, 256)
    z = O.rotate_blocks(w.reshape(512, 8, 32), SB)
    sb = O.half_scales(z)
    s = np.repeat(O.f64_from_bf16_bits(sb), 16, axis=-1)
    q = O.codes_for(z, s)
    cb = O.codebook().astype(np.float64)
    # brute force: argmin over the 16 reconstruction values, first (lower) on ties
    dist = np.abs(z[..., None] - s[..., None] * cb)
    assert np.array_equal(q, np.argmin(dist, axis=-1).astype(np.uint8))
    q2, s2 = O.unpack(O.pack(w, SB))
    assert np.array_equal(q2, q) and np.array_equal(s2, sb)


def test_constructed_ties_go_to_lower_index():
    m = O.midpoints()
    scale = np.float64(0.0625)       # a bf16 value
    z = scale * m                    # exactly on every midpoint
    assert np.array_equal(O.codes_for(z, scale), np.arange(15, dtype=np.uint8))
    z_up = np.nextafter(z, np.inf)
    assert np.array_equal(O.codes_for(z_up, scale), np.arange(1, 16, dtype=np.uint8))


def test_zero_block_and_zero_half():
    w = np.zeros((2, 64), dtype=np.float32)
    p = O.pack(w, SB)
    assert not p.any()
    assert not O.dequant(p, SB).any()


def test_one_hot_block():
    for i in (0, 5, 31):
        for a in (1.0, -0.37, 3e-3):
            w = np.zeros((1, 32), dtype=np.float32)
            w[0, i] = a
            q, s = O.unpack(O.pack(w, SB))
            assert set(np.unique(q)) <= {0, 15}
            wh = O.dequant(O.pack(w, SB), SB)[0]
            e = np.zeros(32)
            e[i] = np.float32(a)
            # only the bf16 rounding of the scale (rel. <= 2^-9) remains
            assert np.max(np.abs(wh - e)) <= abs(a) * 2 ** -8


def test_scale_is_absmax_rounded_twice():
    z = np.zeros((1, 32))
    z[0, 3] = -1.7
    z[0, 20] = 0.9
    sb = O.half_scales(z)
    c15 = float(O.codebook()[-1])
    for h, a in ((0, 1.7), (1, 0.9)):
        f32 = np.float32(a / c15)
        want = O.bf16_bits_from_f32(np.array([f32]))[0]
        assert sb[0, h] == want


@pytest.mark.parametrize("kind", ["gaussian", "student_t3"])
def test_reconstruction_cosine_matches_model_card(kind):
    w = I.weights(512, 2688, kind)
    c = _cos(w, O.dequant(O.pack(w, SB), SB))
    assert 0.9965 <= c <= 0.9978, c


def test_rms_scale_reading_would_miss_the_card():
    """The discriminating alternative: an RMS scale misses ~0.997."""
    w = I.weights(256, 2688)
    z = O.rotate_blocks(w.reshape(256, -1, 32), SB)
    zz = z.reshape(256, -1, 2, 16)
    s = np.sqrt((zz ** 2).mean(-1, keepdims=True))
    s = np.repeat(s, 16, axis=-1).reshape(z.shape)
    q = O.codes_for(z, s)
    zh = s * O.codebook().astype(np.float64)[q]
    c = _cos(z, zh)
    assert c < 0.9965


def test_repack_of_dequant_is_identity():
    w = I.weights(64, 512)
    p = O.pack(w, SB)
    p2 = O.pack(O.dequant(p, SB).astype(np.float32), SB)
    assert np.array_equal(p, p2)


def test_byte_layout():
    w = I.weights(3, 96)
    p = O.pack(w, SB)
    assert p.shape == (3, 3, 20) and p.dtype == np.uint8
    z = O.rotate_blocks(w.reshape(3, 3, 32), SB)
    sb = O.half_scales(z)
    q = O.codes_for(z, np.repeat(O.f64_from_bf16_bits(sb), 16, axis=-1))
    assert np.array_equal(p[..., :16] & 0xF, q[..., 0::2])
    assert np.array_equal(p[..., :16] >> 4, q[..., 1::2])
    assert np.array_equal(p[..., 16].astype(np.uint16) | (p[..., 17].astype(np.uint16) << 8),
                          sb[..., 0])


def test_bits_per_weight_and_checkpoint_size():
    n, k = 8192, 2688
    assert O.packed_size(n, k) * 8 / (n * k) == 5.0        # "~5 bits/weight"
    params = 118e9 / 2                                      # BF16 checkpoint size
    tq4_bytes = params * 5 / 8
    assert 36e9 < tq4_bytes < 38e9                          # "~38 GB" incl. BF16 rest
    assert 55e9 < params * 1.0 <= 63e9                      # fp8 cache "~63 GB"


def test_nonfinite_input_follows_ieee_rule():
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, 2] = np.nan
    p = O.pack(w, SB)          # must not raise; the NaN reaches every z, so S is NaN
    _, s = O.unpack(p)
    assert (s[0, 0, 0] & 0x7F80) == 0x7F80
