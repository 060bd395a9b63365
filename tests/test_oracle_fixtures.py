"""Reference values recorded before the oracle was written.

When the readings of the format were first fixed (block axis, rotation,
codebook, scale rule, ties, byte layout; model card, section What "Config-I"
means), three values were computed from those readings by a separate
throwaway computation: the sign bits drawn from seed 1, the fp32 bit
patterns of the 16-level Lloyd-Max codebook, and the 20 packed bytes of the
first block of the 512x256 layer.  They are not on the pages; they pin the
oracle to an earlier, independent evaluation of the same readings, so that a
later change to the oracle's generator, codebook iteration, rounding or
nibble order shows up here.
"""

import numpy as np

import oracle as O
from block_diffusion_lm_tq4_amd import inputs as I

SIGN_BITS_SEED1 = 0x09F324CE
POSITIVE_LEVEL_BITS = [0x3E0379FD, 0x3EC6AE44, 0x3F28215E, 0x3F713D39,
                       0x3FA0CC2F, 0x3FCF1C25, 0x40046AC7, 0x402EE2BF]
FIRST_BLOCK_512X256 = "20858fc3edac296c613af8a5169f54763f3c3f3c"


def test_sign_bits_from_seed_1():
    assert I.sign_bits() == SIGN_BITS_SEED1


def test_codebook_fp32_bits():
    bits = O.codebook().astype(np.float32).view(np.uint32)
    want = [b | 0x80000000 for b in reversed(POSITIVE_LEVEL_BITS)] + POSITIVE_LEVEL_BITS
    assert [int(b) for b in bits] == want


def test_first_block_of_the_512x256_layer():
    w = I.weights(512, 256)
    p = O.pack(w, SIGN_BITS_SEED1)
    assert p[0, 0].tobytes().hex() == FIRST_BLOCK_512X256
