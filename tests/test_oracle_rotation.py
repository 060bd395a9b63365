"""Pins of the oracle's randomized Walsh-Hadamard rotation.

Model card, section *What "Config-I" means*: a Walsh-Hadamard rotation per
32-element block.  Checked against SciPy's Sylvester Hadamard matrix and the
defining invariants of an orthogonal transform.
"""

import numpy as np
import scipy.linalg
import torch

import oracle as O


def test_h32_is_scipy_sylvester_hadamard():
    assert np.array_equal(O.hadamard32(), scipy.linalg.hadamard(32).astype(np.float64))


def test_h32_squared_is_32_identity():
    h = O.hadamard32()
    assert np.array_equal(h @ h, 32 * np.eye(32))
    assert np.array_equal(h, h.T)


def test_sign_bits_mapping():
    for i in range(32):
        s = O.signs_from_bits(1 << i)
        assert s[i] == -1 and np.sum(s == -1) == 1
    assert np.all(O.signs_from_bits(0) == 1)
    assert np.all(O.signs_from_bits(0xFFFFFFFF) == -1)


def test_rotation_is_orthogonal():
    for sb in (0, 0x09F324CE, 0xFFFFFFFF, 0x80000001):
        r = O.rotation_matrix(sb)
        assert np.max(np.abs(r @ r.T - np.eye(32))) < 1e-12
        x = np.random.default_rng(sb & 0xFFFF).standard_normal((50, 32))
        z = O.rotate_blocks(x, sb)
        assert np.allclose(np.linalg.norm(z, axis=1), np.linalg.norm(x, axis=1),
                           rtol=1e-13, atol=0)


def test_rotate_blocks_equals_explicit_matrix():
    sb = 0x09F324CE
    x = np.random.default_rng(5).standard_normal((7, 3, 32)).astype(np.float32)
    z = O.rotate_blocks(x, sb)
    r = O.rotation_matrix(sb)
    assert np.max(np.abs(z - x.astype(np.float64) @ r.T)) < 1e-14


def test_rotation_against_torch_fwht_definition():
    """The same transform via a different route: torch kron-built Hadamard."""
    h2 = torch.tensor([[1.0, 1.0], [1.0, -1.0]], dtype=torch.float64)
    h = h2
    for _ in range(4):
        h = torch.kron(h, h2)
    sb = 0x12345678
    s = torch.tensor([-1.0 if (sb >> i) & 1 else 1.0 for i in range(32)],
                     dtype=torch.float64)
    x = torch.randn(11, 32, dtype=torch.float64, generator=torch.Generator().manual_seed(3))
    ref = ((x * s) @ h.T) / (32 ** 0.5)
    got = O.rotate_blocks(x.numpy(), sb)
    assert np.max(np.abs(got - ref.numpy())) < 1e-14


def test_dequant_inverts_rotation():
    sb = 0x09F324CE
    z = np.random.default_rng(9).standard_normal((4, 32))
    w = (z @ O.hadamard32().T) * O.RS32 * O.signs_from_bits(sb)
    assert np.max(np.abs(O.rotate_blocks(w, sb) - z)) < 1e-14


def test_rs32_is_correctly_rounded():
    from fractions import Fraction
    v = Fraction(O.RS32)
    # (1/sqrt(32))^2 = 1/32: the fp64 value must be the nearest to 1/sqrt(32)
    ulp = Fraction(2) ** -55
    lo, hi = v - ulp, v + ulp
    assert lo * lo < Fraction(1, 32) < hi * hi
    assert abs(v * v - Fraction(1, 32)) < abs((v + ulp) ** 2 - Fraction(1, 32))
    assert abs(v * v - Fraction(1, 32)) < abs((v - ulp) ** 2 - Fraction(1, 32))
