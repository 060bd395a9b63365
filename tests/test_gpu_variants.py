"""The measurement variants of the linear layer (tq4_linear_variant) against
the fp64 oracle: the rotation undone on the weight tiles (M <= 16 streaming
kernel and the 256 x 256 tile kernel of large M) and the products on the VALU
(M <= 16).  Same bar as the library's own product: relative Frobenius error
<= 2e-3 and max |err| <= 1e-2 * rms(y_ref)."""

import numpy as np
import pytest

import oracle as O
from block_diffusion_lm_tq4_amd import inputs as I

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SB = I.sign_bits()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_lm_tq4_amd import ops  # noqa: F401  (loads libtq4.so)
    return torch.device("cuda:0")


def _ops():
    from block_diffusion_lm_tq4_amd import ops
    return ops


def _check(y, ref, what):
    err = np.asarray(y, np.float64) - ref
    relf = np.linalg.norm(err) / np.linalg.norm(ref)
    rms = np.sqrt(np.mean(ref * ref))
    mx = np.max(np.abs(err))
    print(f"{what}: relF={relf:.3e} max/rms={mx / rms:.3e}")
    assert np.isfinite(y).all()
    assert relf <= 2e-3, (what, relf)
    assert mx <= 1e-2 * rms, (what, mx, rms)


@pytest.mark.parametrize("variant", ["weight_rotation", "valu_product"])
@pytest.mark.parametrize("m,k,n,kind", [
    (16, 2688, 8192, "gaussian"),    # the dense denoiser projection
    (16, 2688, 1000, "student_t3"),
    (5, 256, 100, "gaussian"),       # ragged m, n
    (1, 128, 33, "gaussian"),
    (16, 2944, 64, "gaussian"),      # the streaming kernel's k limit
])
def test_small_m_variants_match_oracle(dev, variant, m, k, n, kind):
    w = I.weights(n, k, kind, seed=m + n)
    x = I.activations_bf16(m, k, seed=7)
    p = _ops().pack(torch.from_numpy(w).to(dev), SB)
    xb = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    y = _ops().linear_variant(xb, p, SB, variant)
    torch.cuda.synchronize()
    _check(y.cpu().numpy(), O.linear(x, O.pack(w, SB), SB), f"{variant} {m}x{k}x{n}")


@pytest.mark.parametrize("m,k,n,kind", [
    (257, 320, 32761, "gaussian"),   # 256 x 256 tiles, ragged m and n
    (4096, 2688, 8192, "student_t3"),  # the prefill projection (sampled rows)
])
def test_large_m_weight_rotation_matches_oracle(dev, m, k, n, kind):
    w = I.weights(n, k, kind, seed=3)
    x = I.activations_bf16(m, k, seed=8)
    p = _ops().pack(torch.from_numpy(w).to(dev), SB)
    xb = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    y = _ops().linear_variant(xb, p, SB, "weight_rotation")
    torch.cuda.synchronize()
    rows = np.unique(np.r_[np.arange(0, m, max(1, m // 40)), m - 1])
    _check(y.cpu().numpy()[rows], O.linear(x[rows], O.pack(w, SB), SB),
           f"weight_rotation {m}x{k}x{n}")


def test_default_variant_is_the_layer(dev):
    w = I.weights(300, 2688, seed=9)
    p = _ops().pack(torch.from_numpy(w).to(dev), SB)
    for m in (16, 100):
        xb = torch.from_numpy(I.activations_bf16(m, 2688).view(np.int16)).to(dev).view(torch.bfloat16)
        assert torch.equal(_ops().linear_variant(xb, p, SB, "default"), _ops().linear(xb, p, SB))


def test_uncovered_shapes_are_rejected(dev):
    from block_diffusion_lm_tq4_amd._lib import TQ4Error
    p = _ops().pack(torch.from_numpy(I.weights(64, 256)).to(dev), SB)
    x = torch.zeros((100, 256), dtype=torch.bfloat16, device=dev)
    with pytest.raises(TQ4Error, match="SHAPE"):
        _ops().linear_variant(x, p, SB, "valu_product")      # m > 16
    with pytest.raises(TQ4Error, match="SHAPE"):
        _ops().linear_variant(x, p, SB, "weight_rotation")   # too few 256 x 256 tiles
