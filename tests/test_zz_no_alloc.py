"""tq4_linear_noalloc (the library's static scratch instead of a workspace)
against tq4_linear, through the C ABI: equal bit for bit on consecutive
calls, the second smaller than the first, and within the usual bar of the
fp64 oracle."""

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


def _case(dev, m, k, n, seed):
    from block_diffusion_lm_tq4_amd import ops
    w = I.weights(n, k, seed=seed)
    x_bits = I.activations_bf16(m, k, seed=seed + 1)
    x = torch.from_numpy(x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    p = ops.pack(torch.from_numpy(w).to(dev), SB)
    return w, x_bits, x, p


@pytest.mark.parametrize("shapes", [
    # rotated activations of 11 MB (256 x 256 tiles), then a split-K call
    # (its partial sums in the scratch too)
    [(2048, 2688, 8192), (40, 512, 256)],
    # split-K first, then the same large product shape with fewer rows
    [(33, 2688, 100), (20, 2688, 100)],
    # a call without scratch (one M <= 16 kernel) between two that use it
    [(300, 1024, 520), (16, 2688, 512), (100, 256, 64)],
])
def test_noalloc_equals_linear(dev, shapes):
    from block_diffusion_lm_tq4_amd import ops
    for i, (m, k, n) in enumerate(shapes):
        w, x_bits, x, p = _case(dev, m, k, n, seed=10 * i + m)
        # poison the output so that a skipped store cannot pass
        y = torch.full((m, n), float("nan"), device=dev)
        ops.linear_noalloc(x, p, SB, out=y)
        want = ops.linear(x, p, SB)
        torch.cuda.synchronize()
        assert torch.equal(y, want), (m, k, n)
        rows = np.unique(np.r_[np.arange(0, m, max(1, m // 12)), m - 1])
        ref = O.linear(x_bits[rows], O.pack(w, SB), SB)
        got = y.cpu().numpy()[rows].astype(np.float64)
        err = got - ref
        rms = np.sqrt(np.mean(ref * ref))
        assert np.linalg.norm(err) / np.linalg.norm(ref) <= 2e-3
        assert np.max(np.abs(err)) <= 1e-2 * rms


def test_noalloc_rejects_sizes_beyond_the_scratch(dev):
    from block_diffusion_lm_tq4_amd import ops
    from block_diffusion_lm_tq4_amd._lib import TQ4Error
    # 8192 x 4096 rotated activations need 64 MiB
    x = torch.zeros((8192, 4096), dtype=torch.bfloat16, device=dev)
    p = torch.zeros((64, 128, 20), dtype=torch.uint8, device=dev)
    with pytest.raises(TQ4Error, match="TOO_LARGE"):
        ops.linear_noalloc(x, p, SB)
