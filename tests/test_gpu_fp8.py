"""GPU parity of the fp8 weight-cache variant against the oracle, through the C ABI.

Codes and scale bytes are compared bit for bit (both sides decide them in
fp64, or from exactly scaled fp32 values for the activations).  The product is
compared with the oracle's fp64 product of the same fp8 operands.  The
block-scaled fp8 MFMA need not sum a 32-block's products exactly: a product
at least 2^-13 of the block's largest is summed exactly and a smaller one errs
by less than 2^-13 of the largest, while block sums and the running sum are
combined in fp32; tests/test_gpu_fp8_window.py checks exactly this on the
device.  So
each element must lie within
    31 * 2^-13 * sum_b max_k|x| max_k|w|   (over the 32-blocks b, k in b)
  + (2 * steps + 8) * 2^-24 * sum_k |x_k w_k|
of the oracle (steps = 128-k steps), and the relative Frobenius error against
the oracle must stay within 2e-3.
"""

import numpy as np
import pytest
import torch

import oracle as O
from block_diffusion_lm_tq4_amd import inputs as I

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


def _bf16(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def _kp(k):
    return (k + 127) // 128 * 128


def _cache(dev, n, k, kind="gaussian", seed=0):
    w = I.weights(n, k, kind, seed=seed)
    p_ref = O.pack(w, SB)
    p_gpu = _ops().pack(torch.from_numpy(w).to(dev), SB)
    cache = _ops().fp8_cache(p_gpu, SB)
    return p_ref, cache


@pytest.mark.parametrize("n,k,kind", [
    (64, 256, "gaussian"), (40, 96, "student_t3"), (33, 160, "gaussian"),
    (8192, 2688, "gaussian"), (1024, 2688, "student_t3"),
])
def test_fp8_cache_bytes_equal_oracle(dev, n, k, kind):
    p_ref, cache = _cache(dev, n, k, kind, seed=n + k)
    codes, scales = (t.cpu().numpy() for t in _ops().fp8_cache_views(cache, n, k))
    rc, rs = O.fp8_cache(p_ref, SB)
    kb = k // 32
    assert np.array_equal(codes[:, :k], rc)
    assert np.array_equal(scales[:, :kb], rs)
    assert not codes[:, k:].any() and not scales[:, kb:].any()   # zero padding


@pytest.mark.parametrize("m,k", [(16, 2688), (5, 96), (300, 256), (1, 32)])
def test_act_mxfp8_bytes_equal_oracle(dev, m, k):
    x = I.activations_bf16(m, k, seed=m)
    codes, scales = (t.cpu().numpy() for t in _ops().act_mxfp8(_bf16(x, dev)))
    rc, rs = O.act_mxfp8(x)
    assert np.array_equal(codes[:, :k], rc)
    assert np.array_equal(scales[:, :k // 32], rs)
    assert not codes[:, k:].any() and not scales[:, k // 32:].any()


def test_act_mxfp8_special_blocks(dev):
    k = 256
    x = np.zeros((6, k), dtype=np.float32)
    x[1] = -0.0                                       # signed zeros
    x[2, :32] = 1e-30                                 # tiny block
    x[2, 32:64] = np.linspace(-3e4, 3e4, 32)          # wide block
    x[3] = 448.0 * np.arange(1, k + 1) / k            # exactly 448 at the block ends
    x[4, :32] = 2.0 ** -130                           # below the smallest scale
    x[5] = np.random.default_rng(4).standard_normal(k) * 1e3
    xb = O.bf16_bits_from_f32(x)
    codes, scales = (t.cpu().numpy() for t in _ops().act_mxfp8(_bf16(xb, dev)))
    rc, rs = O.act_mxfp8(xb)
    assert np.array_equal(codes, rc)
    assert np.array_equal(scales, rs)


def _check_fp8_product(y, x, rc, rs, what):
    xq, xs = O.act_mxfp8(x)
    xd = O.mx_dequant(xq, xs)
    wd = O.mx_dequant(rc, rs)
    ref = xd @ wd.T
    absref = np.abs(xd) @ np.abs(wd).T
    k = x.shape[1]
    ax = np.max(np.abs(xd).reshape(xd.shape[0], k // 32, 32), axis=-1)
    aw = np.max(np.abs(wd).reshape(wd.shape[0], k // 32, 32), axis=-1)
    steps = _kp(k) // 128
    bound = 31 * 2.0 ** -13 * (ax @ aw.T) + (2 * steps + 8) * 2.0 ** -24 * absref
    y = np.asarray(y, np.float64)
    err = np.abs(y - ref)
    relf = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    print(f"{what}: max err/bound = {np.max(err / np.maximum(bound, 1e-300)):.3e}, relF {relf:.2e}")
    assert np.all(err <= bound), what
    assert relf <= 2e-3, (what, relf)
    return ref


@pytest.mark.parametrize("m,k,n", [
    (16, 2688, 8192), (1, 32, 1), (5, 96, 17), (16, 160, 129), (33, 256, 100),
    # m <= 16 streaming kernel at its k limit (kp 3072) and just past it
    (16, 3072, 64), (7, 2944, 100), (16, 3200, 40), (3, 4096, 33),
    (64, 512, 300), (48, 2688, 40),
    # 256 x 128 tiles: ragged m, n and k, steps not a multiple of three
    (65, 256, 130), (300, 160, 200), (512, 2688, 1024), (257, 384, 129),
])
def test_linear_fp8_matches_oracle(dev, m, k, n):
    p_ref, cache = _cache(dev, n, k, seed=m * 3 + n)
    x = I.activations_bf16(m, k, seed=m + 1)
    y = _ops().linear_fp8(_bf16(x, dev), cache, n)
    torch.cuda.synchronize()
    rc, rs = O.fp8_cache(p_ref, SB)
    ref = _check_fp8_product(y.cpu().numpy(), x, rc, rs, f"fp8 {m}x{k}x{n}")
    # against the exact TQ4_1S layer: both operands' e4m3 rounding (2^-4 each)
    exact = O.linear(x, p_ref, SB)
    relf = np.linalg.norm(ref - exact) / np.linalg.norm(exact)
    assert relf < 0.06, relf


def test_linear_fp8_prefill_m4096_sampled_rows(dev):
    m, k, n = 4096, 2688, 8192
    p_ref, cache = _cache(dev, n, k, "student_t3", seed=11)
    x = I.activations_bf16(m, k, seed=12)
    y = _ops().linear_fp8(_bf16(x, dev), cache, n).cpu().numpy()
    rows = np.unique(np.concatenate([np.arange(0, m, 131), [m - 1]]))
    rc, rs = O.fp8_cache(p_ref, SB)
    _check_fp8_product(y[rows], x[rows], rc, rs, "fp8 4096x2688x8192 (sampled rows)")
    assert np.isfinite(y).all()


@pytest.mark.parametrize("m", [16, 300])
def test_linear_fp8_quantized_equals_linear_fp8(dev, m):
    _, cache = _cache(dev, 520, 2688, seed=7)
    x = _bf16(I.activations_bf16(m, 2688, seed=3), dev)
    codes, scales = _ops().act_mxfp8(x)
    a = _ops().linear_fp8(x, cache, 520)
    b = _ops().linear_fp8_quantized(codes, scales, 2688, cache, 520)
    assert torch.equal(a, b)


def test_linear_fp8_deterministic_and_k0(dev):
    _, cache = _cache(dev, 300, 2688, seed=5)
    for m in (16, 300):
        x = _bf16(I.activations_bf16(m, 2688), dev)
        a = _ops().linear_fp8(x, cache, 300).clone()
        b = _ops().linear_fp8(x, cache, 300).clone()
        assert torch.equal(a, b)
    x0 = torch.empty((4, 0), dtype=torch.bfloat16, device=dev)
    y = torch.full((4, 8), 7.0, device=dev)
    _ops().linear_fp8(x0, torch.zeros(16, dtype=torch.uint8, device=dev), 8, out=y)
    assert not y.any()
