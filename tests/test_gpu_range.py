"""GPU parity at the edges of the fp16 operand range.

The products multiply fp16 operands (fp32 accumulation).  The library shifts
the weight operand, the M <= 16 rotation and the MoE hidden rows by exact
powers of two so that weights far smaller than the configurations' N(0, 0.02^2),
activations far larger than N(0, 1) and large hidden values stay inside fp16's
normal range (the domain is stated in include/tq4.h).  Every case here is
checked against the fp64 oracle at the usual bar: relative Frobenius error
<= 2e-3 and max |err| <= 1e-2 * rms(y_ref).  Each case goes through every
kernel that serves its shape: the M <= 16 LDS-direct and register-load
kernels, the small-M split-K kernel and the 128x256 and 256x256 tile kernels.
"""

import numpy as np
import pytest

import oracle as O
from block_diffusion_lm_tq4_amd import inputs as I

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SB = I.sign_bits()
REL_F = 2e-3
MAX_REL_RMS = 1e-2


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_lm_tq4_amd import ops  # noqa: F401  (loads libtq4.so)
    return torch.device("cuda:0")


def _ops():
    from block_diffusion_lm_tq4_amd import ops
    return ops


def _bf16(x_bits, dev):
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(dev).view(torch.bfloat16)


def _check_close(y, ref, what):
    y = np.asarray(y, dtype=np.float64)
    assert np.isfinite(y).all(), (what, "non-finite output")
    err = y - ref
    relf = np.linalg.norm(err) / np.linalg.norm(ref)
    rms = np.sqrt(np.mean(ref * ref))
    mx = np.max(np.abs(err))
    print(f"{what}: relF={relf:.3e} max/rms={mx / rms:.3e}")
    assert relf <= REL_F, (what, relf)
    assert mx <= MAX_REL_RMS * rms, (what, mx, rms)


# one shape per kernel path: (m, k, n)
PATHS = [
    (16, 2688, 1024),    # M <= 16, LDS-direct streaming kernel
    (5, 96, 40),         # M <= 16, register-load kernel (K not a multiple of 128)
    (16, 4096, 64),      # M <= 16, register-load kernel (K above the streaming limit)
    (17, 2688, 300),     # small M, split-K partials
    (300, 512, 520),     # 128 x 256 tiles
    (257, 128, 32768),   # 256 x 256 tiles (sampled rows)
]


def _run_linear(dev, x_bits, w, sb=SB, rows=None):
    p_gpu = _ops().pack(torch.from_numpy(w).to(dev), sb)
    y = _ops().linear(_bf16(x_bits, dev), p_gpu, sb)
    torch.cuda.synchronize()
    p_ref = O.pack(w, sb)
    assert np.array_equal(p_gpu.cpu().numpy(), p_ref)
    y = y.cpu().numpy()
    if rows is not None:
        return y[rows], O.linear(x_bits[rows], p_ref, sb)
    return y, O.linear(x_bits, p_ref, sb)


def _rows(m):
    return None if m <= 64 else np.unique(np.r_[np.arange(0, m, 29), m - 1])


@pytest.mark.parametrize("rms", [1e-4, 1e-5])
@pytest.mark.parametrize("m,k,n", PATHS)
def test_small_weights(dev, m, k, n, rms):
    # half-block scales near 1e-5 .. 1e-4: without the weight shift their
    # products with the smallest levels are fp16 subnormals
    w = I.weights(n, k, seed=m + n, scale=rms)
    x = I.activations_bf16(m, k, seed=3)
    y, ref = _run_linear(dev, x, w, rows=_rows(m))
    _check_close(y, ref, f"weights rms {rms:g} {m}x{k}x{n}")


def _coherent_block(sb, value):
    """A 32-block whose sign pattern matches the rotation signs: its rotated
    element 0 is sum(|x|) / sqrt(32), the largest any block of that
    magnitude reaches."""
    s = O.signs_from_bits(sb)
    return (value * s).astype(np.float32)


@pytest.mark.parametrize("m,k,n", PATHS)
def test_large_activations(dev, m, k, n):
    # x ~ N(0, 1000^2), plus one block per row of coherent |x| = 3072 (exact in
    # bf16): its sum of 32 aligned terms is 98304, beyond fp16's 65504
    rng = np.random.default_rng(m * 13 + k)
    x = (1000.0 * rng.standard_normal((m, k))).astype(np.float32)
    for r in range(m):
        b = (r * 7) % (k // 32)
        x[r, 32 * b: 32 * b + 32] = _coherent_block(SB, 3072.0)
    x_bits = O.bf16_bits_from_f32(x)
    w = I.weights(n, k, seed=n)
    y, ref = _run_linear(dev, x_bits, w, rows=_rows(m))
    _check_close(y, ref, f"x x1e3 + coherent block {m}x{k}x{n}")


@pytest.mark.parametrize("m", [16, 17])
def test_coherent_block_alone(dev, m):
    # every row holds only coherent blocks: the rotated activations are
    # 98304/sqrt(32) at one element per block and 0 elsewhere
    k, n = 256, 96
    x = np.tile(_coherent_block(SB, 3072.0), (m, k // 32))
    x *= np.where(np.arange(m) % 2 == 0, 1.0, -1.0)[:, None].astype(np.float32)
    x_bits = O.bf16_bits_from_f32(x)
    y, ref = _run_linear(dev, x_bits, I.weights(n, k, seed=4))
    _check_close(y, ref, f"coherent rows m={m}")


def _moe_case(dev, x, w1, w2, ids, g, sb, what):
    e = w1.shape[0]
    p1 = np.stack([O.pack(w1[i], sb) for i in range(e)])
    p2 = np.stack([O.pack(w2[i], sb) for i in range(e)])
    x_bits = O.bf16_bits_from_f32(x)
    out = _ops().moe_grouped(_bf16(x_bits, dev), torch.from_numpy(ids).to(dev),
                             torch.from_numpy(g).to(dev), torch.from_numpy(p1).to(dev),
                             torch.from_numpy(p2).to(dev), sb).cpu().numpy()
    ref = O.moe(x_bits, ids, g, list(p1), list(p2), sb)
    # the up products of the case, from the oracle's decoded experts
    xf = O.f64_from_bf16_bits(x_bits)
    u = np.concatenate([xf @ O.dequant(p1[i], sb).T for i in range(e)], axis=1)
    _check_close(out, ref, what)
    return u


@pytest.mark.parametrize("sb", [0, SB])
def test_moe_large_hidden_values(dev, sb):
    # expert 0's first 32 hidden units see u ~ 150 on every token: relu(u)^2
    # ~ 22500 over a whole 32-block.  With sign_bits = 0 the rotation sums
    # that block coherently (32 * 22500 / sqrt(32) ~ 1.3e5 > 65504).
    rng = np.random.default_rng(21)
    e, k, n1, t, topk = 4, 64, 96, 24, 2
    x = np.full((t, k), 48.0, dtype=np.float32) + rng.standard_normal((t, k)).astype(np.float32)
    w1 = (0.05 * rng.standard_normal((e, n1, k))).astype(np.float32)
    w1[:, :32, :] += np.float32(0.05)
    w2 = (0.05 * rng.standard_normal((e, k, n1))).astype(np.float32)
    ids, g = I.route(rng.standard_normal((t, e)), topk)
    u = _moe_case(dev, x, w1, w2, ids, g, sb, f"moe u~150 sb={sb:#x}")
    assert np.abs(u[:, :32]).min() > 100 and np.abs(u).max() < 430, np.abs(u).max()


def test_moe_small_weights_large_x(dev):
    # weights of rms 1e-3 with activations of rms 30: the hidden rows stay in
    # range while the weight operand sits near fp16's small end unshifted
    rng = np.random.default_rng(22)
    e, k, n1, t, topk = 8, 128, 64, 40, 3
    x = (30.0 * rng.standard_normal((t, k))).astype(np.float32)
    w1 = (1e-3 * rng.standard_normal((e, n1, k))).astype(np.float32)
    w2 = (1e-3 * rng.standard_normal((e, k, n1))).astype(np.float32)
    ids, g = I.route(rng.standard_normal((t, e)), topk)
    _moe_case(dev, x, w1, w2, ids, g, SB, "moe w rms 1e-3, x rms 30")
