"""GPU parity of the MoE layer on fp8 expert caches (tq4_moe_grouped_fp8)
against the oracle, through the C ABI.

The layer quantizes its hidden activations, so an output element depends on
integer decisions (block exponents, e4m3 codes) taken on values that the
block-scaled MFMA computes inexactly.  The check brackets every output
element instead of comparing it with one value:

* the up product u is computed exactly by the oracle; the device's fp32 u' is
  within the MFMA bound measured for this instruction (products kept to a
  13-bit window below the largest one of each 32-block, fp32 sums; stated in
  test_gpu_fp8), so relu(u')^2, squared in fp32, lies in [h_lo, h_hi];
* every block exponent and code the device may choose for values in those
  intervals is enumerated (rounding is monotone), giving an interval
  [d_min, d_max] of quantized hidden values per element;
* the down product carries that interval (midpoint and radius through |W2|)
  plus its own MFMA bound, and the gated sum in slot order adds fp32 rounding.

Away from rounding boundaries the interval is as tight as the fp8 product
bound.  The relative Frobenius distance to the oracle's own result (which
quantizes the exact h) is printed and held to 2e-2.
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle as O
from block_diffusion_lm_tq4_amd import inputs as I
from fp8_bracket import check_bracket as _check_bracket

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


class _Experts:
    """A stack of experts: device fp8 caches, oracle caches on demand."""

    def __init__(self, dev, n_exp, n1, k, make):
        self.n_exp, self.n1, self.k, self.make = n_exp, n1, k, make
        p1 = torch.empty((n_exp, n1, k // 32, 20), dtype=torch.uint8, device=dev)
        p2 = torch.empty((n_exp, k, n1 // 32, 20), dtype=torch.uint8, device=dev)
        with ThreadPoolExecutor(8) as ex:
            for e, a, b in ex.map(lambda e: (e, make(e, 1), make(e, 2)), range(n_exp)):
                p1[e] = _ops().pack(torch.from_numpy(a).to(dev), SB)
                p2[e] = _ops().pack(torch.from_numpy(b).to(dev), SB)
        self.c1 = _ops().fp8_cache_experts(p1, SB)
        self.c2 = _ops().fp8_cache_experts(p2, SB)
        del p1, p2
        self._ref = {}

    def oracle(self, experts):
        todo = [int(e) for e in experts if 0 <= e < self.n_exp and int(e) not in self._ref]

        def work(e):
            return e, (O.fp8_cache(O.pack(self.make(e, 1), SB), SB),
                       O.fp8_cache(O.pack(self.make(e, 2), SB), SB))

        with ThreadPoolExecutor(8) as ex:
            for e, caches in ex.map(work, todo):
                self._ref[e] = caches
        c1 = {e: v[0] for e, v in self._ref.items()}
        c2 = {e: v[1] for e, v in self._ref.items()}
        return _Lookup(c1, self.n_exp), _Lookup(c2, self.n_exp)


class _Lookup:
    def __init__(self, d, n):
        self.d, self.n = d, n

    def __getitem__(self, e):
        return self.d[e]

    def __len__(self):
        return self.n


def _small_experts(dev, n_exp, n1, k, seed):
    def make(e, which):
        shape = (n1, k) if which == 1 else (k, n1)
        return I.weights(*shape, seed=[seed, e, which])
    return _Experts(dev, n_exp, n1, k, make)


def _run(dev, ex, x, ids, g):
    return _ops().moe_grouped_fp8(_bf16(x, dev), torch.from_numpy(ids).to(dev),
                                  torch.from_numpy(g).to(dev), ex.c1, ex.c2, ex.n_exp,
                                  ex.n1).cpu().numpy()


@pytest.mark.parametrize("t,n_exp,topk,n1,k", [
    (40, 16, 2, 224, 352),    # 16-row tiles; ragged hidden and model widths
    (300, 4, 2, 160, 288),    # 64-row tiles, three per expert
    (1, 3, 1, 32, 32),        # one pair, one 32-block each way
    (70, 5, 3, 128, 640),     # 64-row tiles, a full and a partial one per expert
    (2100, 8, 4, 64, 96),     # 8400 pairs: the bucketing in chunks
])
def test_moe_fp8_small_matches_oracle(dev, t, n_exp, topk, n1, k):
    ex = _small_experts(dev, n_exp, n1, k, seed=t + n_exp)
    rng = np.random.default_rng(t)
    ids = np.stack([rng.permutation(n_exp)[:topk] for _ in range(t)]).astype(np.int32)
    g = rng.random((t, topk)).astype(np.float32)
    x = I.activations_bf16(t, k, seed=t)
    out = _run(dev, ex, x, ids, g)
    c1, c2 = ex.oracle(range(n_exp))
    _check_bracket(out, x, ids, g, c1, c2, np.arange(t), f"fp8 moe t{t} E{n_exp} {n1}x{k}")


@pytest.mark.parametrize("t,n_exp,topk,n1,k,hot", [
    (300, 2, 1, 96, 160, 0),     # every token on expert 0: five 64-row tiles, the last partial
    (50, 64, 2, 64, 96, 5),      # slot 0 always expert 5: four 16-row tiles of one expert
])
def test_moe_fp8_one_popular_expert(dev, t, n_exp, topk, n1, k, hot):
    ex = _small_experts(dev, n_exp, n1, k, seed=hot + 11)
    rng = np.random.default_rng(hot)
    ids = np.full((t, topk), hot, np.int32)
    if topk > 1:
        others = np.array([e for e in range(n_exp) if e != hot])
        ids[:, 1:] = rng.choice(others, size=(t, topk - 1))
    g = rng.random((t, topk)).astype(np.float32)
    x = I.activations_bf16(t, k, seed=hot + 1)
    out = _run(dev, ex, x, ids, g)
    c1, c2 = ex.oracle(np.unique(ids))
    _check_bracket(out, x, ids, g, c1, c2, np.arange(t), f"fp8 moe hot expert {hot}, t{t}")


def test_moe_fp8_invalid_and_repeated_ids(dev):
    t, n_exp, topk, n1, k = 33, 6, 3, 128, 128
    ex = _small_experts(dev, n_exp, n1, k, seed=9)
    rng = np.random.default_rng(9)
    ids = rng.integers(-2, n_exp + 2, size=(t, topk)).astype(np.int32)
    ids[0] = [2, 2, 2]                 # one expert in every slot
    ids[1] = [-1, n_exp, 7]            # nothing valid: a zero row
    g = rng.random((t, topk)).astype(np.float32)
    x = I.activations_bf16(t, k, seed=4)
    out = _run(dev, ex, x, ids, g)
    assert not out[1].any()
    c1, c2 = ex.oracle(range(n_exp))
    _check_bracket(out, x, ids, g, c1, c2, np.arange(t), "fp8 moe invalid/repeated ids")


@pytest.fixture(scope="module")
def full_experts(dev):
    """The 128-expert layer's weights (same draws as the TQ4 layer's tests)."""
    return _Experts(dev, 128, 1856, 2688, lambda e, w: I.expert_weights(e, w))


@pytest.mark.parametrize("name", ["moe_t16", "moe_t1024_uniform", "moe_t1024_zipf"])
def test_moe_fp8_full_size_sampled_tokens(dev, full_experts, name):
    wl = I.WORKLOADS[name]
    ids, g = I.moe_routing(wl)
    x = I.activations_bf16(wl.t, wl.k)
    out = _run(dev, full_experts, x, ids, g)
    assert np.isfinite(out).all()
    # tokens of the hottest expert (13 64-row tiles under Zipf routing)
    # plus a spread sample
    hot = np.bincount(ids.reshape(-1), minlength=wl.n_experts).argmax()
    tok = np.unique(np.concatenate([np.nonzero((ids == hot).any(1))[0][:3],
                                    np.arange(0, wl.t, max(wl.t // 5, 1)), [wl.t - 1]]))
    c1, c2 = full_experts.oracle(np.unique(ids[tok]))
    _check_bracket(out, x, ids, g, c1, c2, tok, name + " fp8 (sampled tokens)")


def test_moe_fp8_deterministic_and_t0(dev, full_experts):
    wl = I.WORKLOADS["moe_t1024_zipf"]
    ids, g = I.moe_routing(wl)
    x = _bf16(I.activations_bf16(wl.t, wl.k), dev)
    ids_d, g_d = torch.from_numpy(ids).to(dev), torch.from_numpy(g).to(dev)
    a = _ops().moe_grouped_fp8(x, ids_d, g_d, full_experts.c1, full_experts.c2, 128, 1856).clone()
    b = _ops().moe_grouped_fp8(x, ids_d, g_d, full_experts.c1, full_experts.c2, 128, 1856)
    assert torch.equal(a, b)
    e0 = torch.empty((0, wl.k), dtype=torch.bfloat16, device=dev)
    out = _ops().moe_grouped_fp8(e0, torch.empty((0, 6), dtype=torch.int32, device=dev),
                                 torch.empty((0, 6), device=dev), full_experts.c1,
                                 full_experts.c2, 128, 1856)
    assert out.shape == (0, wl.k)
