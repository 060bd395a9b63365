"""CPU self-check of the fp8 MoE output bracket (tests/fp8_bracket.py), before
it is trusted to judge the device: it must accept every result the modelled
device arithmetic can produce and reject results with a plausible mistake.

The modelled device perturbs each up product by up to 0.9 of the MFMA bound,
squares relu(u) in fp32, quantizes those hidden values exactly as the layer
does, perturbs each down product by up to 0.9 of its bound, and sums the gated
slots in fp32.  The mistakes: ReLU dropped (h = u^2), one slot of one token
dropped, the hidden rows not quantized, and the gates renormalized.
"""

import numpy as np
import pytest

import oracle as O
from fp8_bracket import bracket, kp_of, mfma_bound

SB = 0x09F324CE


@pytest.fixture(scope="module")
def case():
    rng = np.random.default_rng(5)
    n_exp, n1, k, t, topk = 4, 64, 96, 10, 2
    c1 = [O.fp8_cache(O.pack((0.05 * rng.standard_normal((n1, k))).astype(np.float32), SB), SB)
          for _ in range(n_exp)]
    c2 = [O.fp8_cache(O.pack((0.05 * rng.standard_normal((k, n1))).astype(np.float32), SB), SB)
          for _ in range(n_exp)]
    x = O.bf16_bits_from_f32((2.0 * rng.standard_normal((t, k))).astype(np.float32))
    ids = np.stack([rng.permutation(n_exp)[:topk] for _ in range(t)]).astype(np.int32)
    g = rng.random((t, topk)).astype(np.float32)
    tokens = np.arange(t)
    centre, radius = bracket(x, ids, g, c1, c2, tokens)
    return dict(x=x, ids=ids, g=g, c1=c1, c2=c2, tokens=tokens, centre=centre, radius=radius)


def _modelled_device(c, rng, relu=True, drop=None, quantize=True, renorm=False):
    xd = O.mx_dequant(*O.act_mxfp8(c["x"]))
    ids, g = c["ids"], c["g"].astype(np.float64)
    if renorm:
        g = g / g.sum(axis=1, keepdims=True)
    out = np.zeros_like(xd, dtype=np.float32)
    for t in range(ids.shape[0]):
        for j in range(ids.shape[1]):
            if drop == (t, j):
                continue
            e = ids[t, j]
            w1 = O.mx_dequant(*c["c1"][e])
            w2 = O.mx_dequant(*c["c2"][e])
            a = xd[t:t + 1]
            u = a @ w1.T
            b1 = mfma_bound(a, w1, kp_of(a.shape[1]))
            u = (u + 0.9 * b1 * rng.uniform(-1, 1, u.shape)).astype(np.float32)
            h = (np.maximum(u, 0) if relu else u) ** 2
            h = h.astype(np.float32).astype(np.float64)
            hq = O.mx_dequant(*O.mx_quantize(h)) if quantize else h
            o = hq @ w2.T
            b2 = mfma_bound(np.abs(hq), w2, kp_of(hq.shape[1]))
            o = (o + 0.9 * b2 * rng.uniform(-1, 1, o.shape)).astype(np.float32)
            out[t] = np.float32(out[t] + np.float32(g[t, j]) * o[0])
    return out.astype(np.float64)


def _inside(c, y):
    return np.abs(y - c["centre"]) <= c["radius"] + 1e-30


def test_oracle_result_is_inside(case):
    ref = O.moe_fp8(case["x"], case["ids"], case["g"], case["c1"], case["c2"])
    assert _inside(case, ref).all()


@pytest.mark.parametrize("seed", range(4))
def test_modelled_device_results_are_inside(case, seed):
    y = _modelled_device(case, np.random.default_rng(seed))
    assert _inside(case, y).all()


@pytest.mark.parametrize("mistake", [
    dict(relu=False),
    dict(drop=(3, 1)),
    dict(quantize=False),
    dict(renorm=True),
])
def test_mistakes_are_rejected(case, mistake):
    y = _modelled_device(case, np.random.default_rng(9), **mistake)
    assert not _inside(case, y).all(), mistake
