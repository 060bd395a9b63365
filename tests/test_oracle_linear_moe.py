"""Pins of the oracle's dequantizing linear layer, MoE layer and bucketing.

Model card, section *Running it*: each quantized Linear becomes an on-the-fly
dequantizing layer, and the MoE is run without host syncs; section *The model
underneath*: 128 experts, top-6.
"""

import math

import numpy as np

import oracle as O
from block_diffusion_lm_tq4_amd import inputs as I

SB = I.sign_bits()


def _explicit_weight(packed_row_block):
    """One block decoded by explicit loops: s_j * sum_i H[j,i] S c_q_i / sqrt(32)."""
    b = packed_row_block
    codes = []
    for i in range(16):
        codes += [int(b[i]) & 15, int(b[i]) >> 4]
    s0 = O.f64_from_bf16_bits(np.array([int(b[16]) | int(b[17]) << 8]))[0]
    s1 = O.f64_from_bf16_bits(np.array([int(b[18]) | int(b[19]) << 8]))[0]
    cb = [float(v) for v in O.codebook()]
    zh = [(s0 if i < 16 else s1) * cb[codes[i]] for i in range(32)]
    out = []
    for j in range(32):
        acc = 0.0
        for i in range(32):
            acc += (-1.0 if bin(i & j).count("1") % 2 else 1.0) * zh[i]
        sj = -1.0 if (SB >> j) & 1 else 1.0
        out.append(sj * acc / math.sqrt(32.0))
    return out


def test_linear_brute_force_elements():
    w = I.weights(40, 128)
    x = I.activations_bf16(6, 128)
    p = O.pack(w, SB)
    y = O.linear(x, p, SB)
    xf = O.f64_from_bf16_bits(x)
    rng = np.random.default_rng(0)
    for _ in range(12):
        m, n = int(rng.integers(6)), int(rng.integers(40))
        acc = 0.0
        for b in range(4):
            wb = _explicit_weight(p[n, b])
            acc += sum(xf[m, b * 32 + j] * wb[j] for j in range(32))
        assert abs(acc - y[m, n]) <= 1e-12 * max(1.0, abs(acc))


def test_identity_rows_read_back_the_weights():
    w = I.weights(64, 96)
    p = O.pack(w, SB)
    eye = np.zeros((96, 96), dtype=np.uint16)
    eye[np.arange(96), np.arange(96)] = 0x3F80      # bf16 1.0
    y = O.linear(eye, p, SB)
    assert np.array_equal(y, O.dequant(p, SB).T)


def test_linear_epilogue_brute_force_and_special_cases():
    w = I.weights(24, 64)
    x = I.activations_bf16(5, 64)
    p = O.pack(w, SB)
    rng = np.random.default_rng(3)
    bias = rng.standard_normal(24).astype(np.float32)
    res = rng.standard_normal((5, 24)).astype(np.float32)
    y = O.linear_epilogue(x, p, SB, bias, res)
    xf = O.f64_from_bf16_bits(x)
    # element by element from the decoded blocks, bias by output feature,
    # residual by (row, feature)
    for m, n in [(0, 0), (4, 23), (2, 7), (3, 16)]:
        acc = 0.0
        for b in range(2):
            wb = _explicit_weight(p[n, b])
            acc += sum(xf[m, b * 32 + j] * wb[j] for j in range(32))
        want = acc + float(bias[n]) + float(res[m, n])
        assert abs(want - y[m, n]) <= 1e-12 * max(1.0, abs(want))
    # zero activations leave exactly bias + residual; no tail leaves the product
    zero = np.zeros_like(x)
    yz = O.linear_epilogue(zero, p, SB, bias, res)
    for m in range(5):
        for n in range(24):
            assert yz[m, n] == float(bias[n]) + float(res[m, n])
    assert np.array_equal(O.linear_epilogue(x, p, SB), O.linear(x, p, SB))
    assert np.array_equal(O.linear_epilogue(zero, p, SB, bias=bias), np.tile(bias, (5, 1)))
    assert np.array_equal(O.linear_epilogue(zero, p, SB, residual=res), res.astype(np.float64))


def test_activation_rotation_identity():
    """x . W_hat^T == (R x) . Z_hat^T per block (R orthogonal)."""
    w = I.weights(128, 256)
    x = I.activations_bf16(16, 256)
    p = O.pack(w, SB)
    y = O.linear(x, p, SB)
    xt = O.rotate_blocks(O.f64_from_bf16_bits(x).reshape(16, -1, 32), SB).reshape(16, -1)
    y2 = xt @ O.dequant_rotated(p).T
    assert np.max(np.abs(y - y2)) <= 1e-12 * np.max(np.abs(y))


# ---------------------------------------------------------------------------- MoE

def _small_moe(t=7, e=8, k=64, n1=96, topk=3, seed=0):
    rng = np.random.default_rng(seed)
    w1 = [O.pack((0.05 * rng.standard_normal((n1, k))).astype(np.float32), SB) for _ in range(e)]
    w2 = [O.pack((0.05 * rng.standard_normal((k, n1))).astype(np.float32), SB) for _ in range(e)]
    x = I.activations_bf16(t, k, seed=seed + 10)
    ids, g = I.route(rng.standard_normal((t, e)), topk)
    return x, ids, g, w1, w2


def test_moe_brute_force_per_pair():
    x, ids, g, w1, w2 = _small_moe()
    out = O.moe(x, ids, g, w1, w2, SB)
    xf = O.f64_from_bf16_bits(x)
    for t in range(x.shape[0]):
        acc = np.zeros(x.shape[1])
        for j in range(ids.shape[1]):
            e = ids[t, j]
            u = O.dequant(w1[e], SB) @ xf[t]
            h = np.where(u > 0, u * u, 0.0)
            acc += float(g[t, j]) * (O.dequant(w2[e], SB) @ h)
        assert np.max(np.abs(acc - out[t])) <= 1e-12 * max(1.0, np.max(np.abs(acc)))


def test_moe_special_cases():
    x, ids, g, w1, w2 = _small_moe()
    xf = O.f64_from_bf16_bits(x)
    # topk = 1, gate 1, every token to expert 3: a dense two-layer MLP
    ids1 = np.full((x.shape[0], 1), 3, dtype=np.int32)
    g1 = np.ones((x.shape[0], 1), dtype=np.float32)
    out = O.moe(x, ids1, g1, w1, w2, SB)
    h = np.maximum(xf @ O.dequant(w1[3], SB).T, 0) ** 2
    assert np.allclose(out, h @ O.dequant(w2[3], SB).T, rtol=1e-12, atol=1e-14)
    # zero gates -> zero output
    assert not O.moe(x, ids, np.zeros_like(g), w1, w2, SB).any()
    # token permutation permutes the output
    perm = np.random.default_rng(1).permutation(x.shape[0])
    a = O.moe(x, ids, g, w1, w2, SB)[perm]
    b = O.moe(x[perm], ids[perm], g[perm], w1, w2, SB)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-15)
    # ids outside [0, E) contribute nothing
    bad = ids.copy()
    bad[:, 0] = -1
    g2 = g.copy()
    g2[:, 0] = 0
    assert np.allclose(O.moe(x, bad, g, w1, w2, SB), O.moe(x, ids, g2, w1, w2, SB),
                       rtol=1e-13, atol=1e-15)
    # a token that lists one expert in two slots gets both terms: the same as
    # one slot whose gate is the sum of the two
    dup = np.stack([ids[:, 0], ids[:, 0]], axis=1)
    gd = g[:, :2].astype(np.float64)
    one = O.moe(x, ids[:, :1], (gd[:, 0] + gd[:, 1])[:, None], w1, w2, SB)
    assert np.allclose(O.moe(x, dup, gd, w1, w2, SB), one, rtol=1e-13, atol=1e-15)


def test_bucketing_invariants_and_brute_force():
    rng = np.random.default_rng(4)
    for t, e, k in ((16, 128, 6), (300, 128, 6), (50, 8, 3)):
        ids = rng.integers(-1, e + 1, size=(t, k)).astype(np.int32)
        counts, offsets, perm, inv = O.bucket_pairs(ids, e)
        flat = ids.reshape(-1)
        valid = (flat >= 0) & (flat < e)
        assert counts.sum() == valid.sum()
        assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
        # brute force: walk experts in order, pairs in order
        want = [p for ex in range(e) for p in range(flat.size) if flat[p] == ex]
        assert perm.tolist() == want
        assert np.all(inv[~valid] == -1)
        assert np.array_equal(inv[perm], np.arange(perm.size))


def test_router_top6_is_softmax_of_largest():
    lg = I.router_logits(32, 128, "uniform")
    ids, g = I.route(lg, 6)
    p = np.exp(lg) / np.exp(lg).sum(1, keepdims=True)
    for t in range(32):
        assert set(ids[t]) == set(np.argsort(-lg[t])[:6])
        assert np.allclose(g[t], p[t, ids[t]], rtol=1e-6)
    lz = I.router_logits(20000, 128, "zipf")
    first = np.argmax(lz, axis=1)
    freq = np.bincount(first, minlength=128) / first.size
    pz = np.arange(1, 129, dtype=np.float64) ** -1.1
    pz /= pz.sum()
    assert abs(freq[0] - pz[0]) < 0.01 and abs(freq[1] - pz[1]) < 0.01


def test_oracle_router_closed_form_and_ties():
    # logits ln(1..8): softmax probabilities are exactly (1..8)/36
    lg = np.log(np.arange(1, 9, dtype=np.float64))[None, :]
    ids, g = O.router(lg, 3)
    assert ids.tolist() == [[7, 6, 5]]
    assert np.allclose(g, [[8 / 36, 7 / 36, 6 / 36]], rtol=1e-14)
    # all logits equal: the lowest ids win, every gate is 1/E
    ids, g = O.router(np.full((2, 16), 0.25), 4)
    assert ids.tolist() == [[0, 1, 2, 3]] * 2
    assert np.allclose(g, 1 / 16, rtol=1e-14)
    # partial ties: among equal logits the lower id comes first
    lt = np.array([[1.0, 3.0, 2.0, 3.0, 2.0, -1.0]])
    ids, _ = O.router(lt, 5)
    assert ids.tolist() == [[1, 3, 2, 4, 0]]
    # a constant shift of the logits changes nothing
    r = np.random.default_rng(7).standard_normal((5, 32))
    a = O.router(r, 6)
    b = O.router(r + 123.0, 6)
    assert np.array_equal(a[0], b[0]) and np.allclose(a[1], b[1], rtol=1e-12)


def test_oracle_router_brute_force_small():
    # every permutation of 5 distinct logits: the ids are the argsort, the
    # gates the softmax of the picked ones
    import itertools
    base = np.array([-1.5, -0.25, 0.0, 0.75, 2.0])
    for perm in itertools.permutations(range(5)):
        lg = base[list(perm)][None, :]
        ids, g = O.router(lg, 3)
        order = sorted(range(5), key=lambda c: (-lg[0, c], c))[:3]
        assert ids[0].tolist() == order
        p = np.exp(lg[0]) / np.exp(lg[0]).sum()
        assert np.allclose(g[0], p[order], rtol=1e-13)
