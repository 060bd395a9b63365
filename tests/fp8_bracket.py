"""The output bracket of the MoE layer on fp8 expert caches (shared by the
GPU parity test and its CPU self-check).

An output element depends on integer decisions (block exponents, e4m3 codes)
taken on values that the block-scaled MFMA computes inexactly, so parity is
an interval per element:

* the up product u is exact in the oracle; the device's fp32 u' lies within
  the instruction's bound (every product of a 32-block within 2^-13 of the
  block's largest product, fp32 sums; checked by tests/test_gpu_fp8_window.py),
  so relu(u')^2, squared in fp32, lies in [h_lo, h_hi];
* every block exponent and code the device may choose for hidden values in
  those intervals is enumerated (rounding is monotone), giving [d_min, d_max]
  per hidden element;
* the down product carries that interval (midpoint and radius through |W2|)
  plus its own bound, and the gated sum in slot order adds fp32 rounding.
"""

import numpy as np

import oracle as O


def kp_of(k):
    return (k + 127) // 128 * 128


def mfma_bound(ad, bd, kp):
    """Bound on |device - exact| for ad . bd^T on the block-scaled fp8 MFMA."""
    k = ad.shape[1]
    aa = np.max(np.abs(ad).reshape(ad.shape[0], k // 32, 32), axis=-1)
    bb = np.max(np.abs(bd).reshape(bd.shape[0], k // 32, 32), axis=-1)
    return (31 * 2.0 ** -13 * (aa @ bb.T)
            + (2 * (kp // 128) + 8) * 2.0 ** -24 * (np.abs(ad) @ np.abs(bd).T))


def quantized_range(h_lo, h_hi):
    """[d_min, d_max] of the MXFP8 values the device may store for hidden
    values in [h_lo, h_hi] (per element, rows x n1)."""
    rows, n1 = h_lo.shape
    blo = h_lo.reshape(rows, n1 // 32, 32)
    bhi = h_hi.reshape(rows, n1 // 32, 32)
    e_lo = O.e8m0_exponent(blo.max(-1))
    e_hi = O.e8m0_exponent(bhi.max(-1))
    assert np.all(e_hi - e_lo <= 1), "error bound too wide to enumerate exponents"
    vals = O.e4m3_values()
    d_min = np.full(blo.shape, np.inf)
    d_max = np.full(blo.shape, -np.inf)
    for c in (0, 1):
        e = (e_lo + c)[..., None]
        ok = np.broadcast_to(e <= e_hi[..., None], blo.shape)
        cap = np.ldexp(448.0, e)
        for src, dst, pick in ((blo, d_min, np.minimum), (bhi, d_max, np.maximum)):
            scaled = np.where(ok, np.ldexp(np.minimum(src, cap), -e), 0.0)
            q = np.ldexp(vals[O.e4m3_round(scaled)], e)
            dst[...] = np.where(ok, pick(dst, q), dst)
    return d_min.reshape(rows, n1), d_max.reshape(rows, n1)


def bracket(x, ids, g, c1, c2, tokens):
    """(centre, radius) of the interval every output element of the tokens
    must lie in."""
    xd = O.mx_dequant(*O.act_mxfp8(x))[tokens]
    sel = ids[tokens]
    gsel = g[tokens].astype(np.float64)
    topk = ids.shape[1]
    k = x.shape[1]
    centre = np.zeros((len(tokens), k))
    radius = np.zeros((len(tokens), k))
    for e in np.unique(sel):
        if e < 0 or e >= len(c1):
            continue
        rows, js = np.nonzero(sel == e)
        w1 = O.mx_dequant(*c1[int(e)])
        w2 = O.mx_dequant(*c2[int(e)])
        a = xd[rows]
        u = a @ w1.T
        b1 = mfma_bound(a, w1, kp_of(k)) * (1 + 1e-9) + 1e-30
        h_lo = np.maximum(u - b1, 0.0) ** 2 * (1 - 2.0 ** -22)
        h_hi = np.maximum(u + b1, 0.0) ** 2 * (1 + 2.0 ** -22) + 2.0 ** -140
        d_min, d_max = quantized_range(h_lo, h_hi)
        mid, rad = (d_min + d_max) / 2, (d_max - d_min) / 2
        mag = np.maximum(np.abs(d_min), np.abs(d_max))
        o_c = mid @ w2.T
        o_r = rad @ np.abs(w2).T + mfma_bound(mag, w2, kp_of(w2.shape[1])) * (1 + 1e-9)
        gj = gsel[rows, js][:, None]
        np.add.at(centre, rows, gj * o_c)
        np.add.at(radius, rows, np.abs(gj) * (o_r + (topk + 1) * 2.0 ** -24 * (np.abs(o_c) + o_r)))
    return centre, radius


def check_bracket(out, x, ids, g, c1, c2, tokens, what):
    """Every out[tokens] element lies in the interval the oracle derives, and
    the relative Frobenius distance to the oracle's own result is <= 2e-2."""
    centre, radius = bracket(x, ids, g, c1, c2, tokens)
    y = np.asarray(out, np.float64)[tokens]
    err = np.abs(y - centre)
    ratio = np.max(err / np.maximum(radius, 1e-300))
    ref = O.moe_fp8(x, ids, g, c1, c2, tokens=tokens)
    relf = np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300)
    print(f"{what}: max err / bracket = {ratio:.3e}, relF to the oracle {relf:.2e}")
    assert np.all(err <= radius + 1e-30), what
    assert relf <= 2e-2, (what, relf)
