"""fp8 weight-cache variant of the TQ4_1S linear layer, written out plainly in
NumPy fp64.

TEST INFRASTRUCTURE ONLY -- imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.  It
shares no code with the HIP library.

Source: the Nemotron-TheHobbit-30B-A3B model card, section *Help wanted*
(both renderings): decode the quantized weights once into a resident fp8 copy
(about 63 GB for both towers, still one GPU) so that no forward pass decodes.
The card names no fp8 encoding, scale granularity or activation precision.
The readings taken here:

* fp8 values are OCP e4m3 ("e4m3fn"): sign, 4 exponent bits (bias 7), 3
  mantissa bits, subnormals, no infinities, NaN only at 0x7F and 0xFF, largest
  finite magnitude 448;
* one power-of-two scale 2^e (stored as the E8M0 byte e + 127) per 32
  consecutive k of a row -- the same 32-weight blocks as TQ4_1S -- with e the
  smallest integer in [-127, 127] for which the block's largest magnitude is
  at most 448 * 2^e (e = -127 for an all-zero block);
* an element v of a block is stored as the e4m3 value nearest to v / 2^e,
  ties to the even code (the one whose mantissa's last bit is 0); the sign of
  v is kept, also for zero;
* the cached weights are the decoded TQ4_1S weights W_hat (rotation undone),
  so a forward pass needs no rotation;
* activations are quantized the same way, per row and 32-block, on every
  call (an fp8 matrix product takes both operands in fp8);
* y = sum_k xq[m, k] * 2^ex[m, b] * wq[n, k] * 2^ew[n, b], b = k / 32, in
  fp64.  About 63 GB for the 59 B weights of both towers matches one byte per
  weight plus one scale byte per 32 (1.03 bytes per weight).
* the MoE layer on fp8 expert caches (the card's 128-expert top-6 MoE,
  section The model underneath, is where most of those bytes are): both
  projections take fp8 operands, so the hidden activations
  h = relu(x W1^T)^2 are quantized the same way, per row and 32-block, before
  the down projection.
"""

from __future__ import annotations

import numpy as np

from .tq4_oracle import dequant, f64_from_bf16_bits

__all__ = [
    "E4M3_MAX",
    "MX_BLOCK",
    "e4m3_values",
    "e4m3_round",
    "e8m0_exponent",
    "mx_quantize",
    "mx_dequant",
    "fp8_cache",
    "act_mxfp8",
    "linear_fp8",
    "moe_fp8",
]

E4M3_MAX = 448.0
MX_BLOCK = 32


def e4m3_values() -> np.ndarray:
    """The 256 code values by the definition above (fp64; NaN at 0x7F, 0xFF)."""
    out = np.empty(256)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            out[c] = np.nan
        elif e == 0:
            out[c] = sign * (m / 8.0) * 2.0 ** -6          # subnormal
        else:
            out[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


def e4m3_round(v: np.ndarray) -> np.ndarray:
    """Codes of the e4m3 values nearest to v (|v| <= 448), ties to even codes."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(a > E4M3_MAX) or np.any(np.isnan(a)):
        raise ValueError("e4m3_round: |v| must be at most 448")
    pos = e4m3_values()[:0x7F]                 # codes 0x00..0x7E, ascending
    hi = np.searchsorted(pos, a, side="left")  # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - pos[lo]
    d_hi = pos[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return code | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)


def e8m0_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest e in [-127, 127] with amax <= 448 * 2^e (-127 for amax = 0).

    A first guess from log2, then exact power-of-two comparisons move each e
    up while amax > 448 * 2^e and down while amax <= 448 * 2^(e - 1)."""
    a = np.asarray(amax, dtype=np.float64)
    nz = a > 0
    with np.errstate(divide="ignore"):
        e = np.where(nz, np.floor(np.log2(np.where(nz, a, 1.0) / E4M3_MAX)), -127.0)
    e = e.astype(np.int64)
    while True:
        up = nz & (a > np.ldexp(E4M3_MAX, e))
        if not up.any():
            break
        e = e + up
    while True:
        down = nz & (e > -127) & (a <= np.ldexp(E4M3_MAX, e - 1))
        if not down.any():
            break
        e = e - down
    return np.clip(e, -127, 127)


def mx_quantize(v: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """[rows, k] fp64 (k % 32 == 0) -> (e4m3 codes [rows, k], E8M0 bytes [rows, k/32])."""
    v = np.asarray(v, dtype=np.float64)
    rows, k = v.shape
    blocks = v.reshape(rows, k // MX_BLOCK, MX_BLOCK)
    e = e8m0_exponent(np.max(np.abs(blocks), axis=-1))
    scaled = np.ldexp(blocks, -e[..., None])       # exact: a power-of-two scale
    codes = e4m3_round(scaled).reshape(rows, k)
    return codes, (e + 127).astype(np.uint8)


def mx_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Inverse of mx_quantize's storage: code value * 2^(scale byte - 127), fp64."""
    rows, k = codes.shape
    vals = e4m3_values()[codes].reshape(rows, k // MX_BLOCK, MX_BLOCK)
    e = scales.astype(np.int64) - 127
    return np.ldexp(vals, e[..., None]).reshape(rows, k)


def fp8_cache(packed: np.ndarray, sign_bits: int) -> tuple[np.ndarray, np.ndarray]:
    """The resident fp8 copy of a packed [N][K/32][20] matrix: (codes, scales)."""
    return mx_quantize(dequant(packed, sign_bits))


def act_mxfp8(x_bf16: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """bf16 activations [M, K] (bit patterns) -> (codes, scales), per call."""
    return mx_quantize(f64_from_bf16_bits(x_bf16))


def linear_fp8(x_bf16: np.ndarray, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """y = dequant(act_mxfp8(x)) . dequant(cache)^T in fp64, [M, N]."""
    xq, xs = act_mxfp8(x_bf16)
    return mx_dequant(xq, xs) @ mx_dequant(codes, scales).T


def moe_fp8(x_bf16: np.ndarray, topk_ids: np.ndarray, topk_w: np.ndarray, w1_cache, w2_cache,
            tokens=None) -> np.ndarray:
    """out_t = sum_j g_tj * dq(q(h_tj)) . dq(W2c_e)^T,  h_tj = relu(dq(q(x_t)) . dq(W1c_e)^T)^2,
    e = topk_ids[t, j], q = mx_quantize, dq = mx_dequant, fp64.

    ``w1_cache[e]`` is expert e's up cache (codes [n1, k], scales [n1, k/32])
    and ``w2_cache[e]`` its down cache (codes [k, n1], scales [k, n1/32]); each
    may be a sequence or a callable e -> (codes, scales).  Ids outside [0, E)
    contribute nothing; ``tokens`` restricts the result to those rows.
    """
    xd = mx_dequant(*act_mxfp8(x_bf16))
    ids = np.asarray(topk_ids)
    g = np.asarray(topk_w, dtype=np.float64)
    t_all = np.arange(xd.shape[0]) if tokens is None else np.asarray(tokens)
    n_exp = None if callable(w1_cache) else len(w1_cache)
    get1 = w1_cache if callable(w1_cache) else (lambda e: w1_cache[e])
    get2 = w2_cache if callable(w2_cache) else (lambda e: w2_cache[e])
    out = np.zeros((len(t_all), xd.shape[1]), dtype=np.float64)
    sel = ids[t_all]
    for e in np.unique(sel):
        if e < 0 or (n_exp is not None and e >= n_exp):
            continue
        w1 = mx_dequant(*get1(int(e)))
        w2 = mx_dequant(*get2(int(e)))
        rows, js = np.nonzero(sel == e)
        h = np.maximum(xd[t_all[rows]] @ w1.T, 0.0) ** 2
        o = mx_dequant(*mx_quantize(h)) @ w2.T
        np.add.at(out, rows, g[t_all[rows], js][:, None] * o)  # a token may list e twice
    return out
