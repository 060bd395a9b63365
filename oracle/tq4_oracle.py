"""TQ4_1S oracle: the format and the layer written out plainly in NumPy fp64.

TEST INFRASTRUCTURE ONLY -- imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.  It
shares no code with the HIP library.

Source of the method: the Nemotron-TheHobbit-30B-A3B model card (English and
Chinese renderings), section *What "Config-I" means*: TurboQuant's TQ4_1S
weight format applies a randomized Walsh-Hadamard rotation to every block of
32 weights, then quantizes to a 4-bit, 16-level Lloyd-Max codebook with two
half-block scales, about 5 bits per weight; one fixed codebook serves every
tensor because the rotation makes each block close to Gaussian.  Section
*Running it* of the same card: the quantized Linears are replaced by an
on-the-fly dequantizing layer and the MoE runs without host syncs; section
*The model underneath*: 128 experts, top-6.

The card states no bit layout, scale rule, codebook precision, sign generator
or Hadamard ordering.  The readings taken here (each one is listed with its
reason in the design notes) are:

* block axis: 32 consecutive input features (K) of one output row;
* rotation: z = H32 (s * w) / sqrt(32), H32 in Sylvester order, H[i,j] =
  (-1)^popcount(i & j); one 32-entry sign vector s for every block;
* codebook: the 16-level Lloyd-Max quantizer of N(0,1), rounded to fp32,
  ascending (code 0 is the most negative level);
* scale rule: per half-block (elements 0-15 and 16-31 of the *rotated*
  block) S = max|z| / c_15, rounded fp64 -> fp32 -> bf16, both
  round-to-nearest-even;
* codes: q = number of midpoints m_k = (c_k + c_{k+1})/2 with z > S*m_k, so a
  value exactly on a midpoint takes the lower index;
* bytes: 16 code bytes (byte i = q_{2i} | q_{2i+1} << 4), then the bf16 bits
  of S_0 and S_1, little-endian: 20 bytes per block, blocks row-major
  [N][K/32];
* dequant: z_hat = S_h * c_q, w_hat = s * (H32 z_hat) / sqrt(32);
* linear: y = x . W_hat^T, no bias, x given as bf16;
* MoE: out_t = sum_j g_tj * relu(x_t . W1_e^T)^2 . W2_e^T with e = ids[t, j];
  expert ids outside [0, E) contribute nothing.
"""

from __future__ import annotations

import math

import numpy as np
from scipy.special import erfc, ndtri

__all__ = [
    "BLOCK",
    "BLOCK_BYTES",
    "RS32",
    "lloyd_max_gaussian",
    "codebook",
    "midpoints",
    "hadamard32",
    "signs_from_bits",
    "rotation_matrix",
    "bf16_bits_from_f32",
    "f64_from_bf16_bits",
    "rotate_blocks",
    "half_scales",
    "codes_for",
    "pack",
    "unpack",
    "dequant_rotated",
    "dequant",
    "linear",
    "linear_epilogue",
    "moe",
    "bucket_pairs",
    "router",
    "packed_size",
]

BLOCK = 32
BLOCK_BYTES = 20
# 1/sqrt(32) = sqrt(2)/8; sqrt is correctly rounded and /8 is exact, so this is
# the correctly rounded fp64 value of 1/sqrt(32).
RS32 = math.sqrt(2.0) / 8.0


# ----------------------------------------------------------------------------
# Codebook: 16-level Lloyd-Max quantizer for N(0, 1)
# (model card, section *What "Config-I" means*: "16-level Lloyd-Max").
# ----------------------------------------------------------------------------

def _phi(x: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _interval_prob(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """P(a < X < b) for X ~ N(0,1), from the nearer tail to avoid cancellation."""
    r2 = math.sqrt(2.0)
    left = 0.5 * erfc(-b / r2) - 0.5 * erfc(-a / r2)   # Phi(b) - Phi(a)
    right = 0.5 * erfc(a / r2) - 0.5 * erfc(b / r2)    # Q(a) - Q(b)
    return np.where(b <= 0.0, left, right)


def lloyd_max_gaussian(levels: int = 16, tol: float = 1e-13,
                       init: np.ndarray | None = None,
                       max_iter: int = 200000) -> tuple[np.ndarray, int]:
    """Lloyd-Max iteration for N(0,1): alternate the two optimality conditions.

    * nearest neighbour: the decision thresholds are the midpoints of
      adjacent levels;
    * centroid: each level is E[X | X in its cell] = (phi(a)-phi(b)) / P(a<X<b).

    Starts from the quantiles Phi^-1((i+1/2)/L) unless ``init`` is given and
    stops when no level moves by ``tol`` or more.  Returns (levels, iterations).
    """
    c = (ndtri((np.arange(levels) + 0.5) / levels) if init is None
         else np.array(init, dtype=np.float64))
    for it in range(1, max_iter + 1):
        t = 0.5 * (c[:-1] + c[1:])
        a = np.concatenate([[-np.inf], t])
        b = np.concatenate([t, [np.inf]])
        new = (_phi(a) - _phi(b)) / _interval_prob(a, b)
        moved = float(np.max(np.abs(new - c)))
        c = new
        if moved < tol:
            return c, it
    raise RuntimeError("Lloyd-Max iteration did not converge")


_CODEBOOK32: np.ndarray | None = None


def codebook() -> np.ndarray:
    """The 16 stored levels: the Lloyd-Max levels rounded to fp32, ascending."""
    global _CODEBOOK32
    if _CODEBOOK32 is None:
        c, _ = lloyd_max_gaussian(16)
        _CODEBOOK32 = c.astype(np.float32)
        _CODEBOOK32.setflags(write=False)
    return _CODEBOOK32


def midpoints(cb32: np.ndarray | None = None) -> np.ndarray:
    """m_k = (c_k + c_{k+1}) / 2 in fp64, k = 0..14 (exact: two fp32 summands)."""
    c = (codebook() if cb32 is None else cb32).astype(np.float64)
    return 0.5 * (c[:-1] + c[1:])


# ----------------------------------------------------------------------------
# Randomized Walsh-Hadamard rotation per 32-block
# (model card, section *What "Config-I" means*: "Walsh-Hadamard (RHT) rotation
# applied per 32-element block").
# ----------------------------------------------------------------------------

def hadamard32() -> np.ndarray:
    """Sylvester-ordered H32 with H[i, j] = (-1)^popcount(i & j), as fp64."""
    i = np.arange(BLOCK)
    par = np.array([[bin(a & b).count("1") & 1 for b in i] for a in i])
    return np.where(par == 0, 1.0, -1.0)


def signs_from_bits(sign_bits: int) -> np.ndarray:
    """s_i = -1 where bit i of ``sign_bits`` is set, else +1 (fp64, 32 entries)."""
    sb = int(sign_bits) & 0xFFFFFFFF
    return np.array([-1.0 if (sb >> i) & 1 else 1.0 for i in range(BLOCK)])


def rotation_matrix(sign_bits: int) -> np.ndarray:
    """R = H32 diag(s) / sqrt(32): z = R w for one block (orthogonal)."""
    return hadamard32() * signs_from_bits(sign_bits)[None, :] / math.sqrt(32.0)


def rotate_blocks(w: np.ndarray, sign_bits: int) -> np.ndarray:
    """z = H32 (s * w) * (1/sqrt(32)) for every trailing 32-vector of ``w``.

    The sign flip is exact, H32 is applied as a plain product with the +-1
    matrix in fp64, and the final multiply rounds once.
    """
    v = np.asarray(w, dtype=np.float64) * signs_from_bits(sign_bits)
    u = v @ hadamard32().T
    return u * RS32


# ----------------------------------------------------------------------------
# bf16 rounding (round to nearest, ties to even), written on the bit pattern.
# ----------------------------------------------------------------------------

def bf16_bits_from_f32(f: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (RNE); returns the 16-bit patterns as uint16."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    is_nan = (u & 0x7FFFFFFF) > 0x7F800000
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    out = np.where(is_nan, 0x7FC0, rounded)
    return out.astype(np.uint16)


def f64_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns as fp64."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# Encoder
# ----------------------------------------------------------------------------

def half_scales(z: np.ndarray, cb32: np.ndarray | None = None) -> np.ndarray:
    """bf16 bits of S_h = bf16(fp32(max_{j in h} |z_j| / c_15)) for h = 0, 1.

    ``z`` has shape [..., 32]; the result has shape [..., 2] (uint16).
    """
    c15 = float((codebook() if cb32 is None else cb32)[-1])
    a = np.abs(z).reshape(z.shape[:-1] + (2, 16)).max(axis=-1)
    with np.errstate(over="ignore", invalid="ignore"):
        s32 = (a / c15).astype(np.float32)
    return bf16_bits_from_f32(s32)


def codes_for(z: np.ndarray, scale: np.ndarray,
              cb32: np.ndarray | None = None) -> np.ndarray:
    """q = #{k : z > S * m_k} elementwise (``scale`` broadcast against ``z``).

    S * m_k is exact in fp64 (8 significant bits times at most 26), so the
    comparison is the exact one and a tie resolves to the lower index.
    """
    m = midpoints(cb32)
    z = np.asarray(z, dtype=np.float64)
    s = np.asarray(scale, dtype=np.float64)
    q = np.zeros(np.broadcast(z, s).shape, dtype=np.uint8)
    with np.errstate(invalid="ignore"):
        for mk in m:
            q += (z > s * mk).astype(np.uint8)
    return q


def pack(w: np.ndarray, sign_bits: int) -> np.ndarray:
    """Encode fp32 W [N, K] (K % 32 == 0) into uint8 [N, K/32, 20]."""
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2 or w.shape[1] % BLOCK:
        raise ValueError("pack expects W of shape [N, K] with K a multiple of 32")
    n, k = w.shape
    kb = k // BLOCK
    out = np.empty((n, kb, BLOCK_BYTES), dtype=np.uint8)
    rows = max(1, (1 << 21) // max(k, 1))        # bound the fp64 temporaries
    for r0 in range(0, n, rows):
        blk = w[r0:r0 + rows].reshape(-1, kb, BLOCK)
        z = rotate_blocks(blk, sign_bits)
        sb = half_scales(z)                                   # [r, kb, 2] bf16 bits
        s64 = np.repeat(f64_from_bf16_bits(sb), 16, axis=-1)  # [r, kb, 32]
        q = codes_for(z, s64)
        o = out[r0:r0 + rows]
        o[..., :16] = q[..., 0::2] | (q[..., 1::2] << 4)
        o[..., 16] = sb[..., 0] & 0xFF
        o[..., 17] = sb[..., 0] >> 8
        o[..., 18] = sb[..., 1] & 0xFF
        o[..., 19] = sb[..., 1] >> 8
    return out


def packed_size(n: int, k: int) -> int:
    return n * (k // BLOCK) * BLOCK_BYTES


# ----------------------------------------------------------------------------
# Decoder and the layer
# ----------------------------------------------------------------------------

def unpack(packed: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """uint8 [..., 20] -> (codes uint8 [..., 32], scale bf16 bits uint16 [..., 2])."""
    p = np.asarray(packed, dtype=np.uint8)
    q = np.empty(p.shape[:-1] + (BLOCK,), dtype=np.uint8)
    q[..., 0::2] = p[..., :16] & 0x0F
    q[..., 1::2] = p[..., :16] >> 4
    s = np.stack([p[..., 16].astype(np.uint16) | (p[..., 17].astype(np.uint16) << 8),
                  p[..., 18].astype(np.uint16) | (p[..., 19].astype(np.uint16) << 8)],
                 axis=-1)
    return q, s


def dequant_rotated(packed: np.ndarray) -> np.ndarray:
    """z_hat = S_h * c_q in the rotated domain, fp64, shape [N, K]."""
    q, s = unpack(packed)
    c = codebook().astype(np.float64)
    scale = np.repeat(f64_from_bf16_bits(s), 16, axis=-1)
    z = scale * c[q]
    return z.reshape(z.shape[0], -1)


def dequant(packed: np.ndarray, sign_bits: int) -> np.ndarray:
    """W_hat = s * (H32 z_hat) / sqrt(32) per block, fp64, shape [N, K].

    H32 is symmetric and H32 H32 = 32 I, so this inverts ``rotate_blocks``.
    """
    z = dequant_rotated(packed)
    n = z.shape[0]
    zb = z.reshape(n, -1, BLOCK)
    w = (zb @ hadamard32().T) * RS32 * signs_from_bits(sign_bits)
    return w.reshape(n, -1)


def linear(x_bf16: np.ndarray, packed: np.ndarray, sign_bits: int) -> np.ndarray:
    """y = x . W_hat^T in fp64; x is given as bf16 bit patterns [M, K]."""
    x = f64_from_bf16_bits(x_bf16)
    return x @ dequant(packed, sign_bits).T


def linear_epilogue(x_bf16: np.ndarray, packed: np.ndarray, sign_bits: int,
                    bias: np.ndarray | None = None,
                    residual: np.ndarray | None = None) -> np.ndarray:
    """y = x . W_hat^T + bias[n] + residual[m, n] in fp64, each term optional.

    The model card (section Running it) swaps the model's quantized Linear
    modules for an on-the-fly dequantizing layer; a Linear's optional bias is
    added per output feature, and the block's residual stream is added per
    element.  Terms are summed left to right: product, bias, residual."""
    y = linear(x_bf16, packed, sign_bits)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    if residual is not None:
        y = y + np.asarray(residual, dtype=np.float64)
    return y


def moe(x_bf16: np.ndarray, topk_ids: np.ndarray, topk_w: np.ndarray,
        w1_packed, w2_packed, sign_bits: int, tokens=None) -> np.ndarray:
    """out_t = sum_j g_tj * relu(x_t . W1_e^T)^2 . W2_e^T, e = topk_ids[t, j].

    ``w1_packed[e]`` is expert e's packed up projection [n1, K/32, 20] and
    ``w2_packed[e]`` its packed down projection [K, n1/32, 20]; each may be a
    sequence or a callable e -> array, so experts can be produced on demand.
    Ids outside [0, E) contribute nothing.  ``tokens`` restricts the result to
    those token rows (all by default).  fp64 throughout.
    """
    x = f64_from_bf16_bits(x_bf16)
    ids = np.asarray(topk_ids)
    g = np.asarray(topk_w, dtype=np.float64)
    t_all = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
    n_exp = len(w1_packed) if not callable(w1_packed) else None
    get1 = w1_packed if callable(w1_packed) else (lambda e: w1_packed[e])
    get2 = w2_packed if callable(w2_packed) else (lambda e: w2_packed[e])
    out = np.zeros((len(t_all), x.shape[1]), dtype=np.float64)
    sel = ids[t_all]
    for e in np.unique(sel):
        if e < 0 or (n_exp is not None and e >= n_exp):
            continue
        w1 = dequant(get1(int(e)), sign_bits)
        w2 = dequant(get2(int(e)), sign_bits)
        rows, js = np.nonzero(sel == e)
        h = np.maximum(x[t_all[rows]] @ w1.T, 0.0) ** 2
        o = h @ w2.T
        np.add.at(out, rows, g[t_all[rows], js][:, None] * o)  # a token may list e twice
    return out


def bucket_pairs(topk_ids: np.ndarray, n_experts: int):
    """Stable counting sort of the T*topk (token, slot) pairs by expert.

    Pair p = t*topk + j.  Returns (counts[E], offsets[E+1], perm[P], inv[P]):
    perm lists the pairs of expert 0 first, then expert 1, ..., each group in
    increasing p; pairs with an id outside [0, E) are left out of perm and get
    inv = -1; inv[perm[i]] = i.
    """
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    valid = (ids >= 0) & (ids < n_experts)
    counts = np.bincount(ids[valid], minlength=n_experts).astype(np.int32)
    offsets = np.zeros(n_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(np.where(valid, ids, n_experts), kind="stable")
    perm = order[: int(valid.sum())].astype(np.int32)
    inv = np.full(ids.shape[0], -1, dtype=np.int32)
    inv[perm] = np.arange(perm.shape[0], dtype=np.int32)
    return counts, offsets, perm, inv


def router(logits: np.ndarray, topk: int):
    """The MoE router before the layer (model card, The model underneath:
    128 experts, top-6): softmax over all expert logits of a token, then the
    topk experts with the largest logits, ties to the lower expert id; each
    gate is that expert's softmax probability, not renormalized over the k.

    logits [T, E] (any float dtype, read exactly); returns (ids int32 [T, k],
    gates fp64 [T, k]) with ids in decreasing logit order.  Plain per-token
    loops, fp64 arithmetic.
    """
    lg = np.asarray(logits, dtype=np.float64)
    t, e = lg.shape
    ids = np.zeros((t, topk), dtype=np.int32)
    gates = np.zeros((t, topk), dtype=np.float64)
    for i in range(t):
        row = lg[i]
        mx = max(row)
        ex = [np.exp(v - mx) for v in row]
        total = sum(ex)
        taken = set()
        for j in range(topk):
            best = -1
            for c in range(e):
                if c in taken:
                    continue
                if best < 0 or row[c] > row[best]:
                    best = c
            taken.add(best)
            ids[i, j] = best
            gates[i, j] = ex[best] / total
    return ids, gates

