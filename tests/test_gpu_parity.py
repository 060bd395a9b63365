"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Bars: packed bytes and integer bucketing bit-exact; products within
relative Frobenius error <= 2e-3 and max |err| <= 1e-2 * rms(y_ref).
Full-size workloads compare every output where the oracle finishes in
seconds and sampled rows/tokens elsewhere.
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


def _check_close(y, ref, what="", out_round=0.0):
    """relF and max-abs bars.  out_round: the relative rounding step of an
    output stored narrower than fp32 (2^-9 for bf16, nearest even): it adds
    at most out_round * |y| per element, so at most out_round to relF and
    out_round * max|ref| to the max-abs bar."""
    y = np.asarray(y, dtype=np.float64)
    err = y - ref
    nref = np.linalg.norm(ref)
    relf = np.linalg.norm(err) / nref if nref > 0 else np.linalg.norm(err)
    rms = np.sqrt(np.mean(ref * ref))
    mx = np.max(np.abs(err)) if err.size else 0.0
    print(f"{what}: relF={relf:.3e} max/rms={mx / max(rms, 1e-300):.3e}")
    big = np.max(np.abs(ref)) if ref.size else 0.0
    assert relf <= REL_F + out_round, (what, relf)
    assert mx <= MAX_REL_RMS * rms + out_round * big * (1 + out_round), (what, mx, rms)


# ----------------------------------------------------------------------------- pack

@pytest.mark.parametrize("n,k,kind", [
    (512, 256, "gaussian"),          # 512x256 layer
    (8192, 2688, "gaussian"),        # dense denoiser projection
    (8192, 2688, "student_t3"),      # heavy-tailed prefill projection
    (3, 32, "gaussian"),
    (1, 2688, "student_t3"),
    (37, 96, "gaussian"),
])
def test_pack_bytes_equal_oracle(dev, n, k, kind):
    w = I.weights(n, k, kind)
    got = _ops().pack(torch.from_numpy(w).to(dev), SB).cpu().numpy()
    want = O.pack(w, SB)
    assert got.shape == want.shape
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} bytes differ, first at {bad[:5].tolist()}"


def test_pack_moe_experts_equal_oracle(experts):
    """All 128 experts' up and down projections, byte for byte."""
    _, _, _, mismatched = experts
    assert mismatched == []


@pytest.mark.parametrize("n,k,kind", [
    (8192, 2688, "gaussian"),        # dense denoiser projection, from bf16
    (1856, 2688, "student_t3"),      # an expert's up projection, heavy-tailed
    (37, 96, "gaussian"),
])
def test_pack_bf16_equals_oracle(dev, n, k, kind):
    # the checkpoint's bf16 weights: the oracle packs the same values widened
    # to fp32 (exact), so the bytes must agree
    w = I.weights(n, k, kind)
    w_bits = O.bf16_bits_from_f32(w)
    w_bf = O.f64_from_bf16_bits(w_bits).astype(np.float32)
    p = _ops().pack(_bf16(w_bits, dev), SB).cpu().numpy()
    assert np.array_equal(p, O.pack(w_bf, SB))
    # and tq4_pack on the widened values gives the same bytes
    p32 = _ops().pack(torch.from_numpy(w_bf).to(dev), SB).cpu().numpy()
    assert np.array_equal(p, p32)


def test_pack_special_blocks(dev):
    w = np.zeros((6, 64), dtype=np.float32)
    w[1, 7] = 1.0                                   # one-hot block
    w[2, :] = 0.5                                   # constant row
    w[3, 40] = -3e-3
    w[4, :32] = np.float32(1e-30)                   # tiny values
    rng = np.random.default_rng(1)
    w[5] = rng.standard_normal(64).astype(np.float32) * 1e4
    got = _ops().pack(torch.from_numpy(w).to(dev), SB).cpu().numpy()
    assert np.array_equal(got, O.pack(w, SB))


def test_pack_nonfinite_counted(dev):
    w = I.weights(4, 96)
    w[1, 5] = np.nan
    w[3, 70] = np.inf
    cnt = torch.zeros(1, dtype=torch.int32, device=dev)
    got = _ops().pack(torch.from_numpy(w).to(dev), SB, nonfinite=cnt).cpu().numpy()
    assert int(cnt.item()) == 2
    assert np.array_equal(got, O.pack(w, SB))


def test_pack_sign_bits_matter(dev):
    w = I.weights(16, 64)
    for sb in (0, 0xFFFFFFFF, 0x80000001):
        got = _ops().pack(torch.from_numpy(w).to(dev), sb).cpu().numpy()
        assert np.array_equal(got, O.pack(w, sb)), hex(sb)


# ----------------------------------------------------------------------- rotation

def test_act_rht_matches_oracle_rotation(dev):
    x = I.activations_bf16(33, 2688)
    got = _ops().act_rht(_bf16(x, dev), SB).cpu().numpy().astype(np.float64)
    want = O.rotate_blocks(O.f64_from_bf16_bits(x).reshape(33, -1, 32), SB).reshape(33, -1)
    # fp16 rounding of the result: |err| <= 2^-11 |v| (normal range)
    assert np.all(np.abs(got - want) <= 2.0 ** -11 * np.abs(want) + 2.0 ** -24)


# ------------------------------------------------------------------------- linear

def _linear_case(dev, m, k, n, kind="gaussian", wseed=0, xseed=2):
    w = I.weights(n, k, kind, seed=wseed)
    x = I.activations_bf16(m, k, seed=xseed)
    p_ref = O.pack(w, SB)
    p_gpu = _ops().pack(torch.from_numpy(w).to(dev), SB)
    y = _ops().linear(_bf16(x, dev), p_gpu, SB)
    torch.cuda.synchronize()
    return x, p_ref, y.cpu().numpy()


def test_linear_512x256_m16(dev):
    x, p, y = _linear_case(dev, 16, 256, 512)
    _check_close(y, O.linear(x, p, SB), "linear 16x256x512")


def test_linear_dense_m16_full(dev):
    x, p, y = _linear_case(dev, 16, 2688, 8192)
    _check_close(y, O.linear(x, p, SB), "linear 16x2688x8192")


@pytest.mark.parametrize("m,k,n", [
    (1, 32, 1), (1, 2688, 8192), (5, 96, 17), (16, 160, 129), (17, 64, 300),
    (33, 2688, 100), (64, 512, 256), (65, 256, 130), (100, 96, 77), (128, 2688, 256),
    (200, 1856, 300), (3, 4096, 64), (16, 8192, 64), (9, 2688, 8200), (16, 4096, 1000),
    # M <= 16 streaming kernel at its limits, and just past them
    (16, 2944, 100), (7, 3072, 64), (16, 128, 40), (2, 384, 33),
    # its split of the last chunks over the SIMDs: 4, 6, 8 and 15 chunks of
    # 128 k (halves only; halves and two split chunks; whole chunks and
    # halves; all three)
    (16, 512, 96), (5, 768, 70), (16, 1024, 64), (3, 1920, 50),
    # large-M kernel: chunk counts padded to a multiple of three, ragged M, N, K
    (300, 512, 520), (129, 96, 33), (256, 2688, 512),
    # 256 x 256 tiles (256 or more of them): K = 64 * (5, 2, 3) chunks (padding
    # of 1, 1, 0), one valid row or column in the last tile
    (257, 320, 32761), (512, 128, 32768), (300, 192, 32769),
])
def test_linear_ragged_shapes(dev, m, k, n):
    x, p, y = _linear_case(dev, m, k, n, wseed=m * 7 + n)
    _check_close(y, O.linear(x, p, SB), f"linear {m}x{k}x{n}")


@pytest.mark.parametrize("offset", [4, 16])
def test_linear_packed_alignment(dev, offset):
    """Packed weights 4 bytes past a 16-byte boundary take the register-load
    M <= 16 kernel; 16 bytes past take the LDS-direct one.  Same results."""
    m, k, n = 16, 2688, 300
    w = I.weights(n, k)
    x = I.activations_bf16(m, k)
    p = _ops().pack(torch.from_numpy(w).to(dev), SB)
    flat = torch.zeros(p.numel() + offset, dtype=torch.uint8, device=dev)
    flat[offset:] = p.reshape(-1)
    pv = flat[offset:].view(p.shape)
    assert (pv.data_ptr() % 16 == 0) == (offset == 16)
    y = _ops().linear(_bf16(x, dev), pv, SB)
    torch.cuda.synchronize()
    _check_close(y.cpu().numpy(), O.linear(x, O.pack(w, SB), SB), f"linear packed offset {offset}")


def test_linear_rejects_unaligned_activations(dev):
    from block_diffusion_lm_tq4_amd._lib import TQ4Error
    flat = torch.zeros(16 * 256 + 1, dtype=torch.bfloat16, device=dev)
    p = _ops().pack(torch.from_numpy(I.weights(64, 256)).to(dev), SB)
    with pytest.raises(TQ4Error, match="ALIGN"):
        _ops().linear(flat[1:].view(16, 256), p, SB)


def test_linear_prefill_m4096_sampled_rows(dev):
    m, k, n = 4096, 2688, 8192
    x, p, y = _linear_case(dev, m, k, n, kind="student_t3")
    rows = np.unique(np.concatenate([np.arange(0, m, 97), [m - 1]]))
    ref = O.linear(x[rows], p, SB)
    _check_close(y[rows], ref, "linear 4096x2688x8192 (sampled rows)")
    # property at full size: no NaN/Inf and the output scale matches
    assert np.isfinite(y).all()


def test_linear_identity_rows_read_the_weights(dev):
    k, n = 96, 64
    w = I.weights(n, k)
    eye = np.zeros((k, k), dtype=np.uint16)
    eye[np.arange(k), np.arange(k)] = 0x3F80
    p_gpu = _ops().pack(torch.from_numpy(w).to(dev), SB)
    y = _ops().linear(_bf16(eye, dev), p_gpu, SB).cpu().numpy()
    _check_close(y, O.dequant(O.pack(w, SB), SB).T, "identity rows")


def test_linear_deterministic(dev):
    w = I.weights(8192, 2688)
    x = _bf16(I.activations_bf16(16, 2688), dev)
    p = _ops().pack(torch.from_numpy(w).to(dev), SB)
    a = _ops().linear(x, p, SB).clone()
    b = _ops().linear(x, p, SB).clone()
    assert torch.equal(a, b)


def test_linear_workspace_reuse_across_shapes(dev):
    # zero-filled once (the exchange slots of the m <= 16 kernel), then shared
    # by calls of every shape, in an order that mixes both paths
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=dev)
    for (m, k, n) in [(16, 2688, 8192), (40, 512, 4096), (5, 256, 640), (100, 2688, 8192),
                      (16, 2688, 8192), (1, 8192, 333)]:
        w = I.weights(n, k, seed=n)
        x = I.activations_bf16(m, k)
        p = _ops().pack(torch.from_numpy(w).to(dev), SB)
        y = _ops().linear(_bf16(x, dev), p, SB, workspace=ws).cpu().numpy()
        _check_close(y, O.linear(x, O.pack(w, SB), SB), f"ws reuse {m}x{k}x{n}")


@pytest.mark.parametrize("m,k,n", [(16, 2688, 8192), (7, 96, 40), (300, 256, 200)])
def test_linear_rotated_equals_linear(dev, m, k, n):
    w = I.weights(n, k, seed=3)
    x = _bf16(I.activations_bf16(m, k), dev)
    p = _ops().pack(torch.from_numpy(w).to(dev), SB)
    a = _ops().linear(x, p, SB)
    b = _ops().linear_rotated(_ops().act_rht(x, SB), p)
    if m > 16:
        assert torch.equal(a, b)        # same kernels on both routes
    else:
        # the fused m <= 16 kernel rotates with MFMA sums: equal up to rounding
        ref = O.linear(I.activations_bf16(m, k), O.pack(w, SB), SB)
        _check_close(a.cpu().numpy(), ref, "fused")
        _check_close(b.cpu().numpy(), ref, "rotated")


@pytest.mark.parametrize("m,k,n,tail", [
    (16, 2688, 8192, "both"),      # M <= 16, LDS-direct kernel
    (16, 256, 512, "residual"),
    (5, 96, 17, "both"),           # M <= 16, register-load kernel
    (7, 3072, 64, "bias"),
    (33, 2688, 100, "both"),       # split-K: the tail rides the reduction
    (300, 512, 520, "both"),
    (64, 256, 32768, "bias"),      # one split, 64-row tiles
    (512, 256, 16384, "both"),     # 128 x 256 tiles
    (512, 128, 32768, "both"),     # 256 x 256 tiles
    (129, 96, 33, "inplace"),      # residual is the output itself
    (16, 2688, 8192, "inplace"),
])
def test_linear_epilogue_matches_oracle(dev, m, k, n, tail):
    w = I.weights(n, k, seed=m + n)
    x = I.activations_bf16(m, k, seed=5)
    p_ref = O.pack(w, SB)
    p_gpu = _ops().pack(torch.from_numpy(w).to(dev), SB)
    ref0 = O.linear(x, p_ref, SB)
    scale = float(np.sqrt(np.mean(ref0 * ref0)))
    rng = np.random.default_rng(m * 31 + n)
    bias = (rng.standard_normal(n) * scale).astype(np.float32)
    res = (rng.standard_normal((m, n)) * scale).astype(np.float32)
    use_b = tail in ("both", "bias", "inplace")
    use_r = tail in ("both", "residual", "inplace")
    xb = _bf16(x, dev)
    b_d = torch.from_numpy(bias).to(dev) if use_b else None
    r_d = torch.from_numpy(res).to(dev) if use_r else None
    if tail == "inplace":
        y = r_d.clone()
        out = _ops().linear_epilogue(xb, p_gpu, SB, bias=b_d, residual=y, out=y)
        assert out.data_ptr() == y.data_ptr()
    else:
        y = _ops().linear_epilogue(xb, p_gpu, SB, bias=b_d, residual=r_d)
    plain = _ops().linear(xb, p_gpu, SB)
    torch.cuda.synchronize()
    ref = O.linear_epilogue(x, p_ref, SB, bias if use_b else None, res if use_r else None)
    _check_close(y.cpu().numpy(), ref, f"epilogue {tail} {m}x{k}x{n}")
    # the fused tail is the plain product followed by two fp32 adds, bit for bit
    want = plain.clone()
    if use_b:
        want += b_d
    if use_r:
        want += r_d
    assert torch.equal(y, want)


@pytest.mark.parametrize("m,k,n,tail", [
    (16, 2688, 8192, "both"),      # M <= 16, LDS-direct kernel
    (5, 96, 17, "both"),           # M <= 16, register-load kernel
    (33, 2688, 100, "both"),       # split-K reduction
    (64, 256, 32768, "bias"),
    (512, 256, 16384, "residual"),  # 128 x 256 tiles
    (512, 128, 32768, "both"),     # 256 x 256 tiles
    (129, 96, 33, "inplace"),
    (16, 2688, 8192, "inplace"),
    (7, 64, 9, "none"),
])
def test_linear_epilogue_bf16_matches_oracle(dev, m, k, n, tail):
    w = I.weights(n, k, seed=m + 2 * n)
    x = I.activations_bf16(m, k, seed=6)
    p_ref = O.pack(w, SB)
    p_gpu = _ops().pack(torch.from_numpy(w).to(dev), SB)
    ref0 = O.linear(x, p_ref, SB)
    scale = float(np.sqrt(np.mean(ref0 * ref0)))
    rng = np.random.default_rng(m * 37 + n)
    bias = (rng.standard_normal(n) * scale).astype(np.float32)
    res16 = O.bf16_bits_from_f32((rng.standard_normal((m, n)) * scale).astype(np.float32))
    use_b = tail in ("both", "bias", "inplace")
    use_r = tail in ("both", "residual", "inplace")
    xb = _bf16(x, dev)
    b_d = torch.from_numpy(bias).to(dev) if use_b else None
    r_d = _bf16(res16, dev) if use_r else None
    if tail == "inplace":
        y = r_d.clone()
        _ops().linear_epilogue_bf16(xb, p_gpu, SB, bias=b_d, residual=y, out=y)
    else:
        y = _ops().linear_epilogue_bf16(xb, p_gpu, SB, bias=b_d, residual=r_d)
    y32 = _ops().linear_epilogue(xb, p_gpu, SB, bias=b_d,
                                 residual=r_d.float() if use_r else None)
    torch.cuda.synchronize()
    # the bf16 output is the fp32 variant's result rounded to nearest even
    assert torch.equal(y, y32.to(torch.bfloat16))
    ref = O.linear_epilogue(x, p_ref, SB, bias if use_b else None,
                            O.f64_from_bf16_bits(res16) if use_r else None)
    y64 = O.f64_from_bf16_bits(y.view(torch.int16).cpu().numpy().view(np.uint16))
    _check_close(y64, ref, f"epilogue bf16 {tail} {m}x{k}x{n}", out_round=2.0 ** -9)


def test_linear_epilogue_without_tail_is_linear(dev):
    w = I.weights(300, 2688, seed=9)
    p = _ops().pack(torch.from_numpy(w).to(dev), SB)
    for m in (16, 100):
        x = _bf16(I.activations_bf16(m, 2688), dev)
        assert torch.equal(_ops().linear_epilogue(x, p, SB), _ops().linear(x, p, SB))


def test_linear_epilogue_k0_writes_the_tail(dev):
    x = torch.empty((4, 0), dtype=torch.bfloat16, device=dev)
    p = torch.empty((8, 0, 20), dtype=torch.uint8, device=dev)
    b = torch.arange(8, dtype=torch.float32, device=dev)
    r = torch.full((4, 8), 0.5, device=dev)
    y = _ops().linear_epilogue(x, p, SB, bias=b, residual=r)
    assert torch.equal(y, b[None, :] + r)
    y = _ops().linear_epilogue(x, p, SB, bias=b)
    assert torch.equal(y, b[None, :].expand(4, 8))
    r16 = torch.full((4, 8), 0.25, dtype=torch.bfloat16, device=dev)
    y = _ops().linear_epilogue_bf16(x, p, SB, bias=b + 0.001, residual=r16)
    assert torch.equal(y, (b[None, :] + 0.001 + 0.25).to(torch.bfloat16).expand(4, 8))
    y = torch.full((4, 8), 3.0, dtype=torch.bfloat16, device=dev)
    _ops().linear_epilogue_bf16(x, p, SB, out=y)
    assert not y.float().any()


def test_linear_k0_writes_zeros(dev):
    x = torch.empty((4, 0), dtype=torch.bfloat16, device=dev)
    p = torch.empty((8, 0, 20), dtype=torch.uint8, device=dev)
    y = torch.full((4, 8), 7.0, device=dev)
    _ops().linear(x, p, SB, out=y)
    assert not y.any()


def test_read_probe_reads_and_keeps_nothing(dev):
    # the streaming-read reference used by the bench: runs over a buffer with
    # a ragged last workgroup and leaves its sink untouched
    buf = torch.randint(0, 255, (16 * 1000 + 16 * 37,), dtype=torch.uint8, device=dev)
    sink = torch.zeros(256, dtype=torch.float32, device=dev)
    _ops().read_probe(buf, sink)
    torch.cuda.synchronize()
    assert not sink.any()


# ---------------------------------------------------------------------------- MoE

@pytest.fixture(scope="module")
def experts(dev):
    """GPU-packed expert stacks for the 128-expert layer, plus the oracle's own
    packing of every expert (computed on the CPU in threads) and the list of
    experts whose GPU bytes differ from it."""
    from concurrent.futures import ThreadPoolExecutor
    n_exp, n1, k = 128, 1856, 2688
    w1 = torch.empty((n_exp, n1, k // 32, 20), dtype=torch.uint8, device=dev)
    w2 = torch.empty((n_exp, k, n1 // 32, 20), dtype=torch.uint8, device=dev)
    ref, bad = {}, []

    def work(e):
        a, b = I.expert_weights(e, 1, n1, k), I.expert_weights(e, 2, n1, k)
        return e, a, b, O.pack(a, SB), O.pack(b, SB)

    with ThreadPoolExecutor(8) as ex:
        for lo in range(0, n_exp, 16):
            for e, a, b, pa, pb in ex.map(work, range(lo, min(lo + 16, n_exp))):
                w1[e] = _ops().pack(torch.from_numpy(a).to(dev), SB)
                w2[e] = _ops().pack(torch.from_numpy(b).to(dev), SB)
                if not (np.array_equal(w1[e].cpu().numpy(), pa)
                        and np.array_equal(w2[e].cpu().numpy(), pb)):
                    bad.append(e)
                ref[e] = (pa, pb)
    return w1, w2, ref, bad


def _oracle_expert(experts, which):
    ref = experts[2]
    return lambda e: ref[int(e)][which - 1]


@pytest.mark.parametrize("name", ["moe_t16", "moe_t1024_uniform", "moe_t1024_zipf"])
def test_route_bit_exact(dev, name):
    wl = I.WORKLOADS[name]
    ids, _ = I.moe_routing(wl)
    counts, offsets, perm, inv = _ops().moe_route(torch.from_numpy(ids).to(dev), wl.n_experts)
    c, o, p, iv = O.bucket_pairs(ids, wl.n_experts)
    assert np.array_equal(counts.cpu().numpy(), c)
    assert np.array_equal(offsets.cpu().numpy(), o)
    assert np.array_equal(perm.cpu().numpy()[: p.size], p)
    assert np.array_equal(inv.cpu().numpy(), iv)


def test_route_invalid_ids_and_small_expert_counts(dev):
    rng = np.random.default_rng(3)
    for t, e, k in ((1, 1, 1), (7, 3, 2), (300, 128, 6), (5000, 512, 4), (64, 8, 8)):
        ids = rng.integers(-2, e + 2, size=(t, k)).astype(np.int32)
        counts, offsets, perm, inv = _ops().moe_route(torch.from_numpy(ids).to(dev), e)
        c, o, p, iv = O.bucket_pairs(ids, e)
        assert np.array_equal(counts.cpu().numpy(), c)
        assert np.array_equal(offsets.cpu().numpy(), o)
        assert np.array_equal(perm.cpu().numpy()[: p.size], p)
        assert np.array_equal(inv.cpu().numpy(), iv)


def _route_ids(t, e, topk, routing, seed):
    rng = np.random.default_rng(seed)
    if routing == "zipf":
        pr = 1.0 / np.arange(1, e + 1) ** 1.1
        ids = rng.choice(e, size=(t, topk), p=pr / pr.sum())
    elif routing == "invalid":
        ids = rng.integers(-3, e + 3, size=(t, topk))
    else:
        ids = rng.integers(0, e, size=(t, topk))
    return ids.astype(np.int32)


@pytest.mark.parametrize("t,e,topk,routing", [
    (1365, 128, 6, "uniform"),      # 8190 pairs: one bucketing workgroup
    (8191, 1, 1, "uniform"),        # its limit, every pair on one expert
    (8192, 1, 1, "uniform"),        # two chunks of 4096, every pair on one expert
    (8193, 7, 1, "invalid"),        # two chunks, the last one pair longer; bad ids
    (4096, 128, 6, "zipf"),         # six chunks, skewed experts
    (3001, 100, 7, "uniform"),      # experts not a multiple of 64, ragged last chunk
    (20000, 512, 8, "invalid"),     # largest expert count
    (65536, 128, 6, "uniform"),     # 96 chunks (prefill-sized layer)
    (700001, 64, 6, "zipf"),        # 4.2 M pairs: chunks of 8192, at most 1024 of them
])
def test_route_chunked_bit_exact(dev, t, e, topk, routing):
    """The bucketing equals the oracle's stable sort on both sides of the
    one-workgroup limit and for many chunks; perm past offsets[E] keeps the
    caller's contents."""
    ids = _route_ids(t, e, topk, routing, seed=t + e)
    counts, offsets, perm, inv = _ops().moe_route(torch.from_numpy(ids).to(dev), e)
    c, o, p, iv = O.bucket_pairs(ids, e)
    assert np.array_equal(counts.cpu().numpy(), c)
    assert np.array_equal(offsets.cpu().numpy(), o)
    pm = perm.cpu().numpy()
    assert np.array_equal(pm[: p.size], p)
    assert (pm[p.size:] == -7).all()
    assert np.array_equal(inv.cpu().numpy(), iv)


def test_moe_layer_chunked_bucketing(dev):
    """A layer whose bucketing takes the three-launch form (2600 tokens x
    top-6 = 15600 pairs): tile list, rotation and products against the
    oracle on every token."""
    t, e, k, n1, topk = 2600, 12, 64, 32, 6
    rng = np.random.default_rng(29)
    w1 = (0.05 * rng.standard_normal((e, n1, k))).astype(np.float32)
    w2 = (0.05 * rng.standard_normal((e, k, n1))).astype(np.float32)
    p1 = np.stack([O.pack(w1[i], SB) for i in range(e)])
    p2 = np.stack([O.pack(w2[i], SB) for i in range(e)])
    x = I.activations_bf16(t, k, seed=30)
    ids = _route_ids(t, e, topk, "zipf", seed=31)
    ids[5, 2] = -1                          # dropped slot
    g = rng.random((t, topk)).astype(np.float32)
    out = _ops().moe_grouped(_bf16(x, dev), torch.from_numpy(ids).to(dev),
                             torch.from_numpy(g).to(dev), torch.from_numpy(p1).to(dev),
                             torch.from_numpy(p2).to(dev), SB).cpu().numpy()
    _check_close(out, O.moe(x, ids, g, list(p1), list(p2), SB), "moe, chunked bucketing")


def test_moe_t16_full(dev, experts):
    wl = I.WORKLOADS["moe_t16"]
    ids, g = I.moe_routing(wl)
    x = I.activations_bf16(wl.t, wl.k)
    out = _ops().moe_grouped(_bf16(x, dev), torch.from_numpy(ids).to(dev),
                             torch.from_numpy(g).to(dev), experts[0], experts[1], SB).cpu().numpy()
    ref = O.moe(x, ids, g, _oracle_expert(experts, 1), _oracle_expert(experts, 2), SB)
    _check_close(out, ref, "moe t16")


@pytest.mark.parametrize("name", ["moe_t1024_uniform", "moe_t1024_zipf"])
def test_moe_t1024_sampled_tokens(dev, experts, name):
    wl = I.WORKLOADS[name]
    ids, g = I.moe_routing(wl)
    x = I.activations_bf16(wl.t, wl.k)
    out = _ops().moe_grouped(_bf16(x, dev), torch.from_numpy(ids).to(dev),
                             torch.from_numpy(g).to(dev), experts[0], experts[1], SB).cpu().numpy()
    assert np.isfinite(out).all()
    # tokens routed to the hottest expert plus a spread sample
    hot = np.bincount(ids.reshape(-1), minlength=128).argmax()
    tok = np.unique(np.concatenate([np.nonzero((ids == hot).any(1))[0][:4],
                                    np.arange(0, wl.t, 97), [wl.t - 1]]))
    ref = O.moe(x, ids, g, _oracle_expert(experts, 1), _oracle_expert(experts, 2), SB,
                tokens=tok)
    _check_close(out[tok], ref, name + " (sampled tokens)")


@pytest.mark.parametrize("t,e,k,routing", [
    (1024, 128, 6, "uniform"),       # batched block diffusion, uniform logits
    (1024, 128, 6, "zipf"),          # Zipf(1.1) expert popularity
    (16, 128, 6, "uniform"),         # one 16-token block
    (37, 100, 8, "uniform"),         # experts not a multiple of 64, ragged tokens
    (5, 512, 16, "zipf"),            # largest expert count
    (3, 1, 1, "uniform"),            # single expert
])
def test_router_matches_oracle(dev, t, e, k, routing):
    lg = I.router_logits(t, e, routing, seed=11).astype(np.float32)
    ids, g = _ops().moe_router(torch.from_numpy(lg).to(dev), k)
    ref_ids, ref_g = O.router(lg, k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert np.allclose(g.cpu().numpy(), ref_g, rtol=2e-6, atol=0)


def test_router_ties_and_empty(dev):
    lg = np.zeros((4, 128), dtype=np.float32)
    lg[1, [5, 9, 70, 71]] = 1.0           # ties among the top, across lanes
    lg[2, ::2] = 0.5                      # half the experts tied
    lg[3] = np.repeat(np.arange(32, dtype=np.float32), 4)  # ties in groups of 4
    ids, g = _ops().moe_router(torch.from_numpy(lg).to(dev), 6)
    ref_ids, ref_g = O.router(lg, 6)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert np.allclose(g.cpu().numpy(), ref_g, rtol=2e-6, atol=0)
    e_ids, e_g = _ops().moe_router(torch.empty((0, 128), device=dev), 6)
    assert e_ids.shape == (0, 6) and e_g.shape == (0, 6)


def test_moe_from_logits_matches_oracle(dev, experts):
    # router on the device feeding the grouped layer, against the oracle's
    # router feeding the oracle's layer (16 tokens, all outputs)
    wl = I.WORKLOADS["moe_t16"]
    lg = I.router_logits(wl.t, wl.n_experts, "uniform", seed=5).astype(np.float32)
    x_bits = I.activations_bf16(wl.t, wl.k)
    ids, g = _ops().moe_router(torch.from_numpy(lg).to(dev), wl.topk)
    out = _ops().moe_grouped(_bf16(x_bits, dev), ids, g, experts[0], experts[1], SB)
    ref_ids, ref_g = O.router(lg, wl.topk)
    ref = O.moe(x_bits, ref_ids, ref_g, _oracle_expert(experts, 1), _oracle_expert(experts, 2), SB)
    _check_close(out.cpu().numpy(), ref, "moe from logits")


@pytest.mark.parametrize("name", ["moe_t16", "moe_t1024_zipf"])
def test_moe_block_matches_oracle_and_the_two_calls(dev, experts, name):
    # tq4_moe_block: router + layer in one call; the same bits as the two
    # calls made separately, and the oracle's router + layer on sampled tokens
    wl = I.WORKLOADS[name]
    routing = "zipf" if "zipf" in name else "uniform"
    lg = I.router_logits(wl.t, wl.n_experts, routing, seed=7).astype(np.float32)
    x_bits = I.activations_bf16(wl.t, wl.k, seed=8)
    xb = _bf16(x_bits, dev)
    lg_d = torch.from_numpy(lg).to(dev)
    out = _ops().moe_block(xb, lg_d, wl.topk, experts[0], experts[1], SB)
    ids, g = _ops().moe_router(lg_d, wl.topk)
    two = _ops().moe_grouped(xb, ids, g, experts[0], experts[1], SB)
    torch.cuda.synchronize()
    assert torch.equal(out, two)
    tokens = np.arange(wl.t) if wl.t <= 16 else np.unique(np.r_[np.arange(0, wl.t, 97), wl.t - 1])
    ref_ids, ref_g = O.router(lg[tokens], wl.topk)
    ref = O.moe(x_bits[tokens], ref_ids, ref_g, _oracle_expert(experts, 1),
                _oracle_expert(experts, 2), SB)
    _check_close(out.cpu().numpy()[tokens], ref, f"moe block {name}")


@pytest.mark.parametrize("t,e,topk", [
    (17, 128, 6),    # the router inside the bucketing launch: 2 tokens per wave
    (64, 128, 6),    # its limit: 4 tokens per wave
    (65, 128, 6),    # past it: the separate router launch
    (40, 100, 4),    # experts not a multiple of 64
    (64, 100, 8),
    (1400, 16, 6),   # 8400 pairs: the bucketing in chunks
])
def test_moe_block_router_placements(dev, t, e, topk):
    """tq4_moe_block equals tq4_moe_router + tq4_moe_grouped bit for bit on
    both sides of the fused-router limit and for expert counts that do not
    fill a wave, and matches the oracle's router + layer."""
    rng = np.random.default_rng(t * 131 + e)
    k, n1 = 96, 64
    w1 = (0.05 * rng.standard_normal((e, n1, k))).astype(np.float32)
    w2 = (0.05 * rng.standard_normal((e, k, n1))).astype(np.float32)
    p1 = np.stack([O.pack(w1[i], SB) for i in range(e)])
    p2 = np.stack([O.pack(w2[i], SB) for i in range(e)])
    lg = I.router_logits(t, e, "zipf", seed=t).astype(np.float32)
    x_bits = I.activations_bf16(t, k, seed=t + 1)
    xb = _bf16(x_bits, dev)
    lg_d = torch.from_numpy(lg).to(dev)
    p1d, p2d = torch.from_numpy(p1).to(dev), torch.from_numpy(p2).to(dev)
    out = _ops().moe_block(xb, lg_d, topk, p1d, p2d, SB)
    ids, g = _ops().moe_router(lg_d, topk)
    two = _ops().moe_grouped(xb, ids, g, p1d, p2d, SB)
    torch.cuda.synchronize()
    assert torch.equal(out, two)
    ref_ids, ref_g = O.router(lg, topk)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    _check_close(out.cpu().numpy(), O.moe(x_bits, ref_ids, ref_g, list(p1), list(p2), SB),
                 f"moe block t{t} e{e} top{topk}")


def test_moe_block_persistent_t16_equals_moe_block(dev, experts):
    """tq4_moe_block_persistent on the 16-token block of the 128-expert layer:
    the same bits as tq4_moe_block (each of its steps runs the code of the
    corresponding launch on the same data), twice on one workspace (the grid
    barrier's counters are cleared per call), and the oracle's router + layer
    on every token."""
    wl = I.WORKLOADS["moe_t16"]
    lg = I.router_logits(wl.t, wl.n_experts, "uniform", seed=9).astype(np.float32)
    x_bits = I.activations_bf16(wl.t, wl.k, seed=10)
    xb = _bf16(x_bits, dev)
    lg_d = torch.from_numpy(lg).to(dev)
    out = _ops().moe_block_persistent(xb, lg_d, wl.topk, experts[0], experts[1], SB).clone()
    again = _ops().moe_block_persistent(xb, lg_d, wl.topk, experts[0], experts[1], SB)
    ref = _ops().moe_block(xb, lg_d, wl.topk, experts[0], experts[1], SB)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert torch.equal(again, ref)
    ref_ids, ref_g = O.router(lg, wl.topk)
    oracle = O.moe(x_bits, ref_ids, ref_g, _oracle_expert(experts, 1), _oracle_expert(experts, 2),
                   SB)
    _check_close(out.cpu().numpy(), oracle, "moe block persistent t16")


@pytest.mark.parametrize("t,e,topk", [
    (1, 8, 2),       # one token, fewer pairs than waves
    (17, 128, 6),
    (64, 100, 8),    # experts not a multiple of 64
    (40, 512, 4),    # the largest expert count
    (300, 128, 6),   # 1800 pairs: many 16-row tiles per expert
])
def test_moe_block_persistent_shapes(dev, t, e, topk):
    """tq4_moe_block_persistent equals tq4_moe_block bit for bit and matches
    the oracle's router + layer, over token and expert counts."""
    rng = np.random.default_rng(t * 7 + e)
    k, n1 = 96, 64
    w1 = (0.05 * rng.standard_normal((e, n1, k))).astype(np.float32)
    w2 = (0.05 * rng.standard_normal((e, k, n1))).astype(np.float32)
    p1 = np.stack([O.pack(w1[i], SB) for i in range(e)])
    p2 = np.stack([O.pack(w2[i], SB) for i in range(e)])
    lg = I.router_logits(t, e, "zipf", seed=t + 3).astype(np.float32)
    x_bits = I.activations_bf16(t, k, seed=t + 4)
    xb = _bf16(x_bits, dev)
    lg_d = torch.from_numpy(lg).to(dev)
    p1d, p2d = torch.from_numpy(p1).to(dev), torch.from_numpy(p2).to(dev)
    out = _ops().moe_block_persistent(xb, lg_d, topk, p1d, p2d, SB)
    ref = _ops().moe_block(xb, lg_d, topk, p1d, p2d, SB)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    ref_ids, ref_g = O.router(lg, topk)
    _check_close(out.cpu().numpy(), O.moe(x_bits, ref_ids, ref_g, list(p1), list(p2), SB),
                 f"moe block persistent t{t} e{e} top{topk}")


def test_moe_deterministic(dev, experts):
    wl = I.WORKLOADS["moe_t1024_zipf"]
    ids, g = I.moe_routing(wl)
    x = _bf16(I.activations_bf16(wl.t, wl.k), dev)
    idt, gt = torch.from_numpy(ids).to(dev), torch.from_numpy(g).to(dev)
    a = _ops().moe_grouped(x, idt, gt, experts[0], experts[1], SB).clone()
    b = _ops().moe_grouped(x, idt, gt, experts[0], experts[1], SB).clone()
    assert torch.equal(a, b)


def test_moe_small_shapes_and_invalid_ids(dev):
    rng = np.random.default_rng(11)
    for (t, e, k, n1, topk) in ((1, 4, 32, 32, 1), (9, 8, 64, 96, 3), (40, 16, 96, 64, 4),
                                (300, 8, 64, 32, 2)):
        w1 = (0.05 * rng.standard_normal((e, n1, k))).astype(np.float32)
        w2 = (0.05 * rng.standard_normal((e, k, n1))).astype(np.float32)
        p1 = np.stack([O.pack(w1[i], SB) for i in range(e)])
        p2 = np.stack([O.pack(w2[i], SB) for i in range(e)])
        x = I.activations_bf16(t, k, seed=t)
        ids, g = I.route(rng.standard_normal((t, e)), topk)
        ids = ids.copy()
        ids[0, 0] = -1                      # dropped slot
        out = _ops().moe_grouped(_bf16(x, dev), torch.from_numpy(ids).to(dev),
                                 torch.from_numpy(g).to(dev), torch.from_numpy(p1).to(dev),
                                 torch.from_numpy(p2).to(dev), SB).cpu().numpy()
        _check_close(out, O.moe(x, ids, g, list(p1), list(p2), SB), f"moe t{t} e{e}")


# ------------------------------------------------------------------- graph replay

def test_graph_replays_match_eager(dev, experts):
    """Captured calls replayed several times, with eager work and syncs in
    between, give the eager results bit for bit."""
    ops = _ops()
    w = I.weights(8192, 2688)
    p = ops.pack(torch.from_numpy(w).to(dev), SB)
    x16 = _bf16(I.activations_bf16(16, 2688), dev)
    x100 = _bf16(I.activations_bf16(100, 2688), dev)
    wl = I.WORKLOADS["moe_t16"]
    ids, g = I.moe_routing(wl)
    xm = _bf16(I.activations_bf16(wl.t, wl.k), dev)
    idt, gt = torch.from_numpy(ids).to(dev), torch.from_numpy(g).to(dev)
    y16 = torch.empty((16, 8192), device=dev)
    y100 = torch.empty((100, 8192), device=dev)
    om = torch.empty((wl.t, wl.k), device=dev)
    ws_lin = torch.zeros(ops.linear_workspace_size(100, 2688, 8192), dtype=torch.uint8, device=dev)
    ws_moe = torch.zeros(ops.moe_workspace_size(wl.t, 6, 128, 1856, 2688), dtype=torch.uint8,
                         device=dev)
    # the fp8 variants: dense at M=16 and M=100, and the MoE layer
    c = ops.fp8_cache(p, SB)
    c1, c2 = ops.fp8_cache_experts(experts[0], SB), ops.fp8_cache_experts(experts[1], SB)
    f16 = torch.empty((16, 8192), device=dev)
    f100 = torch.empty((100, 8192), device=dev)
    fm = torch.empty((wl.t, wl.k), device=dev)
    ws_f16 = torch.zeros(ops.linear_fp8_workspace_size(16, 2688, 8192), dtype=torch.uint8,
                         device=dev)
    ws_f100 = torch.zeros(ops.linear_fp8_workspace_size(100, 2688, 8192), dtype=torch.uint8,
                          device=dev)
    ws_fm = torch.zeros(ops.moe_grouped_fp8_workspace_size(wl.t, 6, 128, 1856, 2688),
                        dtype=torch.uint8, device=dev)
    outs = (y16, y100, om, f16, f100, fm)

    def run():
        ops.linear(x16, p, SB, out=y16)
        ops.linear(x100, p, SB, out=y100, workspace=ws_lin)
        ops.moe_grouped(xm, idt, gt, experts[0], experts[1], SB, out=om, workspace=ws_moe)
        ops.linear_fp8(x16, c, 8192, out=f16, workspace=ws_f16)
        ops.linear_fp8(x100, c, 8192, out=f100, workspace=ws_f100)
        ops.moe_grouped_fp8(xm, idt, gt, c1, c2, 128, 1856, out=fm, workspace=ws_fm)

    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        junk = ops.linear(x100, p, SB)          # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk).all()
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a, b), (rep, i)
