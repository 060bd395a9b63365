"""How the block-scaled fp8 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4) sums
products: the arithmetic that the fp8 weight-cache products' error bound rests
on (tests/test_gpu_fp8.py, tests/test_gpu_fp8_moe.py).

The bound assumes that inside one 32-element block every product at least
2^-13 of the block's largest product is summed exactly and any smaller one
errs by less than 2^-13 of the largest (kept, rounded or dropped), that the
block sums and the accumulator are combined in fp32, and that a block
whose scale is 2^-127 (E8M0 byte 0) or whose data are zero leaves the
accumulator bit for bit unchanged (the padding of the cache rows and the dead
steps rely on it).  Each case below isolates one of these facts on a single
output element; every other element must come out exactly as its accumulator
input.  The operands are e4m3 codes chosen so that each product is a power
of two, exactly representable: 1.0 = 0x38, 2^-6 = 0x08 (the smallest normal),
2^-7 = 0x04, 2^-8 = 0x02 (subnormals m * 2^-9).
"""

import ctypes
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native",
                   "libmfma_scale_probe.so")
ONE, P6, P7, P8 = 0x38, 0x08, 0x04, 0x02
UNIT = 127                      # E8M0 scale 2^0


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB)
    lib.tq4test_mfma_scale_probe.argtypes = [ctypes.c_void_p] * 7
    dev = torch.device("cuda:0")

    def run(a, b, sa, sb, c):
        t = [torch.from_numpy(np.ascontiguousarray(v)).to(dev) for v in (a, b, sa, sb, c)]
        d = torch.empty((16, 16), dtype=torch.float32, device=dev)
        rc = lib.tq4test_mfma_scale_probe(*(v.data_ptr() for v in t), d.data_ptr(),
                                          torch.cuda.current_stream().cuda_stream)
        assert rc == 0
        torch.cuda.synchronize()
        return d.cpu().numpy()
    return run


def _case(seed=0):
    """Zero operands, unit scales, and an accumulator of distinct values."""
    a = np.zeros((16, 128), dtype=np.uint8)
    b = np.zeros((16, 128), dtype=np.uint8)
    sa = np.full((16, 4), UNIT, dtype=np.uint8)
    sb = np.full((16, 4), UNIT, dtype=np.uint8)
    c = np.random.default_rng(seed).standard_normal((16, 16)).astype(np.float32)
    return a, b, sa, sb, c


def _check(d, c, want00):
    """d[0, 0] == want00 exactly (as fp32); every other element equals c."""
    assert np.float32(d[0, 0]) == np.float32(want00), (float(d[0, 0]), float(want00))
    rest = np.ones((16, 16), dtype=bool)
    rest[0, 0] = False
    assert np.array_equal(d[rest].view(np.uint32), c[rest].view(np.uint32))


def test_a_product_is_exact(probe):
    a, b, sa, sb, c = _case()
    c[0, 0] = 0.0
    a[0, 5], b[0, 5] = ONE, P7
    _check(probe(a, b, sa, sb, c), c, 2.0 ** -7)


@pytest.mark.parametrize("blk", [0, 3])
def test_products_2e13_below_the_largest_are_kept(probe, blk):
    # products 1 and 2^-13 in one block: 1 + 2^-13 (exact in fp32)
    a, b, sa, sb, c = _case(1)
    c[0, 0] = 0.0
    k0 = 32 * blk
    a[0, k0], b[0, k0] = ONE, ONE
    a[0, k0 + 17], b[0, k0 + 17] = P6, P7
    _check(probe(a, b, sa, sb, c), c, 1.0 + 2.0 ** -13)


@pytest.mark.parametrize("ca,cb,p", [
    (P6, P8, -14), (P6, 0x01, -15), (P8, P8, -16), (P8, 0x01, -17), (0x01, 0x01, -18),
])
def test_smaller_products_err_by_less_than_2e13(probe, ca, cb, p):
    # products 1 and 2^p (p < -13) in one block: whether the instruction keeps
    # or drops the small one, the result stays within 2^-13 of 1 + 2^p, which
    # is all the error bound assumes of a product below its 13-bit window
    # (1 + 2^p is exact in fp32 down to p = -23, so any loss is the
    # instruction's own)
    a, b, sa, sb, c = _case(2)
    c[0, 0] = 0.0
    a[0, 0], b[0, 0] = ONE, ONE
    a[0, 9], b[0, 9] = ca, cb
    d = probe(a, b, sa, sb, c)
    exact = 1.0 + 2.0 ** p
    got = float(d[0, 0])
    how = "kept" if got == exact else ("dropped" if got == 1.0 else "rounded")
    print(f"1 + 2^{p}: device {got!r} ({how})")
    assert abs(got - exact) < 2.0 ** -13
    rest = np.ones((16, 16), dtype=bool)
    rest[0, 0] = False
    assert np.array_equal(d[rest].view(np.uint32), c[rest].view(np.uint32))


def test_the_window_is_per_block(probe):
    # 1 in block 0, 2^-20 in block 1: the block sums meet in fp32, so the small
    # one survives although it is 2^-20 of the large one
    a, b, sa, sb, c = _case(3)
    c[0, 0] = 0.0
    a[0, 0], b[0, 0] = ONE, ONE
    a[0, 40], b[0, 40] = P6, P7
    sa[0, 1] = UNIT - 7               # block 1 of row 0 scaled by 2^-7
    _check(probe(a, b, sa, sb, c), c, 1.0 + 2.0 ** -20)


def test_the_accumulator_is_added_in_fp32(probe):
    a, b, sa, sb, c = _case(4)
    c[0, 0] = 1.0
    a[0, 3], b[0, 3] = P6, P7
    sa[0, 0] = UNIT - 10              # product 2^-23: 1 + 2^-23 is the next fp32 up
    _check(probe(a, b, sa, sb, c), c, 1.0 + 2.0 ** -23)


def test_scale_2e_127_leaves_the_accumulator_unchanged(probe):
    a, b, sa, sb, c = _case(5)
    a[:, :] = ONE
    b[:, :] = ONE
    sa[:, :] = 0                      # every block of A scaled by 2^-127
    d = probe(a, b, sa, sb, c)
    assert np.array_equal(d.view(np.uint32), c.view(np.uint32))


def test_zero_data_leave_the_accumulator_unchanged(probe):
    a, b, sa, sb, c = _case(6)
    sa[:, :] = UNIT + 20
    sb[:, :] = UNIT + 20
    d = probe(a, b, sa, sb, c)
    assert np.array_equal(d.view(np.uint32), c.view(np.uint32))


def test_all_elements_follow_the_same_layout(probe):
    # one product per output element, 2^-(m+n) scaled by A's and B's row
    # scales, read back element by element: the operand and accumulator
    # layout the fp8 kernels use
    a, b, sa, sb, c = _case(7)
    c[:, :] = 0.0
    a[:, 64] = ONE
    b[:, 64] = ONE
    for m in range(16):
        sa[m, 2] = UNIT - m
        sb[m, 2] = UNIT - 2 * m
    d = probe(a, b, sa, sb, c)
    want = np.array([[2.0 ** -(m + 2 * n) for n in range(16)] for m in range(16)], dtype=np.float32)
    assert np.array_equal(d, want)
