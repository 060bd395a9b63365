"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the device."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from block_diffusion_lm_tq4_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq4.h")

OK, E_NULL, E_SHAPE, E_ALIGN, E_WS = 0, 1, 2, 3, 4
FAKE = 0x10000          # a non-null, 256-byte aligned address that is never touched
MIS = FAKE + 2          # misaligned


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libtq4.so is not built (run __graft_entry__.build())")
    return _lib.lib()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tq4_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(L):
    names = _declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.SIGNATURES)


def test_status_strings_and_version(L):
    for s in range(7):
        assert L.tq4_status_string(s)
    assert L.tq4_status_string(99) == b"unknown status"
    assert L.tq4_version() >= 100


def test_codebook_equals_oracle_bit_for_bit(L):
    out = (ctypes.c_float * 16)()
    assert L.tq4_codebook(ctypes.addressof(out)) == OK
    lib_cb = np.frombuffer(out, dtype=np.float32)
    assert np.array_equal(lib_cb.view(np.uint32), O.codebook().view(np.uint32))
    assert L.tq4_codebook(None) == E_NULL


def test_packed_size(L):
    assert L.tq4_packed_size(8192, 2688) == 13762560
    assert L.tq4_packed_size(512, 256) == 81920
    assert L.tq4_packed_size(3, 33) == 0
    assert L.tq4_packed_size(-1, 32) == 0
    assert L.tq4_packed_size(0, 64) == 0


def test_pack_argument_errors(L):
    assert L.tq4_pack(FAKE, 4, 33, 0, FAKE, None, None) == E_SHAPE
    assert L.tq4_pack(FAKE, -1, 32, 0, FAKE, None, None) == E_SHAPE
    assert L.tq4_pack(None, 4, 32, 0, FAKE, None, None) == E_NULL
    assert L.tq4_pack(FAKE, 4, 32, 0, None, None, None) == E_NULL
    assert L.tq4_pack(FAKE + 4, 4, 32, 0, FAKE, None, None) == E_ALIGN
    assert L.tq4_pack(FAKE, 4, 32, 0, FAKE + 1, None, None) == E_ALIGN
    assert L.tq4_pack(FAKE, 4, 32, 0, FAKE, FAKE + 2, None) == E_ALIGN
    assert L.tq4_pack(None, 0, 32, 0, None, None, None) == OK      # empty: no-op


def test_pack_bf16_argument_errors(L):
    assert L.tq4_pack_bf16(FAKE, 4, 33, 0, FAKE, None, None) == E_SHAPE
    assert L.tq4_pack_bf16(FAKE, -1, 32, 0, FAKE, None, None) == E_SHAPE
    assert L.tq4_pack_bf16(FAKE, 0, 32, 0, None, None, None) == OK
    assert L.tq4_pack_bf16(None, 4, 32, 0, FAKE, None, None) == E_NULL
    assert L.tq4_pack_bf16(FAKE, 4, 32, 0, None, None, None) == E_NULL
    assert L.tq4_pack_bf16(FAKE + 8, 4, 32, 0, FAKE, None, None) == E_ALIGN
    assert L.tq4_pack_bf16(FAKE, 4, 32, 0, FAKE + 2, None, None) == E_ALIGN


def test_act_rht_argument_errors(L):
    assert L.tq4_act_rht(FAKE, 4, 40, 0, FAKE, None) == E_SHAPE
    assert L.tq4_act_rht(None, 4, 32, 0, FAKE, None) == E_NULL
    assert L.tq4_act_rht(MIS, 4, 32, 0, FAKE, None) == E_ALIGN
    assert L.tq4_act_rht(None, 0, 32, 0, None, None) == OK


def test_linear_argument_errors(L):
    ws = L.tq4_linear_workspace_size(100, 2688, 8192)
    assert ws >= 100 * 2688 * 2                      # room for the rotated activations
    assert L.tq4_linear_workspace_size(16, 33, 8) == 0
    args = dict(x=FAKE, m=100, k=2688, p=FAKE, n=8192, sb=0, y=FAKE, ws=FAKE, wsb=ws)

    def call(**kw):
        a = dict(args, **kw)
        return L.tq4_linear(a["x"], a["m"], a["k"], a["p"], a["n"], a["sb"], a["y"], a["ws"],
                            a["wsb"], None)

    assert call(k=2690) == E_SHAPE
    assert call(m=-1) == E_SHAPE
    assert call(x=None) == E_NULL
    assert call(p=None) == E_NULL
    assert call(y=None) == E_NULL
    assert call(x=MIS) == E_ALIGN
    assert call(p=FAKE + 2) == E_ALIGN
    assert call(y=FAKE + 2) == E_ALIGN
    assert call(ws=None) == E_WS
    assert call(wsb=ws - 1) == E_WS
    assert call(ws=FAKE + 16) == E_ALIGN
    assert call(m=0) == OK and call(n=0) == OK      # empty output: no-op


def test_linear_noalloc_argument_errors(L):
    """tq4_linear_noalloc rejects bad arguments and sizes beyond its static
    scratch before any device call (these run without a GPU)."""
    E_TOO_LARGE = 6
    assert L.tq4_status_string(E_TOO_LARGE) != b"unknown status"
    args = dict(x=FAKE, m=100, k=2688, p=FAKE, n=8192, sb=0, y=FAKE)

    def call(**kw):
        a = dict(args, **kw)
        return L.tq4_linear_noalloc(a["x"], a["m"], a["k"], a["p"], a["n"], a["sb"], a["y"],
                                    None)

    assert call(k=2690) == E_SHAPE
    assert call(m=-1) == E_SHAPE
    assert call(x=None) == E_NULL
    assert call(p=None) == E_NULL
    assert call(y=None) == E_NULL
    assert call(x=MIS) == E_ALIGN
    assert call(y=FAKE + 2) == E_ALIGN
    assert call(m=0) == OK and call(n=0) == OK      # empty output: no-op
    # 8192 x 4096 rotated activations alone are 64 MiB, beyond the 32 MiB scratch
    assert L.tq4_linear_workspace_size(8192, 4096, 64) > (32 << 20)
    assert call(m=8192, k=4096, n=64) == E_TOO_LARGE
    # M=4096 at K=2688 (256 x 256 tiles, no split) fits
    assert L.tq4_linear_workspace_size(4096, 2688, 8192) <= (32 << 20)


def test_linear_variant_argument_errors(L):
    def call(variant, **kw):
        a = dict(x=FAKE, m=16, k=2688, p=FAKE, n=8192, y=FAKE)
        a.update(kw)
        return L.tq4_linear_variant(a["x"], a["m"], a["k"], a["p"], a["n"], 0, a["y"], None, 0,
                                    variant, None)

    assert call(7) == E_SHAPE                        # no such variant
    assert call(-1) == E_SHAPE
    for v in (1, 2):
        assert call(v, k=2690) == E_SHAPE
        assert call(v, x=None) == E_NULL
        assert call(v, y=None) == E_NULL
        assert call(v, x=MIS) == E_ALIGN
        assert call(v, m=0) == OK


def test_linear_epilogue_argument_errors(L):
    ws = L.tq4_linear_workspace_size(100, 2688, 8192)
    y = FAKE
    args = dict(x=FAKE, m=100, k=2688, p=FAKE, n=8192, sb=0, b=FAKE, r=FAKE + (1 << 24), y=y,
                ws=FAKE, wsb=ws)

    def call(**kw):
        a = dict(args, **kw)
        return L.tq4_linear_epilogue(a["x"], a["m"], a["k"], a["p"], a["n"], a["sb"], a["b"],
                                     a["r"], a["y"], a["ws"], a["wsb"], None)

    assert call(k=2690) == E_SHAPE
    assert call(x=None) == E_NULL
    assert call(y=None) == E_NULL
    assert call(b=FAKE + 2) == E_ALIGN
    assert call(r=FAKE + (1 << 24) + 2) == E_ALIGN
    # a residual that overlaps y without being y (y spans 100 * 8192 * 4 bytes)
    assert call(r=y + 4) == E_SHAPE
    assert call(r=y + 100 * 8192 * 4 - 4) == E_SHAPE
    assert call(ws=None) == E_WS                     # r == y and disjoint r are accepted
    assert call(r=y, ws=None) == E_WS
    assert call(r=y + 100 * 8192 * 4, ws=None) == E_WS
    assert call(b=None, r=None, ws=None) == E_WS
    assert call(m=0) == OK and call(n=0) == OK


def test_linear_epilogue_bf16_argument_errors(L):
    ws = L.tq4_linear_workspace_size(100, 2688, 8192)
    y = FAKE
    args = dict(x=FAKE, m=100, k=2688, p=FAKE, n=8192, sb=0, b=FAKE, r=FAKE + (1 << 24), y=y,
                ws=FAKE, wsb=ws)

    def call(**kw):
        a = dict(args, **kw)
        return L.tq4_linear_epilogue_bf16(a["x"], a["m"], a["k"], a["p"], a["n"], a["sb"],
                                          a["b"], a["r"], a["y"], a["ws"], a["wsb"], None)

    assert call(y=None) == E_NULL
    assert call(y=FAKE + 1) == E_ALIGN
    assert call(r=FAKE + (1 << 24) + 1) == E_ALIGN
    assert call(b=FAKE + 2) == E_ALIGN
    # bf16 arrays are 2-byte aligned and span 100 * 8192 * 2 bytes
    assert call(y=FAKE + 2, r=FAKE + 2 + 100 * 8192 * 2, ws=None) == E_WS
    assert call(r=y + 2) == E_SHAPE
    assert call(r=y + 100 * 8192 * 2 - 2) == E_SHAPE
    assert call(r=y + 100 * 8192 * 2, ws=None) == E_WS
    assert call(r=y, ws=None) == E_WS
    assert call(m=0) == OK


def test_fp8_argument_errors(L):
    # sizes: codes n * kp then scale bytes n * kp / 32, kp = k rounded up to 128
    assert L.tq4_fp8_cache_size(8192, 2688) == 8192 * 2688 + 8192 * 84
    assert L.tq4_fp8_cache_size(10, 96) == 10 * 128 + 10 * 4
    assert L.tq4_fp8_cache_size(10, 33) == 0 and L.tq4_fp8_cache_size(-1, 64) == 0
    assert L.tq4_linear_fp8_workspace_size(16, 2688, 8192) >= 16 * 2688 + 16 * 84
    assert L.tq4_linear_fp8_workspace_size(0, 2688, 8192) == 0
    assert L.tq4_fp8_cache(FAKE, 8, 96, 0, None, None) == E_NULL
    assert L.tq4_fp8_cache(None, 8, 96, 0, FAKE, None) == E_NULL
    assert L.tq4_fp8_cache(FAKE, 8, 95, 0, FAKE, None) == E_SHAPE
    assert L.tq4_fp8_cache(FAKE + 2, 8, 96, 0, FAKE, None) == E_ALIGN
    assert L.tq4_fp8_cache(FAKE, 8, 96, 0, FAKE + 4, None) == E_ALIGN
    assert L.tq4_fp8_cache(FAKE, 0, 96, 0, None, None) == OK
    assert L.tq4_act_mxfp8(FAKE, 4, 64, FAKE, None, None) == E_NULL
    assert L.tq4_act_mxfp8(FAKE + 2, 4, 64, FAKE, FAKE, None) == E_ALIGN
    assert L.tq4_act_mxfp8(FAKE, 4, 64, FAKE + 8, FAKE, None) == E_ALIGN
    assert L.tq4_act_mxfp8(FAKE, 4, 48, FAKE, FAKE, None) == E_SHAPE
    ws = L.tq4_linear_fp8_workspace_size(100, 2688, 8192)

    def call(**kw):
        a = dict(dict(x=FAKE, m=100, k=2688, c=FAKE, n=8192, y=FAKE, ws=FAKE, wsb=ws), **kw)
        return L.tq4_linear_fp8(a["x"], a["m"], a["k"], a["c"], a["n"], a["y"], a["ws"],
                                a["wsb"], None)

    assert call(k=2690) == E_SHAPE
    assert call(m=-1) == E_SHAPE
    assert call(x=None) == E_NULL
    assert call(c=None) == E_NULL
    assert call(y=None) == E_NULL
    assert call(x=MIS) == E_ALIGN
    assert call(c=FAKE + 4) == E_ALIGN
    assert call(y=FAKE + 2) == E_ALIGN
    assert call(ws=None) == E_WS
    assert call(wsb=ws - 1) == E_WS
    assert call(ws=FAKE + 16) == E_ALIGN
    assert call(m=0) == OK and call(n=0) == OK
    q = L.tq4_linear_fp8_quantized
    assert q(FAKE, FAKE, 100, 2688, FAKE, 8192, None, None) == E_NULL
    assert q(None, FAKE, 100, 2688, FAKE, 8192, FAKE, None) == E_NULL
    assert q(FAKE, FAKE + 2, 100, 2688, FAKE, 8192, FAKE, None) == E_ALIGN
    assert q(FAKE + 8, FAKE, 100, 2688, FAKE, 8192, FAKE, None) == E_ALIGN
    assert q(FAKE, FAKE, 100, 2690, FAKE, 8192, FAKE, None) == E_SHAPE


def test_moe_block_argument_errors(L):
    ws = L.tq4_moe_block_workspace_size(16, 6, 128, 1856, 2688)
    assert ws > L.tq4_moe_workspace_size(16, 6, 128, 1856, 2688)
    assert L.tq4_moe_block_workspace_size(16, 6, 128, 1850, 2688) == 0

    def call(**kw):
        a = dict(dict(x=FAKE, t=16, k=2688, lg=FAKE, e=128, topk=6, w1=FAKE, n1=1856, w2=FAKE,
                      out=FAKE, ws=FAKE, wsb=ws), **kw)
        return L.tq4_moe_block(a["x"], a["t"], a["k"], a["lg"], a["e"], a["topk"], a["w1"],
                               a["n1"], a["w2"], 0, a["out"], a["ws"], a["wsb"], None)

    assert call(topk=129) == E_SHAPE
    assert call(e=513) == E_SHAPE
    assert call(n1=1850) == E_SHAPE
    assert call(lg=None) == E_NULL
    assert call(w1=None) == E_NULL
    assert call(lg=FAKE + 2) == E_ALIGN
    assert call(x=MIS) == E_ALIGN
    assert call(ws=None) == E_WS
    assert call(wsb=ws - 1) == E_WS
    assert call(t=0) == OK


def test_moe_block_persistent_argument_errors(L):
    ws = L.tq4_moe_block_persistent_workspace_size(16, 6, 128, 1856, 2688)
    assert ws > L.tq4_moe_block_workspace_size(16, 6, 128, 1856, 2688)
    # 16-row tiles only: t * topk <= 16 * n_experts
    assert L.tq4_moe_block_persistent_workspace_size(341, 6, 128, 1856, 2688) > 0
    assert L.tq4_moe_block_persistent_workspace_size(342, 6, 128, 1856, 2688) == 0
    assert L.tq4_moe_block_persistent_workspace_size(16, 6, 128, 1850, 2688) == 0

    def call(**kw):
        a = dict(dict(x=FAKE, t=16, k=2688, lg=FAKE, e=128, topk=6, w1=FAKE, n1=1856, w2=FAKE,
                      out=FAKE, ws=FAKE, wsb=ws), **kw)
        return L.tq4_moe_block_persistent(a["x"], a["t"], a["k"], a["lg"], a["e"], a["topk"],
                                          a["w1"], a["n1"], a["w2"], 0, a["out"], a["ws"],
                                          a["wsb"], None)

    assert call(t=342) == E_SHAPE
    assert call(topk=129) == E_SHAPE
    assert call(e=513) == E_SHAPE
    assert call(n1=1850) == E_SHAPE
    assert call(lg=None) == E_NULL
    assert call(w2=None) == E_NULL
    assert call(lg=FAKE + 2) == E_ALIGN
    assert call(out=MIS) == E_ALIGN
    assert call(ws=None) == E_WS
    assert call(wsb=ws - 1) == E_WS
    assert call(t=0) == OK


def test_moe_grouped_fp8_argument_errors(L):
    ws = L.tq4_moe_grouped_fp8_workspace_size(16, 6, 128, 1856, 2688)
    # route lists, 16-row tiles, xq/xs (kp 2688), hq/hs (n1p 1920), fp32 o
    assert ws >= 16 * 2688 * 33 // 32 + 96 * 1920 * 33 // 32 + 96 * 2688 * 4
    assert L.tq4_moe_grouped_fp8_workspace_size(16, 6, 128, 1850, 2688) == 0   # n1 % 32
    assert L.tq4_moe_grouped_fp8_workspace_size(16, 7, 4, 64, 64) == 0         # topk > E
    assert L.tq4_moe_grouped_fp8_workspace_size(1 << 20, 6, 128, 1856, 2688) == 0  # t * kp

    def call(**kw):
        a = dict(dict(x=FAKE, t=16, k=2688, ids=FAKE, g=FAKE, topk=6, e=128, w1=FAKE, n1=1856,
                      w2=FAKE, out=FAKE, ws=FAKE, wsb=ws), **kw)
        return L.tq4_moe_grouped_fp8(a["x"], a["t"], a["k"], a["ids"], a["g"], a["topk"], a["e"],
                                     a["w1"], a["n1"], a["w2"], a["out"], a["ws"], a["wsb"], None)

    assert call(topk=129) == E_SHAPE
    assert call(e=513) == E_SHAPE
    assert call(n1=1850) == E_SHAPE
    assert call(k=2690) == E_SHAPE
    assert call(ids=None) == E_NULL
    assert call(w2=None) == E_NULL
    assert call(out=None) == E_NULL
    assert call(g=FAKE + 2) == E_ALIGN
    assert call(w1=FAKE + 4) == E_ALIGN
    assert call(x=MIS) == E_ALIGN
    assert call(ws=None) == E_WS
    assert call(wsb=ws - 1) == E_WS
    assert call(ws=FAKE + 16) == E_ALIGN
    assert call(t=0) == OK


def test_moe_argument_errors(L):
    ws = L.tq4_moe_workspace_size(16, 6, 128, 1856, 2688)
    assert ws > 0
    assert L.tq4_moe_workspace_size(16, 6, 128, 1850, 2688) == 0     # n1 % 32
    assert L.tq4_moe_workspace_size(16, 7, 4, 64, 64) == 0           # topk > E
    assert L.tq4_moe_workspace_size(16, 6, 513, 64, 64) == 0         # E too large
    a = [FAKE, 16, 2688, FAKE, FAKE, 6, 128, FAKE, 1856, FAKE, 0, FAKE, FAKE, ws, None]

    def call(i=None, v=None):
        b = list(a)
        if i is not None:
            b[i] = v
        return L.tq4_moe_grouped(*b)

    assert call(2, 2689) == E_SHAPE
    assert call(5, 0) == E_SHAPE
    assert call(0, None) == E_NULL
    assert call(3, None) == E_NULL
    assert call(7, None) == E_NULL
    assert call(0, MIS) == E_ALIGN
    assert call(11, FAKE + 4) == E_ALIGN
    assert call(12, None) == E_WS
    assert call(13, ws - 1) == E_WS
    assert call(1, 0) == OK                                           # t == 0: no-op


def test_route_argument_errors(L):
    assert L.tq4_moe_route(FAKE, 4, 0, 8, FAKE, FAKE, FAKE, FAKE, None) == E_SHAPE
    assert L.tq4_moe_route(FAKE, 4, 2, 600, FAKE, FAKE, FAKE, FAKE, None) == E_SHAPE
    assert L.tq4_moe_route(FAKE, 4, 2, 8, None, FAKE, FAKE, FAKE, None) == E_NULL
    assert L.tq4_moe_route(None, 4, 2, 8, FAKE, FAKE, FAKE, FAKE, None) == E_NULL
    assert L.tq4_moe_route(FAKE, 4, 2, 8, FAKE, FAKE + 1, FAKE, FAKE, None) == E_ALIGN


def test_router_argument_errors(L):
    assert L.tq4_moe_router(FAKE, -1, 128, 6, FAKE, FAKE, None) == E_SHAPE
    assert L.tq4_moe_router(FAKE, 4, 0, 1, FAKE, FAKE, None) == E_SHAPE
    assert L.tq4_moe_router(FAKE, 4, 513, 6, FAKE, FAKE, None) == E_SHAPE
    assert L.tq4_moe_router(FAKE, 4, 128, 0, FAKE, FAKE, None) == E_SHAPE
    assert L.tq4_moe_router(FAKE, 4, 8, 9, FAKE, FAKE, None) == E_SHAPE
    assert L.tq4_moe_router(None, 0, 128, 6, None, None, None) == OK
    assert L.tq4_moe_router(None, 4, 128, 6, FAKE, FAKE, None) == E_NULL
    assert L.tq4_moe_router(FAKE, 4, 128, 6, None, FAKE, None) == E_NULL
    assert L.tq4_moe_router(FAKE, 4, 128, 6, FAKE, None, None) == E_NULL
    assert L.tq4_moe_router(FAKE + 2, 4, 128, 6, FAKE, FAKE, None) == E_ALIGN


def test_read_probe_argument_errors(L):
    assert L.tq4_read_probe(FAKE, 40, FAKE, None) == E_SHAPE
    assert L.tq4_read_probe(FAKE, -16, FAKE, None) == E_SHAPE
    assert L.tq4_read_probe(FAKE, 0, None, None) == OK      # empty: nothing to check
    assert L.tq4_read_probe(None, 64, FAKE, None) == E_NULL
    assert L.tq4_read_probe(FAKE, 64, None, None) == E_NULL
    assert L.tq4_read_probe(FAKE + 8, 64, FAKE, None) == E_ALIGN


def test_binding_refuses_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        _lib.lib()
