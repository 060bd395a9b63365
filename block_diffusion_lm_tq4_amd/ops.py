"""Torch-facing binding of the TQ4_1S C ABI: argument marshalling only.

Every function takes device tensors, checks dtypes and shapes, and passes raw
pointers, sizes and the current HIP stream to libtq4.so.  All arithmetic runs
in the library's kernels; torch only provides memory and streams.
"""

from __future__ import annotations

import torch

from ._lib import check, lib

BLOCK = 32
BLOCK_BYTES = 20


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _cuda_contig(t: torch.Tensor, name: str, dtype) -> None:
    _require(t.is_cuda, f"{name} must be a device tensor")
    _require(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _require(t.is_contiguous(), f"{name} must be contiguous")


class Workspace:
    """Grow-only, zero-initialised device scratch buffers, one per (device, purpose)."""

    def __init__(self):
        self._bufs: dict = {}

    def get(self, device: torch.device, key: str, nbytes: int) -> torch.Tensor:
        k = (str(device), key)
        buf = self._bufs.get(k)
        if buf is None or buf.numel() < nbytes:
            buf = torch.zeros(max(nbytes, 1024), dtype=torch.uint8, device=device)
            self._bufs[k] = buf
        return buf


_WS = Workspace()


def codebook() -> torch.Tensor:
    """The 16 stored levels (fp32, CPU tensor), as the library computes them."""
    out = torch.empty(16, dtype=torch.float32)
    check("tq4_codebook", lib().tq4_codebook(out.data_ptr()))
    return out


def packed_size(n: int, k: int) -> int:
    return int(lib().tq4_packed_size(n, k))


def pack(w: torch.Tensor, sign_bits: int, nonfinite: torch.Tensor | None = None,
         out: torch.Tensor | None = None) -> torch.Tensor:
    """fp32 or bf16 W [n, k] -> packed uint8 [n, k/32, 20] (tq4_pack / tq4_pack_bf16)."""
    _require(w.dtype in (torch.float32, torch.bfloat16), "w must be fp32 or bf16")
    _cuda_contig(w, "w", w.dtype)
    _require(w.dim() == 2 and w.shape[1] % BLOCK == 0, "w must be [n, k] with k % 32 == 0")
    n, k = w.shape
    if out is None:
        out = torch.empty((n, k // BLOCK, BLOCK_BYTES), dtype=torch.uint8, device=w.device)
    _cuda_contig(out, "out", torch.uint8)
    _require(out.numel() == n * (k // BLOCK) * BLOCK_BYTES, "out must hold n * k/32 * 20 bytes")
    if nonfinite is not None:
        _cuda_contig(nonfinite, "nonfinite", torch.int32)
    fn = "tq4_pack" if w.dtype == torch.float32 else "tq4_pack_bf16"
    check(fn, getattr(lib(), fn)(w.data_ptr(), n, k, sign_bits & 0xFFFFFFFF, out.data_ptr(),
                                 _ptr(nonfinite), _stream(w.device)))
    return out


def act_rht(x: torch.Tensor, sign_bits: int) -> torch.Tensor:
    """bf16 x [m, k] -> fp16 R x per 32-block (tq4_act_rht)."""
    _cuda_contig(x, "x", torch.bfloat16)
    m, k = x.shape
    out = torch.empty((m, k), dtype=torch.float16, device=x.device)
    check("tq4_act_rht", lib().tq4_act_rht(x.data_ptr(), m, k, sign_bits & 0xFFFFFFFF,
                                           out.data_ptr(), _stream(x.device)))
    return out


def linear_workspace_size(m: int, k: int, n: int) -> int:
    return int(lib().tq4_linear_workspace_size(m, k, n))


def linear(x: torch.Tensor, packed: torch.Tensor, sign_bits: int,
           out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y = x . W_hat^T, fp32 [m, n] (tq4_linear)."""
    _cuda_contig(x, "x", torch.bfloat16)
    _cuda_contig(packed, "packed", torch.uint8)
    _require(x.dim() == 2, "x must be [m, k]")
    m, k = x.shape
    _require(packed.dim() == 3 and packed.shape[1] * BLOCK == k and packed.shape[2] == BLOCK_BYTES,
             "packed must be [n, k/32, 20]")
    n = packed.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _cuda_contig(out, "out", torch.float32)
    _require(tuple(out.shape) == (m, n), "out must be [m, n]")
    need = linear_workspace_size(m, k, n)
    if workspace is None:
        workspace = _WS.get(x.device, "linear", need)
    check("tq4_linear", lib().tq4_linear(x.data_ptr(), m, k, packed.data_ptr(), n,
                                         sign_bits & 0xFFFFFFFF, out.data_ptr(),
                                         workspace.data_ptr(), workspace.numel(),
                                         _stream(x.device)))
    return out


def _linear_tail(fn: str, x, packed, sign_bits, bias, residual, out, workspace, ydtype):
    _cuda_contig(x, "x", torch.bfloat16)
    _cuda_contig(packed, "packed", torch.uint8)
    _require(x.dim() == 2, "x must be [m, k]")
    m, k = x.shape
    _require(packed.dim() == 3 and packed.shape[1] * BLOCK == k and packed.shape[2] == BLOCK_BYTES,
             "packed must be [n, k/32, 20]")
    n = packed.shape[0]
    if bias is not None:
        _cuda_contig(bias, "bias", torch.float32)
        _require(tuple(bias.shape) == (n,), "bias must be [n]")
    if residual is not None:
        _cuda_contig(residual, "residual", ydtype)
        _require(tuple(residual.shape) == (m, n), "residual must be [m, n]")
    if out is None:
        out = torch.empty((m, n), dtype=ydtype, device=x.device)
    _cuda_contig(out, "out", ydtype)
    _require(tuple(out.shape) == (m, n), "out must be [m, n]")
    need = linear_workspace_size(m, k, n)
    if workspace is None:
        workspace = _WS.get(x.device, "linear", need)
    check(fn, getattr(lib(), fn)(x.data_ptr(), m, k, packed.data_ptr(), n, sign_bits & 0xFFFFFFFF,
                                 _ptr(bias), _ptr(residual), out.data_ptr(), workspace.data_ptr(),
                                 workspace.numel(), _stream(x.device)))
    return out


def linear_epilogue(x: torch.Tensor, packed: torch.Tensor, sign_bits: int,
                    bias: torch.Tensor | None = None, residual: torch.Tensor | None = None,
                    out: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y = x . W_hat^T + bias + residual, fp32 [m, n] (tq4_linear_epilogue).

    bias is fp32 [n] or None; residual is fp32 [m, n] or None and may be `out`
    itself (the sum is then taken in place)."""
    return _linear_tail("tq4_linear_epilogue", x, packed, sign_bits, bias, residual, out,
                        workspace, torch.float32)


def linear_epilogue_bf16(x: torch.Tensor, packed: torch.Tensor, sign_bits: int,
                         bias: torch.Tensor | None = None, residual: torch.Tensor | None = None,
                         out: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None) -> torch.Tensor:
    """bf16(x . W_hat^T + bias + residual), bf16 [m, n] (tq4_linear_epilogue_bf16).

    bias is fp32 [n] or None; residual is bf16 [m, n] or None and may be `out`
    itself.  The sum is formed in fp32 and rounded once."""
    return _linear_tail("tq4_linear_epilogue_bf16", x, packed, sign_bits, bias, residual, out,
                        workspace, torch.bfloat16)


def fp8_padded_k(k: int) -> int:
    return (k + 127) // 128 * 128


def fp8_cache(packed: torch.Tensor, sign_bits: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """packed [n, k/32, 20] -> the fp8 weight cache (flat uint8: codes [n][kp],
    then scale bytes [n][kp/32]) (tq4_fp8_cache)."""
    _cuda_contig(packed, "packed", torch.uint8)
    _require(packed.dim() == 3 and packed.shape[2] == BLOCK_BYTES, "packed must be [n, k/32, 20]")
    n, k = packed.shape[0], packed.shape[1] * BLOCK
    size = int(lib().tq4_fp8_cache_size(n, k))
    if out is None:
        out = torch.empty(max(size, 16), dtype=torch.uint8, device=packed.device)
    _cuda_contig(out, "out", torch.uint8)
    _require(out.numel() >= size, "out is smaller than tq4_fp8_cache_size(n, k)")
    check("tq4_fp8_cache", lib().tq4_fp8_cache(packed.data_ptr(), n, k, sign_bits & 0xFFFFFFFF,
                                               out.data_ptr(), _stream(packed.device)))
    return out


def fp8_cache_views(cache: torch.Tensor, n: int, k: int) -> tuple[torch.Tensor, torch.Tensor]:
    """(codes [n, kp], scales [n, kp/32]) views of a flat cache."""
    kp = fp8_padded_k(k)
    return cache[:n * kp].view(n, kp), cache[n * kp:n * kp + n * kp // 32].view(n, kp // 32)


def linear_fp8_workspace_size(m: int, k: int, n: int) -> int:
    return int(lib().tq4_linear_fp8_workspace_size(m, k, n))


def act_mxfp8(x: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """bf16 x [m, k] -> (codes [m, kp], scales [m, kp/32]) uint8 (tq4_act_mxfp8)."""
    _cuda_contig(x, "x", torch.bfloat16)
    m, k = x.shape
    kp = fp8_padded_k(k)
    codes = torch.empty((m, kp), dtype=torch.uint8, device=x.device)
    scales = torch.empty((m, kp // 32), dtype=torch.uint8, device=x.device)
    check("tq4_act_mxfp8", lib().tq4_act_mxfp8(x.data_ptr(), m, k, codes.data_ptr(),
                                               scales.data_ptr(), _stream(x.device)))
    return codes, scales


def linear_fp8(x: torch.Tensor, cache: torch.Tensor, n: int, out: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y = x . W^T from the fp8 cache of an [n, k] matrix, fp32 [m, n] (tq4_linear_fp8)."""
    _cuda_contig(x, "x", torch.bfloat16)
    _cuda_contig(cache, "cache", torch.uint8)
    _require(x.dim() == 2, "x must be [m, k]")
    m, k = x.shape
    _require(cache.numel() >= int(lib().tq4_fp8_cache_size(n, k)), "cache too small for [n, k]")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _cuda_contig(out, "out", torch.float32)
    _require(tuple(out.shape) == (m, n), "out must be [m, n]")
    need = int(lib().tq4_linear_fp8_workspace_size(m, k, n))
    if workspace is None:
        workspace = _WS.get(x.device, "linear_fp8", need)
    check("tq4_linear_fp8", lib().tq4_linear_fp8(x.data_ptr(), m, k, cache.data_ptr(), n,
                                                 out.data_ptr(), workspace.data_ptr(),
                                                 workspace.numel(), _stream(x.device)))
    return out


def linear_fp8_quantized(x_codes: torch.Tensor, x_scales: torch.Tensor, k: int,
                         cache: torch.Tensor, n: int,
                         out: torch.Tensor | None = None) -> torch.Tensor:
    """y from activations already quantized by act_mxfp8 (tq4_linear_fp8_quantized)."""
    _cuda_contig(x_codes, "x_codes", torch.uint8)
    _cuda_contig(x_scales, "x_scales", torch.uint8)
    _cuda_contig(cache, "cache", torch.uint8)
    m = x_codes.shape[0]
    kp = fp8_padded_k(k)
    _require(tuple(x_codes.shape) == (m, kp) and tuple(x_scales.shape) == (m, kp // 32),
             "x_codes must be [m, kp] and x_scales [m, kp/32]")
    _require(cache.numel() >= int(lib().tq4_fp8_cache_size(n, k)), "cache too small for [n, k]")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x_codes.device)
    _cuda_contig(out, "out", torch.float32)
    _require(tuple(out.shape) == (m, n), "out must be [m, n]")
    check("tq4_linear_fp8_quantized",
          lib().tq4_linear_fp8_quantized(x_codes.data_ptr(), x_scales.data_ptr(), m, k,
                                         cache.data_ptr(), n, out.data_ptr(),
                                         _stream(x_codes.device)))
    return out


VARIANTS = {"default": 0, "weight_rotation": 1, "valu_product": 2}


def linear_variant(x: torch.Tensor, packed: torch.Tensor, sign_bits: int, variant: str,
                   out: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None) -> torch.Tensor:
    """The layer with another rotation placement or product arithmetic
    (tq4_linear_variant): "default", "weight_rotation" or "valu_product"."""
    _cuda_contig(x, "x", torch.bfloat16)
    _cuda_contig(packed, "packed", torch.uint8)
    m, k = x.shape
    n = packed.shape[0]
    _require(packed.dim() == 3 and packed.shape[1] * BLOCK == k and packed.shape[2] == BLOCK_BYTES,
             "packed must be [n, k/32, 20]")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _cuda_contig(out, "out", torch.float32)
    need = max(linear_workspace_size(m, k, n), m * k * 2)
    if workspace is None:
        workspace = _WS.get(x.device, "linear", need)
    check("tq4_linear_variant", lib().tq4_linear_variant(
        x.data_ptr(), m, k, packed.data_ptr(), n, sign_bits & 0xFFFFFFFF, out.data_ptr(),
        workspace.data_ptr(), workspace.numel(), VARIANTS[variant], _stream(x.device)))
    return out


def linear_noalloc(x: torch.Tensor, packed: torch.Tensor, sign_bits: int,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """tq4_linear on the library's static scratch, no workspace (tq4_linear_noalloc)."""
    _cuda_contig(x, "x", torch.bfloat16)
    _cuda_contig(packed, "packed", torch.uint8)
    m, k = x.shape
    n = packed.shape[0]
    _require(packed.dim() == 3 and packed.shape[1] * BLOCK == k and packed.shape[2] == BLOCK_BYTES,
             "packed must be [n, k/32, 20]")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _cuda_contig(out, "out", torch.float32)
    _require(tuple(out.shape) == (m, n), "out must be [m, n]")
    check("tq4_linear_noalloc", lib().tq4_linear_noalloc(
        x.data_ptr(), m, k, packed.data_ptr(), n, sign_bits & 0xFFFFFFFF, out.data_ptr(),
        _stream(x.device)))
    return out


def linear_rotated(xt: torch.Tensor, packed: torch.Tensor, out: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y = xt . Z_hat^T with xt = act_rht(x) already rotated (tq4_linear_rotated)."""
    _cuda_contig(xt, "xt", torch.float16)
    _cuda_contig(packed, "packed", torch.uint8)
    m, k = xt.shape
    _require(packed.dim() == 3 and packed.shape[1] * BLOCK == k and packed.shape[2] == BLOCK_BYTES,
             "packed must be [n, k/32, 20]")
    n = packed.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=xt.device)
    _cuda_contig(out, "out", torch.float32)
    _require(tuple(out.shape) == (m, n), "out must be [m, n]")
    need = linear_workspace_size(m, k, n)
    if workspace is None:
        workspace = _WS.get(xt.device, "linear", need)
    check("tq4_linear_rotated", lib().tq4_linear_rotated(
        xt.data_ptr(), m, k, packed.data_ptr(), n, out.data_ptr(), workspace.data_ptr(),
        workspace.numel(), _stream(xt.device)))
    return out


def moe_route(topk_ids: torch.Tensor, n_experts: int):
    """Stable bucketing of (token, slot) pairs by expert (tq4_moe_route)."""
    _cuda_contig(topk_ids, "topk_ids", torch.int32)
    t, topk = topk_ids.shape
    dev = topk_ids.device
    counts = torch.empty(n_experts, dtype=torch.int32, device=dev)
    offsets = torch.empty(n_experts + 1, dtype=torch.int32, device=dev)
    perm = torch.full((t * topk,), -7, dtype=torch.int32, device=dev)
    inv = torch.empty(t * topk, dtype=torch.int32, device=dev)
    check("tq4_moe_route", lib().tq4_moe_route(topk_ids.data_ptr(), t, topk, n_experts,
                                               counts.data_ptr(), offsets.data_ptr(),
                                               perm.data_ptr(), inv.data_ptr(), _stream(dev)))
    return counts, offsets, perm, inv


def moe_router(logits: torch.Tensor, topk: int,
               ids: torch.Tensor | None = None, gates: torch.Tensor | None = None):
    """Router of the MoE layer (tq4_moe_router): (ids int32 [t, topk], gates fp32 [t, topk])."""
    _cuda_contig(logits, "logits", torch.float32)
    _require(logits.dim() == 2, "logits must be [t, n_experts]")
    t, e = logits.shape
    if ids is None:
        ids = torch.empty((t, topk), dtype=torch.int32, device=logits.device)
    if gates is None:
        gates = torch.empty((t, topk), dtype=torch.float32, device=logits.device)
    _cuda_contig(ids, "ids", torch.int32)
    _cuda_contig(gates, "gates", torch.float32)
    _require(tuple(ids.shape) == (t, topk) and tuple(gates.shape) == (t, topk),
             "ids and gates must be [t, topk]")
    check("tq4_moe_router", lib().tq4_moe_router(logits.data_ptr(), t, e, topk, ids.data_ptr(),
                                                 gates.data_ptr(), _stream(logits.device)))
    return ids, gates


def moe_workspace_size(t: int, topk: int, n_experts: int, n1: int, k: int) -> int:
    return int(lib().tq4_moe_workspace_size(t, topk, n_experts, n1, k))


def moe_grouped(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor,
                w1_packed: torch.Tensor, w2_packed: torch.Tensor, sign_bits: int,
                out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
    """The TQ4_1S MoE layer (tq4_moe_grouped); fp32 [t, k]."""
    _cuda_contig(x, "x", torch.bfloat16)
    _cuda_contig(topk_ids, "topk_ids", torch.int32)
    _cuda_contig(topk_w, "topk_w", torch.float32)
    _cuda_contig(w1_packed, "w1_packed", torch.uint8)
    _cuda_contig(w2_packed, "w2_packed", torch.uint8)
    t, k = x.shape
    _require(topk_ids.dim() == 2 and topk_ids.shape[0] == t, "topk_ids must be [t, topk]")
    topk = topk_ids.shape[1]
    _require(tuple(topk_w.shape) == (t, topk), "topk_w must be [t, topk]")
    e, n1, kb1, bb = w1_packed.shape
    _require(kb1 * BLOCK == k and bb == BLOCK_BYTES, "w1_packed must be [E, n1, k/32, 20]")
    _require(tuple(w2_packed.shape) == (e, k, n1 // BLOCK, BLOCK_BYTES),
             "w2_packed must be [E, k, n1/32, 20]")
    if out is None:
        out = torch.empty((t, k), dtype=torch.float32, device=x.device)
    _cuda_contig(out, "out", torch.float32)
    need = moe_workspace_size(t, topk, e, n1, k)
    if workspace is None:
        workspace = _WS.get(x.device, "moe", need)
    check("tq4_moe_grouped", lib().tq4_moe_grouped(
        x.data_ptr(), t, k, topk_ids.data_ptr(), topk_w.data_ptr(), topk, e,
        w1_packed.data_ptr(), n1, w2_packed.data_ptr(), sign_bits & 0xFFFFFFFF,
        out.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(x.device)))
    return out


def fp8_cache_experts(packed: torch.Tensor, sign_bits: int) -> torch.Tensor:
    """Experts' packed weights [E, n, k/32, 20] -> the fp8 cache of the stacked
    [E * n, k] matrix (the layout tq4_moe_grouped_fp8 takes)."""
    _require(packed.dim() == 4, "packed must be [E, n, k/32, 20]")
    e, n, kb, bb = packed.shape
    return fp8_cache(packed.view(e * n, kb, bb), sign_bits)


def moe_grouped_fp8_workspace_size(t: int, topk: int, n_experts: int, n1: int, k: int) -> int:
    return int(lib().tq4_moe_grouped_fp8_workspace_size(t, topk, n_experts, n1, k))


def moe_grouped_fp8(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor,
                    w1_cache: torch.Tensor, w2_cache: torch.Tensor, n_experts: int, n1: int,
                    out: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None) -> torch.Tensor:
    """The MoE layer on fp8 expert caches (tq4_moe_grouped_fp8); fp32 [t, k]."""
    _cuda_contig(x, "x", torch.bfloat16)
    _cuda_contig(topk_ids, "topk_ids", torch.int32)
    _cuda_contig(topk_w, "topk_w", torch.float32)
    _cuda_contig(w1_cache, "w1_cache", torch.uint8)
    _cuda_contig(w2_cache, "w2_cache", torch.uint8)
    t, k = x.shape
    _require(topk_ids.dim() == 2 and topk_ids.shape[0] == t, "topk_ids must be [t, topk]")
    topk = topk_ids.shape[1]
    _require(tuple(topk_w.shape) == (t, topk), "topk_w must be [t, topk]")
    _require(w1_cache.numel() >= int(lib().tq4_fp8_cache_size(n_experts * n1, k)),
             "w1_cache too small for [E * n1, k]")
    _require(w2_cache.numel() >= int(lib().tq4_fp8_cache_size(n_experts * k, n1)),
             "w2_cache too small for [E * k, n1]")
    if out is None:
        out = torch.empty((t, k), dtype=torch.float32, device=x.device)
    _cuda_contig(out, "out", torch.float32)
    need = moe_grouped_fp8_workspace_size(t, topk, n_experts, n1, k)
    if workspace is None:
        workspace = _WS.get(x.device, "moe_fp8", need)
    check("tq4_moe_grouped_fp8", lib().tq4_moe_grouped_fp8(
        x.data_ptr(), t, k, topk_ids.data_ptr(), topk_w.data_ptr(), topk, n_experts,
        w1_cache.data_ptr(), n1, w2_cache.data_ptr(), out.data_ptr(), workspace.data_ptr(),
        workspace.numel(), _stream(x.device)))
    return out


def moe_block_workspace_size(t: int, topk: int, n_experts: int, n1: int, k: int) -> int:
    return int(lib().tq4_moe_block_workspace_size(t, topk, n_experts, n1, k))


def moe_block(x: torch.Tensor, logits: torch.Tensor, topk: int, w1_packed: torch.Tensor,
              w2_packed: torch.Tensor, sign_bits: int, out: torch.Tensor | None = None,
              workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Router logits [t, E] -> the MoE layer's output, fp32 [t, k] (tq4_moe_block)."""
    _cuda_contig(x, "x", torch.bfloat16)
    _cuda_contig(logits, "logits", torch.float32)
    _cuda_contig(w1_packed, "w1_packed", torch.uint8)
    _cuda_contig(w2_packed, "w2_packed", torch.uint8)
    t, k = x.shape
    e, n1, kb1, bb = w1_packed.shape
    _require(tuple(logits.shape) == (t, e), "logits must be [t, E]")
    _require(kb1 * BLOCK == k and bb == BLOCK_BYTES, "w1_packed must be [E, n1, k/32, 20]")
    _require(tuple(w2_packed.shape) == (e, k, n1 // BLOCK, BLOCK_BYTES),
             "w2_packed must be [E, k, n1/32, 20]")
    if out is None:
        out = torch.empty((t, k), dtype=torch.float32, device=x.device)
    _cuda_contig(out, "out", torch.float32)
    need = moe_block_workspace_size(t, topk, e, n1, k)
    if workspace is None:
        workspace = _WS.get(x.device, "moe_block", need)
    check("tq4_moe_block", lib().tq4_moe_block(
        x.data_ptr(), t, k, logits.data_ptr(), e, topk, w1_packed.data_ptr(), n1,
        w2_packed.data_ptr(), sign_bits & 0xFFFFFFFF, out.data_ptr(), workspace.data_ptr(),
        workspace.numel(), _stream(x.device)))
    return out


def moe_block_persistent_workspace_size(t: int, topk: int, n_experts: int, n1: int,
                                        k: int) -> int:
    return int(lib().tq4_moe_block_persistent_workspace_size(t, topk, n_experts, n1, k))


def moe_block_persistent(x: torch.Tensor, logits: torch.Tensor, topk: int,
                         w1_packed: torch.Tensor, w2_packed: torch.Tensor, sign_bits: int,
                         out: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None) -> torch.Tensor:
    """moe_block in one persistent launch (tq4_moe_block_persistent); 16-row tiles only."""
    _cuda_contig(x, "x", torch.bfloat16)
    _cuda_contig(logits, "logits", torch.float32)
    _cuda_contig(w1_packed, "w1_packed", torch.uint8)
    _cuda_contig(w2_packed, "w2_packed", torch.uint8)
    t, k = x.shape
    e, n1, kb1, bb = w1_packed.shape
    _require(tuple(logits.shape) == (t, e), "logits must be [t, E]")
    _require(kb1 * BLOCK == k and bb == BLOCK_BYTES, "w1_packed must be [E, n1, k/32, 20]")
    _require(tuple(w2_packed.shape) == (e, k, n1 // BLOCK, BLOCK_BYTES),
             "w2_packed must be [E, k, n1/32, 20]")
    if out is None:
        out = torch.empty((t, k), dtype=torch.float32, device=x.device)
    _cuda_contig(out, "out", torch.float32)
    need = moe_block_persistent_workspace_size(t, topk, e, n1, k)
    _require(need > 0, "sizes outside tq4_moe_block_persistent's range")
    if workspace is None:
        workspace = _WS.get(x.device, "moe_block_persistent", need)
    check("tq4_moe_block_persistent", lib().tq4_moe_block_persistent(
        x.data_ptr(), t, k, logits.data_ptr(), e, topk, w1_packed.data_ptr(), n1,
        w2_packed.data_ptr(), sign_bits & 0xFFFFFFFF, out.data_ptr(), workspace.data_ptr(),
        workspace.numel(), _stream(x.device)))
    return out


def read_probe(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """One streaming read of a whole device buffer (tq4_read_probe), for timing."""
    _require(buf.is_cuda and buf.is_contiguous(), "buf must be a contiguous device tensor")
    _cuda_contig(sink, "sink", torch.float32)
    _require(sink.numel() >= 256, "sink must hold 256 floats")
    nbytes = buf.numel() * buf.element_size()
    check("tq4_read_probe", lib().tq4_read_probe(buf.data_ptr(), nbytes, sink.data_ptr(),
                                                 _stream(buf.device)))
