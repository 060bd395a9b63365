// C ABI of the TQ4_1S library: argument validation, workspace layout and
// dispatch.  Every argument check happens before any HIP call, so invalid
// calls return without touching the GPU (and can be tested without one).
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/tq4.h"
#include "moe_block.h"
#include "tq4_internal.h"

namespace {

using tq4::DensePlan;
using tq4::MoEPlan;
using tq4::MoETile;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

int device_status(hipError_t e) { return e == hipSuccess ? TQ4_OK : TQ4_E_DEVICE; }

// ---- tq4_linear workspace ------------------------------------------------
// m <= 16: one fused kernel, no workspace.  Otherwise [xt fp16 m*k][split-K
// partial sums]; tq4_linear_rotated needs only the partial sums.
struct LinearLayout {
  size_t xt, partial, total;
};

LinearLayout linear_layout(int64_t m, int64_t k, int64_t n, bool rotated) {
  LinearLayout l{};
  if (!rotated && tq4::skinny_fits(m, k, n)) return l;
  const DensePlan p = tq4::plan_dense(m, k, n);
  l.xt = 0;
  l.partial = rotated ? 0 : align_up(static_cast<size_t>(m) * k * 2);
  l.total = l.partial + align_up(p.partial_bytes);
  return l;
}

int check_workspace(const void *ws, size_t bytes, size_t need) {
  if (need == 0) return TQ4_OK;
  if (ws == nullptr || bytes < need) return TQ4_E_WORKSPACE;
  if (!aligned(ws, kAlign)) return TQ4_E_ALIGN;
  return TQ4_OK;
}

constexpr int64_t kFusedRouterTokens = 64;

// ---- tq4_moe_grouped workspace ------------------------------------------
struct MoELayout {
  size_t counts, offsets, perm, inv, tiles, meta, xt, ht, o, total;
};

MoELayout moe_layout(int64_t t, int32_t topk, int32_t e, int64_t n1, int64_t k,
                     const MoEPlan &p) {
  const size_t pairs = static_cast<size_t>(t) * topk;
  MoELayout l{};
  size_t off = 0;
  l.counts = off;  off += align_up(sizeof(int32_t) * e);
  l.offsets = off; off += align_up(sizeof(int32_t) * (e + 1));
  l.perm = off;    off += align_up(sizeof(int32_t) * pairs);
  l.inv = off;     off += align_up(sizeof(int32_t) * pairs);
  l.tiles = off;   off += align_up(sizeof(MoETile) * p.max_tiles);
  l.meta = off;    off += kAlign;  // [0] tile count, [1] bad-id count
  l.xt = off;      off += align_up(static_cast<size_t>(t) * k * 2);
  l.ht = off;      off += align_up(pairs * n1 * 2);
  l.o = off;       off += align_up(pairs * k * 4);
  l.total = off;
  return l;
}

bool moe_shape_ok(int64_t t, int32_t topk, int32_t e, int64_t n1, int64_t k) {
  if (t < 0 || topk < 1 || e < 1 || e > 512 || topk > e) return false;
  if (n1 <= 0 || k <= 0 || n1 % 32 != 0 || k % 32 != 0) return false;
  const MoEPlan p = tq4::plan_moe(t * topk, e);
  if (p.max_tiles > 65535) return false;
  if (t * topk > INT32_MAX) return false;
  return true;
}

}  // namespace

extern "C" {

const char *tq4_status_string(int status) {
  switch (status) {
    case TQ4_OK: return "ok";
    case TQ4_E_NULL: return "required pointer is NULL";
    case TQ4_E_SHAPE: return "size out of range";
    case TQ4_E_ALIGN: return "pointer misaligned";
    case TQ4_E_WORKSPACE: return "workspace missing or too small";
    case TQ4_E_DEVICE: return "HIP call or kernel launch failed";
    case TQ4_E_TOO_LARGE: return "sizes need more scratch than the static scratch holds";
    default: return "unknown status";
  }
}

int tq4_version(void) { return 100; }

int tq4_codebook(float *out) {
  if (out == nullptr) return TQ4_E_NULL;
  memcpy(out, tq4::codebook().c, sizeof(float) * 16);
  return TQ4_OK;
}

size_t tq4_packed_size(int64_t n, int64_t k) {
  if (n < 0 || k < 0 || k % 32 != 0) return 0;
  return static_cast<size_t>(n) * static_cast<size_t>(k / 32) * 20;
}

int tq4_pack(const float *w, int64_t n, int64_t k, uint32_t sign_bits, uint8_t *packed,
             int32_t *nonfinite_count, void *stream) {
  if (n < 0 || k < 0 || k % 32 != 0) return TQ4_E_SHAPE;
  if (n == 0 || k == 0) return TQ4_OK;
  if (w == nullptr || packed == nullptr) return TQ4_E_NULL;
  if (!aligned(w, 16) || !aligned(packed, 4) ||
      (nonfinite_count != nullptr && !aligned(nonfinite_count, 4)))
    return TQ4_E_ALIGN;
  return device_status(
      tq4::launch_pack(w, n * (k / 32), sign_bits, packed, nonfinite_count, as_stream(stream)));
}

int tq4_pack_bf16(const uint16_t *w_bf16, int64_t n, int64_t k, uint32_t sign_bits,
                  uint8_t *packed, int32_t *nonfinite_count, void *stream) {
  if (n < 0 || k < 0 || k % 32 != 0) return TQ4_E_SHAPE;
  if (n == 0 || k == 0) return TQ4_OK;
  if (w_bf16 == nullptr || packed == nullptr) return TQ4_E_NULL;
  if (!aligned(w_bf16, 16) || !aligned(packed, 4) ||
      (nonfinite_count != nullptr && !aligned(nonfinite_count, 4)))
    return TQ4_E_ALIGN;
  return device_status(tq4::launch_pack_bf16(w_bf16, n * (k / 32), sign_bits, packed,
                                             nonfinite_count, as_stream(stream)));
}

int tq4_act_rht(const uint16_t *x_bf16, int64_t m, int64_t k, uint32_t sign_bits,
                uint16_t *xt_f16, void *stream) {
  if (m < 0 || k < 0 || k % 32 != 0) return TQ4_E_SHAPE;
  if (m == 0 || k == 0) return TQ4_OK;
  if (x_bf16 == nullptr || xt_f16 == nullptr) return TQ4_E_NULL;
  if (!aligned(x_bf16, 16) || !aligned(xt_f16, 16)) return TQ4_E_ALIGN;
  return device_status(tq4::launch_act_rht_bf16(x_bf16, m, k, sign_bits, xt_f16, as_stream(stream)));
}

size_t tq4_linear_workspace_size(int64_t m, int64_t k, int64_t n) {
  if (m < 0 || k < 0 || n < 0 || k % 32 != 0) return 0;
  if (m == 0 || n == 0 || k == 0) return 0;
  const size_t a = linear_layout(m, k, n, false).total;
  const size_t b = linear_layout(m, k, n, true).total;
  return a > b ? a : b;
}

namespace {

// Argument checks of the linear layer; none touches the device.  TQ4_OK means
// the call may proceed (it is then a no-op if m or n is 0).
int linear_args(const uint16_t *x_bf16, int64_t m, int64_t k, const uint8_t *packed, int64_t n,
                const tq4::Tail &tail, const void *y) {
  if (m < 0 || k < 0 || n < 0 || k % 32 != 0) return TQ4_E_SHAPE;
  if (m == 0 || n == 0) return TQ4_OK;
  if (y == nullptr) return TQ4_E_NULL;
  const size_t elem = tail.bf16 ? 2 : 4;
  if (!aligned(y, elem) || !aligned(tail.bias, 4) || !aligned(tail.residual, elem))
    return TQ4_E_ALIGN;
  // the residual is read where y is written: the same array or disjoint
  if (tail.residual != nullptr && tail.residual != y) {
    const uintptr_t r0 = reinterpret_cast<uintptr_t>(tail.residual);
    const uintptr_t y0 = reinterpret_cast<uintptr_t>(y);
    const uintptr_t bytes = static_cast<uintptr_t>(m) * static_cast<uintptr_t>(n) * elem;
    if (r0 < y0 + bytes && y0 < r0 + bytes) return TQ4_E_SHAPE;
  }
  if (k == 0) return TQ4_OK;
  if (x_bf16 == nullptr || packed == nullptr) return TQ4_E_NULL;
  if (!aligned(x_bf16, 16) || !aligned(packed, 4)) return TQ4_E_ALIGN;
  return TQ4_OK;
}

int linear_impl(const uint16_t *x_bf16, int64_t m, int64_t k, const uint8_t *packed, int64_t n,
                uint32_t sign_bits, const tq4::Tail &tail, void *y, void *workspace,
                size_t workspace_bytes, void *stream) {
  const int st = linear_args(x_bf16, m, k, packed, n, tail, y);
  if (st != TQ4_OK) return st;
  if (m == 0 || n == 0) return TQ4_OK;
  hipStream_t s = as_stream(stream);
  float *yf = static_cast<float *>(y);  // bf16 outputs are addressed as such by the kernels
  const bool plain = tail.bias == nullptr && tail.residual == nullptr && !tail.bf16;
  if (k == 0)
    return device_status(plain ? tq4::launch_fill_zero(yf, m * n, s)
                               : tq4::launch_tail_only(tail, m, n, yf, s));
  const LinearLayout l = linear_layout(m, k, n, false);
  const int ws_status = check_workspace(workspace, workspace_bytes, l.total);
  if (ws_status != TQ4_OK) return ws_status;
  if (tq4::skinny_fits(m, k, n))
    return device_status(tq4::launch_skinny(x_bf16, m, k, packed, n, sign_bits, yf, s, tail));
  char *ws = static_cast<char *>(workspace);
  uint16_t *xt = reinterpret_cast<uint16_t *>(ws + l.xt);
  hipError_t e = tq4::launch_act_rht_bf16(x_bf16, m, k, sign_bits, xt, s);
  if (e != hipSuccess) return TQ4_E_DEVICE;
  const DensePlan p = tq4::plan_dense(m, k, n);
  e = tq4::launch_dense(p, xt, m, k, packed, n, yf, reinterpret_cast<float *>(ws + l.partial), s,
                        tail);
  return device_status(e);
}

}  // namespace

int tq4_linear(const uint16_t *x_bf16, int64_t m, int64_t k, const uint8_t *packed, int64_t n,
               uint32_t sign_bits, float *y, void *workspace, size_t workspace_bytes,
               void *stream) {
  return linear_impl(x_bf16, m, k, packed, n, sign_bits, tq4::Tail{}, y, workspace,
                     workspace_bytes, stream);
}

int tq4_linear_epilogue(const uint16_t *x_bf16, int64_t m, int64_t k, const uint8_t *packed,
                        int64_t n, uint32_t sign_bits, const float *bias, const float *residual,
                        float *y, void *workspace, size_t workspace_bytes, void *stream) {
  return linear_impl(x_bf16, m, k, packed, n, sign_bits, tq4::Tail{bias, residual, 0}, y,
                     workspace, workspace_bytes, stream);
}

int tq4_linear_epilogue_bf16(const uint16_t *x_bf16, int64_t m, int64_t k, const uint8_t *packed,
                             int64_t n, uint32_t sign_bits, const float *bias,
                             const uint16_t *residual_bf16, uint16_t *y_bf16, void *workspace,
                             size_t workspace_bytes, void *stream) {
  return linear_impl(x_bf16, m, k, packed, n, sign_bits, tq4::Tail{bias, residual_bf16, 1},
                     y_bf16, workspace, workspace_bytes, stream);
}

int tq4_linear_variant(const uint16_t *x_bf16, int64_t m, int64_t k, const uint8_t *packed,
                       int64_t n, uint32_t sign_bits, float *y, void *workspace,
                       size_t workspace_bytes, int variant, void *stream) {
  if (variant == TQ4_VARIANT_DEFAULT)
    return linear_impl(x_bf16, m, k, packed, n, sign_bits, tq4::Tail{}, y, workspace,
                       workspace_bytes, stream);
  if (variant != TQ4_VARIANT_WEIGHT_ROTATION && variant != TQ4_VARIANT_VALU_PRODUCT)
    return TQ4_E_SHAPE;
  const int st = linear_args(x_bf16, m, k, packed, n, tq4::Tail{}, y);
  if (st != TQ4_OK) return st;
  if (m == 0 || n == 0) return TQ4_OK;
  if (k == 0) return TQ4_E_SHAPE;
  hipStream_t s = as_stream(stream);
  if (tq4::skinny_dma_fits(m, k, n, x_bf16, packed))
    return device_status(tq4::launch_skinny_variant(
        variant == TQ4_VARIANT_WEIGHT_ROTATION ? 1 : 2, x_bf16, m, k, packed, n, sign_bits, y, s));
  if (variant != TQ4_VARIANT_WEIGHT_ROTATION || m <= 16 || !tq4::dense_huge_fits(m, k, n))
    return TQ4_E_SHAPE;
  const size_t need = static_cast<size_t>(m) * static_cast<size_t>(k) * 2;
  const int ws_status = check_workspace(workspace, workspace_bytes, need);
  if (ws_status != TQ4_OK) return ws_status;
  uint16_t *xs = static_cast<uint16_t *>(workspace);
  hipError_t e = tq4::launch_act_sign_f16(x_bf16, m, k, sign_bits, xs, s);
  if (e == hipSuccess) e = tq4::launch_dense_weight_side(xs, m, k, packed, n, y, s);
  return device_status(e);
}

int tq4_linear_rotated(const uint16_t *xt_f16, int64_t m, int64_t k, const uint8_t *packed,
                       int64_t n, float *y, void *workspace, size_t workspace_bytes,
                       void *stream) {
  if (m < 0 || k < 0 || n < 0 || k % 32 != 0) return TQ4_E_SHAPE;
  if (m == 0 || n == 0) return TQ4_OK;
  if (y == nullptr) return TQ4_E_NULL;
  if (!aligned(y, 4)) return TQ4_E_ALIGN;
  hipStream_t s = as_stream(stream);
  if (k == 0) return device_status(tq4::launch_fill_zero(y, m * n, s));
  if (xt_f16 == nullptr || packed == nullptr) return TQ4_E_NULL;
  if (!aligned(xt_f16, 16) || !aligned(packed, 4)) return TQ4_E_ALIGN;
  const LinearLayout l = linear_layout(m, k, n, true);
  const int ws_status = check_workspace(workspace, workspace_bytes, l.total);
  if (ws_status != TQ4_OK) return ws_status;
  const DensePlan p = tq4::plan_dense(m, k, n);
  char *ws = static_cast<char *>(workspace);
  return device_status(tq4::launch_dense(p, xt_f16, m, k, packed, n, y,
                                         reinterpret_cast<float *>(ws + l.partial), s));
}

int tq4_moe_route(const int32_t *topk_ids, int64_t t, int32_t topk, int32_t n_experts,
                  int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv, void *stream) {
  if (t < 0 || topk < 1 || n_experts < 1 || n_experts > 512) return TQ4_E_SHAPE;
  if (t * topk > INT32_MAX) return TQ4_E_SHAPE;
  if (counts == nullptr || offsets == nullptr) return TQ4_E_NULL;
  if (t > 0 && (topk_ids == nullptr || perm == nullptr || inv == nullptr)) return TQ4_E_NULL;
  if (!aligned(counts, 4) || !aligned(offsets, 4) || !aligned(perm, 4) || !aligned(inv, 4) ||
      !aligned(topk_ids, 4))
    return TQ4_E_ALIGN;
  // Bucketing only: no tile list is requested (tiles == nullptr).
  return device_status(tq4::launch_route(topk_ids, t * topk, topk, n_experts, counts, offsets,
                                         perm, inv, nullptr, nullptr, 0, nullptr,
                                         as_stream(stream)));
}

size_t tq4_moe_workspace_size(int64_t t, int32_t topk, int32_t n_experts, int64_t n1, int64_t k) {
  if (!moe_shape_ok(t, topk, n_experts, n1, k)) return 0;
  const MoEPlan p = tq4::plan_moe(t * topk, n_experts);
  return moe_layout(t, topk, n_experts, n1, k, p).total;
}

namespace {

// The layer after validation: workspace of at least moe_layout(...).total
// bytes, 256-byte aligned.  With logits != nullptr the bucketing launch also
// routes the tokens, writing topk_ids and topk_w (then writable).
hipError_t moe_layer(const uint16_t *x_bf16, int64_t t, int64_t k, const int32_t *topk_ids,
                     const float *topk_w, int32_t topk, int32_t n_experts,
                     const uint8_t *w1_packed, int64_t n1, const uint8_t *w2_packed,
                     uint32_t sign_bits, float *out, char *ws, hipStream_t s,
                     const float *logits = nullptr) {
  const MoEPlan p = tq4::plan_moe(t * topk, n_experts);
  const MoELayout l = moe_layout(t, topk, n_experts, n1, k, p);
  int32_t *counts = reinterpret_cast<int32_t *>(ws + l.counts);
  int32_t *offsets = reinterpret_cast<int32_t *>(ws + l.offsets);
  int32_t *perm = reinterpret_cast<int32_t *>(ws + l.perm);
  int32_t *inv = reinterpret_cast<int32_t *>(ws + l.inv);
  MoETile *tiles = reinterpret_cast<MoETile *>(ws + l.tiles);
  int32_t *meta = reinterpret_cast<int32_t *>(ws + l.meta);
  uint16_t *xt = reinterpret_cast<uint16_t *>(ws + l.xt);
  uint16_t *ht = reinterpret_cast<uint16_t *>(ws + l.ht);
  float *o = reinterpret_cast<float *>(ws + l.o);
  const int64_t pairs = t * topk;
  hipError_t e = tq4::launch_route(topk_ids, pairs, topk, n_experts, counts, offsets, perm, inv,
                                   tiles, meta, p.tile_rows, nullptr, s, x_bf16, t * (k / 32),
                                   sign_bits, xt, logits, const_cast<float *>(topk_w));
  if (e == hipSuccess)
    e = tq4::launch_moe_gemm(p, 0, xt, k, perm, topk, w1_packed, n1, tiles, meta, nullptr, ht,
                             sign_bits, s);
  if (e == hipSuccess)
    e = tq4::launch_moe_gemm(p, 1, ht, n1, perm, topk, w2_packed, k, tiles, meta, o, nullptr,
                             sign_bits, s);
  if (e == hipSuccess) e = tq4::launch_combine(o, inv, topk_w, t, topk, k, out, s);
  return e;
}

int moe_args_status(const uint16_t *x_bf16, const uint8_t *w1_packed, const uint8_t *w2_packed,
                     const float *out) {
  if (x_bf16 == nullptr || w1_packed == nullptr || w2_packed == nullptr || out == nullptr)
    return TQ4_E_NULL;
  if (!aligned(x_bf16, 16) || !aligned(w1_packed, 4) || !aligned(w2_packed, 4) ||
      !aligned(out, 16))
    return TQ4_E_ALIGN;
  return TQ4_OK;
}

}  // namespace

int tq4_moe_grouped(const uint16_t *x_bf16, int64_t t, int64_t k, const int32_t *topk_ids,
                    const float *topk_w, int32_t topk, int32_t n_experts,
                    const uint8_t *w1_packed, int64_t n1, const uint8_t *w2_packed,
                    uint32_t sign_bits, float *out, void *workspace, size_t workspace_bytes,
                    void *stream) {
  if (!moe_shape_ok(t, topk, n_experts, n1, k)) return TQ4_E_SHAPE;
  if (t == 0) return TQ4_OK;
  if (topk_ids == nullptr || topk_w == nullptr) return TQ4_E_NULL;
  const int st = moe_args_status(x_bf16, w1_packed, w2_packed, out);
  if (st != TQ4_OK) return st;
  if (!aligned(topk_ids, 4) || !aligned(topk_w, 4)) return TQ4_E_ALIGN;
  const MoEPlan p = tq4::plan_moe(t * topk, n_experts);
  const MoELayout l = moe_layout(t, topk, n_experts, n1, k, p);
  if (workspace == nullptr || workspace_bytes < l.total) return TQ4_E_WORKSPACE;
  if (!aligned(workspace, kAlign)) return TQ4_E_ALIGN;
  return device_status(moe_layer(x_bf16, t, k, topk_ids, topk_w, topk, n_experts, w1_packed, n1,
                                 w2_packed, sign_bits, out, static_cast<char *>(workspace),
                                 as_stream(stream)));
}

size_t tq4_moe_block_workspace_size(int64_t t, int32_t topk, int32_t n_experts, int64_t n1,
                                    int64_t k) {
  if (!moe_shape_ok(t, topk, n_experts, n1, k)) return 0;
  const size_t layer = tq4_moe_workspace_size(t, topk, n_experts, n1, k);
  if (layer == 0) return 0;
  const size_t slots = static_cast<size_t>(t) * static_cast<size_t>(topk);
  return layer + align_up(slots * sizeof(int32_t)) + align_up(slots * sizeof(float));
}

int tq4_moe_block(const uint16_t *x_bf16, int64_t t, int64_t k, const float *logits,
                  int32_t n_experts, int32_t topk, const uint8_t *w1_packed, int64_t n1,
                  const uint8_t *w2_packed, uint32_t sign_bits, float *out, void *workspace,
                  size_t workspace_bytes, void *stream) {
  if (!moe_shape_ok(t, topk, n_experts, n1, k)) return TQ4_E_SHAPE;
  if (t == 0) return TQ4_OK;
  if (logits == nullptr) return TQ4_E_NULL;
  const int st = moe_args_status(x_bf16, w1_packed, w2_packed, out);
  if (st != TQ4_OK) return st;
  if (!aligned(logits, 4)) return TQ4_E_ALIGN;
  const size_t need = tq4_moe_block_workspace_size(t, topk, n_experts, n1, k);
  if (workspace == nullptr || workspace_bytes < need) return TQ4_E_WORKSPACE;
  if (!aligned(workspace, kAlign)) return TQ4_E_ALIGN;
  char *ws = static_cast<char *>(workspace);
  const size_t layer = tq4_moe_workspace_size(t, topk, n_experts, n1, k);
  const size_t slots = static_cast<size_t>(t) * static_cast<size_t>(topk);
  int32_t *ids = reinterpret_cast<int32_t *>(ws + layer);
  float *gates = reinterpret_cast<float *>(ws + layer + align_up(slots * sizeof(int32_t)));
  hipStream_t s = as_stream(stream);
  // up to 64 tokens (4 per wave of the bucketing workgroup) the router runs
  // inside the bucketing launch; above that as its own launch of t / 4
  // workgroups.  Both use the same per-token routine: the same ids and gates.
  if (t <= kFusedRouterTokens)
    return device_status(moe_layer(x_bf16, t, k, ids, gates, topk, n_experts, w1_packed, n1,
                                   w2_packed, sign_bits, out, ws, s, logits));
  hipError_t e = tq4::launch_router(logits, t, n_experts, topk, ids, gates, s);
  if (e == hipSuccess)
    e = moe_layer(x_bf16, t, k, ids, gates, topk, n_experts, w1_packed, n1, w2_packed, sign_bits,
                  out, ws, s);
  return device_status(e);
}

size_t tq4_moe_block_persistent_workspace_size(int64_t t, int32_t topk, int32_t n_experts,
                                               int64_t n1, int64_t k) {
  const size_t blk = tq4_moe_block_workspace_size(t, topk, n_experts, n1, k);
  if (blk == 0 || tq4::plan_moe(t * topk, n_experts).msub != 1) return 0;
  return blk + align_up(tq4::moe_block_persistent_scratch_bytes());
}

int tq4_moe_block_persistent(const uint16_t *x_bf16, int64_t t, int64_t k, const float *logits,
                             int32_t n_experts, int32_t topk, const uint8_t *w1_packed,
                             int64_t n1, const uint8_t *w2_packed, uint32_t sign_bits,
                             float *out, void *workspace, size_t workspace_bytes, void *stream) {
  if (!moe_shape_ok(t, topk, n_experts, n1, k)) return TQ4_E_SHAPE;
  const MoEPlan p = tq4::plan_moe(t * topk, n_experts);
  if (p.msub != 1) return TQ4_E_SHAPE;
  if (t == 0) return TQ4_OK;
  if (logits == nullptr) return TQ4_E_NULL;
  const int st = moe_args_status(x_bf16, w1_packed, w2_packed, out);
  if (st != TQ4_OK) return st;
  if (!aligned(logits, 4)) return TQ4_E_ALIGN;
  const size_t need = tq4_moe_block_persistent_workspace_size(t, topk, n_experts, n1, k);
  if (workspace == nullptr || workspace_bytes < need) return TQ4_E_WORKSPACE;
  if (!aligned(workspace, kAlign)) return TQ4_E_ALIGN;
  char *ws = static_cast<char *>(workspace);
  const MoELayout l = moe_layout(t, topk, n_experts, n1, k, p);
  const size_t slots = static_cast<size_t>(t) * static_cast<size_t>(topk);
  tq4::MoEScratch sc{};
  sc.counts = reinterpret_cast<int32_t *>(ws + l.counts);
  sc.offsets = reinterpret_cast<int32_t *>(ws + l.offsets);
  sc.perm = reinterpret_cast<int32_t *>(ws + l.perm);
  sc.inv = reinterpret_cast<int32_t *>(ws + l.inv);
  sc.tiles = reinterpret_cast<MoETile *>(ws + l.tiles);
  sc.n_tiles = reinterpret_cast<int32_t *>(ws + l.meta);
  sc.xt = reinterpret_cast<uint16_t *>(ws + l.xt);
  sc.ht = reinterpret_cast<uint16_t *>(ws + l.ht);
  sc.o = reinterpret_cast<float *>(ws + l.o);
  sc.ids = reinterpret_cast<int32_t *>(ws + l.total);
  sc.gates = reinterpret_cast<float *>(ws + l.total + align_up(slots * sizeof(int32_t)));
  sc.bar = reinterpret_cast<uint32_t *>(ws + l.total + align_up(slots * sizeof(int32_t)) +
                                        align_up(slots * sizeof(float)));
  return device_status(tq4::launch_moe_block_persistent(x_bf16, t, k, logits, n_experts, topk,
                                                        w1_packed, n1, w2_packed, sign_bits, out,
                                                        sc, as_stream(stream)));
}

// ---- fp8 weight cache ---------------------------------------------------

namespace {

bool fp8_sizes_ok(int64_t rows, int64_t k) {
  return rows >= 0 && k >= 0 && k % 32 == 0 && (k == 0 || tq4::fp8_shape_fits(1, k, 1));
}

size_t fp8_rows_bytes(int64_t rows, int64_t k) {
  const int64_t kp = tq4::fp8_padded_k(k);
  return static_cast<size_t>(rows) * static_cast<size_t>(kp) +
         static_cast<size_t>(rows) * static_cast<size_t>(kp / 32);
}

}  // namespace

size_t tq4_fp8_cache_size(int64_t n, int64_t k) {
  if (!fp8_sizes_ok(n, k) || k == 0) return 0;
  return fp8_rows_bytes(n, k);
}

int tq4_fp8_cache(const uint8_t *packed, int64_t n, int64_t k, uint32_t sign_bits, uint8_t *cache,
                  void *stream) {
  if (!fp8_sizes_ok(n, k)) return TQ4_E_SHAPE;
  if (n == 0 || k == 0) return TQ4_OK;
  if (packed == nullptr || cache == nullptr) return TQ4_E_NULL;
  if (!aligned(packed, 4) || !aligned(cache, 16)) return TQ4_E_ALIGN;
  const int64_t kp = tq4::fp8_padded_k(k);
  return device_status(tq4::launch_fp8_cache(packed, n, k, sign_bits, cache, cache + n * kp,
                                             as_stream(stream)));
}

int tq4_act_mxfp8(const uint16_t *x_bf16, int64_t m, int64_t k, uint8_t *codes, uint8_t *scales,
                  void *stream) {
  if (!fp8_sizes_ok(m, k)) return TQ4_E_SHAPE;
  if (m == 0 || k == 0) return TQ4_OK;
  if (x_bf16 == nullptr || codes == nullptr || scales == nullptr) return TQ4_E_NULL;
  if (!aligned(x_bf16, 16) || !aligned(codes, 16)) return TQ4_E_ALIGN;
  return device_status(tq4::launch_act_mxfp8(x_bf16, m, k, codes, scales, as_stream(stream)));
}

size_t tq4_linear_fp8_workspace_size(int64_t m, int64_t k, int64_t n) {
  if (!fp8_sizes_ok(m, k) || n < 0) return 0;
  if (m == 0 || n == 0 || k == 0) return 0;
  const int64_t kp = tq4::fp8_padded_k(k);
  return align_up(static_cast<size_t>(m) * static_cast<size_t>(kp)) +
         align_up(static_cast<size_t>(m) * static_cast<size_t>(kp / 32));
}

int tq4_linear_fp8(const uint16_t *x_bf16, int64_t m, int64_t k, const uint8_t *cache, int64_t n,
                   float *y, void *workspace, size_t workspace_bytes, void *stream) {
  if (!fp8_sizes_ok(m, k) || n < 0) return TQ4_E_SHAPE;
  if (m == 0 || n == 0) return TQ4_OK;
  if (y == nullptr) return TQ4_E_NULL;
  if (!aligned(y, 4)) return TQ4_E_ALIGN;
  hipStream_t s = as_stream(stream);
  if (k == 0) return device_status(tq4::launch_fill_zero(y, m * n, s));
  if (x_bf16 == nullptr || cache == nullptr) return TQ4_E_NULL;
  if (!aligned(x_bf16, 16) || !aligned(cache, 16)) return TQ4_E_ALIGN;
  const int ws_status =
      check_workspace(workspace, workspace_bytes, tq4_linear_fp8_workspace_size(m, k, n));
  if (ws_status != TQ4_OK) return ws_status;
  const int64_t kp = tq4::fp8_padded_k(k);
  uint8_t *xq = static_cast<uint8_t *>(workspace);
  uint8_t *xs = xq + align_up(static_cast<size_t>(m) * static_cast<size_t>(kp));
  hipError_t e = tq4::launch_act_mxfp8(x_bf16, m, k, xq, xs, s);
  if (e != hipSuccess) return TQ4_E_DEVICE;
  return device_status(
      tq4::launch_linear_fp8(xq, xs, m, k, cache, cache + n * kp, n, y, s));
}

int tq4_linear_fp8_quantized(const uint8_t *x_codes, const uint8_t *x_scales, int64_t m,
                             int64_t k, const uint8_t *cache, int64_t n, float *y,
                             void *stream) {
  if (!fp8_sizes_ok(m, k) || n < 0) return TQ4_E_SHAPE;
  if (m == 0 || n == 0) return TQ4_OK;
  if (y == nullptr) return TQ4_E_NULL;
  if (!aligned(y, 4)) return TQ4_E_ALIGN;
  hipStream_t s = as_stream(stream);
  if (k == 0) return device_status(tq4::launch_fill_zero(y, m * n, s));
  if (x_codes == nullptr || x_scales == nullptr || cache == nullptr) return TQ4_E_NULL;
  if (!aligned(x_codes, 16) || !aligned(x_scales, 4) || !aligned(cache, 16)) return TQ4_E_ALIGN;
  const int64_t kp = tq4::fp8_padded_k(k);
  return device_status(
      tq4::launch_linear_fp8(x_codes, x_scales, m, k, cache, cache + n * kp, n, y, s));
}

// ---- fp8 MoE --------------------------------------------------------------

namespace {

struct MoEFp8Layout {
  int tile_rows;
  int64_t max_tiles;
  size_t counts, offsets, perm, inv, tiles, meta, xq, xs, hq, hs, o, total;
};

MoEFp8Layout moe_fp8_layout(int64_t t, int32_t topk, int32_t e, int64_t n1, int64_t k) {
  const int64_t pairs = t * topk;
  const int64_t kp = tq4::fp8_padded_k(k);
  const int64_t n1p = tq4::fp8_padded_k(n1);
  MoEFp8Layout l{};
  l.tile_rows = tq4::fp8_moe_tile_rows(pairs, e);
  const int64_t busy = pairs < e ? pairs : e;
  l.max_tiles = pairs / l.tile_rows + busy + 1;
  const size_t p = static_cast<size_t>(pairs);
  size_t off = 0;
  l.counts = off;  off += align_up(sizeof(int32_t) * e);
  l.offsets = off; off += align_up(sizeof(int32_t) * (e + 1));
  l.perm = off;    off += align_up(sizeof(int32_t) * p);
  l.inv = off;     off += align_up(sizeof(int32_t) * p);
  l.tiles = off;   off += align_up(sizeof(MoETile) * static_cast<size_t>(l.max_tiles));
  l.meta = off;    off += kAlign;
  l.xq = off;      off += align_up(static_cast<size_t>(t) * kp);
  l.xs = off;      off += align_up(static_cast<size_t>(t) * (kp / 32));
  l.hq = off;      off += align_up(p * n1p);
  l.hs = off;      off += align_up(p * (n1p / 32));
  l.o = off;       off += align_up(p * k * 4);
  l.total = off;
  return l;
}

bool moe_fp8_shape_ok(int64_t t, int32_t topk, int32_t e, int64_t n1, int64_t k) {
  if (!moe_shape_ok(t, topk, e, n1, k)) return false;
  if (!tq4::fp8_shape_fits(1, k, 1) || !tq4::fp8_shape_fits(1, n1, 1)) return false;
  if (!tq4::fp8_moe_shape_fits(t, k, n1) || !tq4::fp8_moe_shape_fits(t * topk, n1, k))
    return false;
  return moe_fp8_layout(t, topk, e, n1, k).max_tiles <= 65535;
}

}  // namespace

size_t tq4_moe_grouped_fp8_workspace_size(int64_t t, int32_t topk, int32_t n_experts, int64_t n1,
                                          int64_t k) {
  if (!moe_fp8_shape_ok(t, topk, n_experts, n1, k)) return 0;
  return moe_fp8_layout(t, topk, n_experts, n1, k).total;
}

int tq4_moe_grouped_fp8(const uint16_t *x_bf16, int64_t t, int64_t k, const int32_t *topk_ids,
                        const float *topk_w, int32_t topk, int32_t n_experts,
                        const uint8_t *w1_cache, int64_t n1, const uint8_t *w2_cache, float *out,
                        void *workspace, size_t workspace_bytes, void *stream) {
  if (!moe_fp8_shape_ok(t, topk, n_experts, n1, k)) return TQ4_E_SHAPE;
  if (t == 0) return TQ4_OK;
  if (x_bf16 == nullptr || topk_ids == nullptr || topk_w == nullptr || w1_cache == nullptr ||
      w2_cache == nullptr || out == nullptr)
    return TQ4_E_NULL;
  if (!aligned(x_bf16, 16) || !aligned(topk_ids, 4) || !aligned(topk_w, 4) ||
      !aligned(w1_cache, 16) || !aligned(w2_cache, 16) || !aligned(out, 16))
    return TQ4_E_ALIGN;
  const MoEFp8Layout l = moe_fp8_layout(t, topk, n_experts, n1, k);
  if (workspace == nullptr || workspace_bytes < l.total) return TQ4_E_WORKSPACE;
  if (!aligned(workspace, kAlign)) return TQ4_E_ALIGN;
  char *ws = static_cast<char *>(workspace);
  int32_t *counts = reinterpret_cast<int32_t *>(ws + l.counts);
  int32_t *offsets = reinterpret_cast<int32_t *>(ws + l.offsets);
  int32_t *perm = reinterpret_cast<int32_t *>(ws + l.perm);
  int32_t *inv = reinterpret_cast<int32_t *>(ws + l.inv);
  MoETile *tiles = reinterpret_cast<MoETile *>(ws + l.tiles);
  int32_t *meta = reinterpret_cast<int32_t *>(ws + l.meta);
  uint8_t *xq = reinterpret_cast<uint8_t *>(ws + l.xq);
  uint8_t *xs = reinterpret_cast<uint8_t *>(ws + l.xs);
  uint8_t *hq = reinterpret_cast<uint8_t *>(ws + l.hq);
  uint8_t *hs = reinterpret_cast<uint8_t *>(ws + l.hs);
  float *o = reinterpret_cast<float *>(ws + l.o);
  const int64_t pairs = t * topk;
  const int64_t kp = tq4::fp8_padded_k(k);
  const int64_t n1p = tq4::fp8_padded_k(n1);
  // stacked caches: codes of all E * rows rows, then their scale bytes
  const uint8_t *w1s = w1_cache + static_cast<int64_t>(n_experts) * n1 * kp;
  const uint8_t *w2s = w2_cache + static_cast<int64_t>(n_experts) * k * n1p;
  hipStream_t s = as_stream(stream);
  hipError_t e = tq4::launch_act_mxfp8(x_bf16, t, k, xq, xs, s);
  if (e == hipSuccess)
    e = tq4::launch_route(topk_ids, pairs, topk, n_experts, counts, offsets, perm, inv, tiles,
                          meta, l.tile_rows, nullptr, s);
  if (e == hipSuccess)
    e = tq4::launch_moe_fp8(0, l.tile_rows, xq, xs, t, k, perm, topk, w1_cache, w1s, n1, n1p,
                            tiles, meta, l.max_tiles, nullptr, hq, hs, s);
  if (e == hipSuccess)
    e = tq4::launch_moe_fp8(1, l.tile_rows, hq, hs, pairs, n1, perm, topk, w2_cache, w2s, k, k,
                            tiles, meta, l.max_tiles, o, nullptr, nullptr, s);
  if (e == hipSuccess) e = tq4::launch_combine(o, inv, topk_w, t, topk, k, out, s);
  return device_status(e);
}

int tq4_read_probe(const void *src, int64_t bytes, float *sink, void *stream) {
  if (bytes < 0 || bytes % 16 != 0) return TQ4_E_SHAPE;
  if (bytes == 0) return TQ4_OK;
  if (src == nullptr || sink == nullptr) return TQ4_E_NULL;
  if (!aligned(src, 16) || !aligned(sink, 4)) return TQ4_E_ALIGN;
  return device_status(tq4::launch_read_probe(src, bytes, sink, as_stream(stream)));
}

int tq4_moe_router(const float *logits, int64_t t, int32_t n_experts, int32_t topk,
                   int32_t *topk_ids, float *topk_w, void *stream) {
  if (t < 0 || n_experts < 1 || n_experts > 512 || topk < 1 || topk > n_experts)
    return TQ4_E_SHAPE;
  if (t > (int64_t{1} << 33)) return TQ4_E_SHAPE;  // grid of t / 4 workgroups
  if (t == 0) return TQ4_OK;
  if (logits == nullptr || topk_ids == nullptr || topk_w == nullptr) return TQ4_E_NULL;
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4)) return TQ4_E_ALIGN;
  return device_status(
      tq4::launch_router(logits, t, n_experts, topk, topk_ids, topk_w, as_stream(stream)));
}

// ---- tq4_linear without a workspace argument -------------------------------
// The scratch of tq4_linear (rotated activations and split-K partial sums)
// lives in a device array of the library, one per GPU, so that the call
// allocates nothing.  Host code never uses the array's name as an address:
// its device address is looked up once per device and kept below.

}  // extern "C"

static __device__ __attribute__((aligned(256))) uint8_t scratch[TQ4_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch`, looked up on its first use; NULL if
// the lookup fails.
void *scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int tq4_linear_noalloc(const uint16_t *x_bf16, int64_t m, int64_t k, const uint8_t *packed,
                       int64_t n, uint32_t sign_bits, float *y, void *stream) {
  const int st = linear_args(x_bf16, m, k, packed, n, tq4::Tail{}, y);
  if (st != TQ4_OK) return st;
  if (m == 0 || n == 0) return TQ4_OK;
  const size_t need = tq4_linear_workspace_size(m, k, n);
  if (need > TQ4_NOALLOC_SCRATCH_BYTES) return TQ4_E_TOO_LARGE;
  void *ws = nullptr;
  if (need > 0) {
    ws = scratch_for_current_device();
    if (ws == nullptr) return TQ4_E_DEVICE;
  }
  return linear_impl(x_bf16, m, k, packed, n, sign_bits, tq4::Tail{}, y, ws,
                     TQ4_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
