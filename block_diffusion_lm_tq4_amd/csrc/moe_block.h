// The MoE block as one persistent kernel (gemm.hip), for the C ABI (api.cpp).
#pragma once
#include "tq4_internal.h"

namespace tq4 {
// Device buffers of one MoE layer call (pieces of the caller's workspace).
struct MoEScratch {
  int32_t *ids;       // [t * topk] routed expert ids
  float *gates;       // [t * topk] their gates
  int32_t *counts, *offsets, *perm, *inv;
  MoETile *tiles;
  int32_t *n_tiles;   // device tile count
  uint16_t *xt, *ht;  // rotated activation rows, rotated hidden rows
  float *o;           // down-product rows [pairs][k]
  uint32_t *bar;      // moe_block_persistent_scratch_bytes() for the grid barrier
};
// The MoE block from router logits in one cooperative launch (after a small
// reset launch), bit-equal to the launches of the layer; 16-row tiles only
// (plan_moe(t * topk, n_experts).msub == 1).
size_t moe_block_persistent_scratch_bytes();
hipError_t launch_moe_block_persistent(const uint16_t *x, int64_t t, int64_t k,
                                       const float *logits, int32_t n_experts, int32_t topk,
                                       const uint8_t *w1, int64_t n1, const uint8_t *w2,
                                       uint32_t sign_bits, float *out, const MoEScratch &sc,
                                       hipStream_t s);

}  // namespace tq4
