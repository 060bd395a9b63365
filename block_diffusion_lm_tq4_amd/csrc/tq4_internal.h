// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq4 {

// The 16 stored levels (fp32, ascending); passed to kernels by value.
struct Codebook {
  float c[16];
};

// Lloyd-Max levels of N(0,1) rounded to fp32, computed once on the host.
const Codebook &codebook();

// ---- launchers (return hipSuccess or the launch error) --------------------
hipError_t launch_pack(const float *w, int64_t n_blocks, uint32_t sign_bits,
                       uint8_t *packed, int32_t *nonfinite, hipStream_t s);

// Rotate [m, k] bf16 rows to fp16.
hipError_t launch_act_rht_bf16(const uint16_t *x, int64_t m, int64_t k, uint32_t sign_bits,
                               uint16_t *xt, hipStream_t s);

hipError_t launch_fill_zero(float *p, int64_t count, hipStream_t s);

// Dense product y[m, n] = xt[m, :] . Zhat[n, :]^T with xt already rotated.
struct DensePlan {
  int msub;       // 16-row MFMA tiles per wave along m
  int nsub;       // 16-row MFMA tiles per wave along n
  int waves_m;    // waves per workgroup along m
  int waves_n;    // waves per workgroup along n
  int ksplit;     // workgroups along k (partial sums reduced in fixed order)
  int64_t m_tiles, n_tiles, chunks;
  size_t partial_bytes;  // split-K partial sums (workspace, beyond xt)
};
DensePlan plan_dense(int64_t m, int64_t k, int64_t n);
hipError_t launch_dense(const DensePlan &p, const uint16_t *xt, int64_t m, int64_t k,
                        const uint8_t *packed, int64_t n, float *y, float *partial,
                        hipStream_t s);

// Single-kernel path for m <= 16 (rotation fused, no workspace).
bool skinny_fits(int64_t m, int64_t k, int64_t n);
hipError_t launch_skinny(const uint16_t *x, int64_t m, int64_t k, const uint8_t *packed,
                         int64_t n, uint32_t sign_bits, float *y, hipStream_t s);

// MoE pieces.
struct MoETile {  // one m-tile of one expert's segment in bucket order
  int32_t expert;
  int32_t row0;   // first row (bucket position) of the tile
  int32_t rows;   // rows in this tile (<= tile height)
  int32_t pad;
};
hipError_t launch_route(const int32_t *ids, int64_t pairs, int32_t topk, int32_t n_experts,
                        int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv,
                        MoETile *tiles, int32_t *n_tiles, int32_t tile_rows,
                        int32_t *status, hipStream_t s);

struct MoEPlan {
  int msub, nsub, waves_m, waves_n;
  int tile_rows;       // rows per MoE tile = 16 * msub * waves_m
  int64_t max_tiles;   // upper bound on tiles over all experts
};
MoEPlan plan_moe(int64_t pairs, int32_t n_experts);

// Grouped product over MoE tiles.  mode 0 (up): A rows gathered through
// perm[]/topk from xt [t, k]; output out16[row, n] = the rotation (sign_bits,
// per 32-block, fp16) of relu(acc)^2, n % 32 == 0.  mode 1 (down): A rows are
// the bucket rows of ht [pairs, k]; output out[row, n] = acc (fp32).
hipError_t launch_moe_gemm(const MoEPlan &p, int mode, const uint16_t *a, int64_t k,
                           const int32_t *perm, int32_t topk, const uint8_t *w_packed,
                           int64_t n, const MoETile *tiles, const int32_t *n_tiles,
                           float *out, uint16_t *out16, uint32_t sign_bits, hipStream_t s);

// Streaming read of `bytes` (a multiple of 16) from a 16-byte aligned buffer.
hipError_t launch_read_probe(const void *src, int64_t bytes, float *sink, hipStream_t s);

hipError_t launch_combine(const float *o, const int32_t *inv, const float *topk_w,
                          int64_t t, int32_t topk, int64_t k, float *out, hipStream_t s);

}  // namespace tq4
