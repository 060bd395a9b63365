// Activation-side rotation: xt = H32 (s .* x) / sqrt(32) on every 32-block of
// every row, fp32 butterfly, fp16 result.
//
// The format rotates each weight block, z = R w with R = H32 diag(s)/sqrt(32)
// (Nemotron-TheHobbit-30B-A3B model card, What "Config-I" means).  R is
// orthogonal, so x . w_hat = (R x) . z_hat blockwise: rotating the M
// activation rows once replaces an inverse transform of all N weight rows,
// and the weight side of the product is only codebook lookup times scale.
#include "tq4_internal.h"

namespace tq4 {
namespace {

__global__ __launch_bounds__(256) void act_rht_kernel(const uint16_t *__restrict__ x,
                                                      int64_t n_blocks, uint32_t sign_bits,
                                                      uint16_t *__restrict__ xt) {
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (blk >= n_blocks) return;
  rotate_block_bf16(x + blk * 32, sign_bits, xt + blk * 32);
}

hipError_t launch(const uint16_t *x, int64_t m, int64_t k, uint32_t sign_bits, uint16_t *xt,
                  hipStream_t s) {
  const int64_t n_blocks = m * (k / 32);
  if (n_blocks == 0) return hipSuccess;
  const int threads = 256;
  const int64_t grid = (n_blocks + threads - 1) / threads;
  hipLaunchKernelGGL(act_rht_kernel, dim3(static_cast<unsigned>(grid)), dim3(threads), 0, s,
                     x, n_blocks, sign_bits, xt);
  return hipGetLastError();
}

// s .* x per 32-block, bf16 to fp16 (no rotation): the activations of the
// weight-side measurement variant, whose weights carry the rotation.
__global__ __launch_bounds__(256) void act_sign_kernel(const uint16_t *__restrict__ x,
                                                       int64_t n_blocks, uint32_t sign_bits,
                                                       uint16_t *__restrict__ xs) {
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (blk >= n_blocks) return;
  const uint4 *q = reinterpret_cast<const uint4 *>(x + blk * 32);
  uint4 *dst = reinterpret_cast<uint4 *>(xs + blk * 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 d = q[i];
    const uint32_t w[4] = {d.x, d.y, d.z, d.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 8 * i + 2 * j;
      const float lo = __uint_as_float((w[j] << 16) ^ (((sign_bits >> e) & 1u) << 31));
      const float hi = __uint_as_float((w[j] & 0xFFFF0000u) ^ (((sign_bits >> (e + 1)) & 1u) << 31));
      o[j] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(lo))) |
             (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(hi))) << 16);
    }
    dst[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float *__restrict__ p, int64_t count) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < count) p[i] = 0.f;
}

// y = bias + residual, for a product with an empty k.
__global__ __launch_bounds__(256) void tail_only_kernel(Tail t, int64_t m, int64_t n, float *y) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= m * n) return;
  const int64_t col = t.bias != nullptr ? i % n : 0;  // the column only feeds the bias
  const float res = t.residual != nullptr ? tail_residual(t, i) : 0.f;
  tail_store(t, y, i, tail_sum(t, 0.f, col, res));
}

}  // namespace

hipError_t launch_tail_only(const Tail &t, int64_t m, int64_t n, float *y, hipStream_t s) {
  const int64_t count = m * n;
  if (count == 0) return hipSuccess;
  hipLaunchKernelGGL(tail_only_kernel, dim3(static_cast<unsigned>((count + 255) / 256)), dim3(256),
                     0, s, t, m, n, y);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float *p, int64_t count, hipStream_t s) {
  if (count == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>((count + 255) / 256)), dim3(256),
                     0, s, p, count);
  return hipGetLastError();
}

hipError_t launch_act_sign_f16(const uint16_t *x, int64_t m, int64_t k, uint32_t sign_bits,
                               uint16_t *xs, hipStream_t s) {
  const int64_t n_blocks = m * (k / 32);
  if (n_blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(act_sign_kernel, dim3(static_cast<unsigned>((n_blocks + 255) / 256)),
                     dim3(256), 0, s, x, n_blocks, sign_bits, xs);
  return hipGetLastError();
}

hipError_t launch_act_rht_bf16(const uint16_t *x, int64_t m, int64_t k, uint32_t sign_bits,
                               uint16_t *xt, hipStream_t s) {
  return launch(x, m, k, sign_bits, xt, s);
}

}  // namespace tq4
