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

template <typename In>
__device__ inline void load_block(const In *p, float (&v)[32]);

template <>
__device__ inline void load_block<uint16_t>(const uint16_t *p, float (&v)[32]) {
  const uint4 *q = reinterpret_cast<const uint4 *>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 d = q[i];
    const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
      v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
}

template <typename In>
__global__ __launch_bounds__(256) void act_rht_kernel(const In *__restrict__ x, int64_t n_blocks,
                                                      uint32_t sign_bits,
                                                      uint16_t *__restrict__ xt) {
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (blk >= n_blocks) return;
  float v[32];
  load_block<In>(x + blk * 32, v);
#pragma unroll
  for (int i = 0; i < 32; ++i)
    if ((sign_bits >> i) & 1u) v[i] = -v[i];
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
  const float rs32 = 0x1.6a09e6p-3f;  // 1/sqrt(32) rounded to fp32
  uint4 *dst = reinterpret_cast<uint4 *>(xt + blk * 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const _Float16 lo = static_cast<_Float16>(v[8 * i + 2 * j] * rs32);
      const _Float16 hi = static_cast<_Float16>(v[8 * i + 2 * j + 1] * rs32);
      w[j] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
             (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
    }
    dst[i] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <typename In>
hipError_t launch(const In *x, int64_t m, int64_t k, uint32_t sign_bits, uint16_t *xt,
                  hipStream_t s) {
  const int64_t n_blocks = m * (k / 32);
  if (n_blocks == 0) return hipSuccess;
  const int threads = 256;
  const int64_t grid = (n_blocks + threads - 1) / threads;
  hipLaunchKernelGGL(act_rht_kernel<In>, dim3(static_cast<unsigned>(grid)), dim3(threads), 0, s,
                     x, n_blocks, sign_bits, xt);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float *__restrict__ p, int64_t count) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < count) p[i] = 0.f;
}

}  // namespace

hipError_t launch_fill_zero(float *p, int64_t count, hipStream_t s) {
  if (count == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>((count + 255) / 256)), dim3(256),
                     0, s, p, count);
  return hipGetLastError();
}

hipError_t launch_act_rht_bf16(const uint16_t *x, int64_t m, int64_t k, uint32_t sign_bits,
                               uint16_t *xt, hipStream_t s) {
  return launch<uint16_t>(x, m, k, sign_bits, xt, s);
}

}  // namespace tq4
