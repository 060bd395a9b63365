// TQ4_1S encoder (offline quantizer; Nemotron-TheHobbit-30B-A3B model card,
// sections What "Config-I" means and Reproduction).
//
// One thread encodes one 32-weight block entirely in fp64:
//   v = s .* w                       (exact)
//   u = H32 v                        (in-place radix-2 butterfly, Sylvester order)
//   z = u * (1/sqrt 32)              (one rounding)
//   S_h = bf16(fp32(max_{j in h}|z_j| / c_15))   h = elements 0-15, 16-31
//   q_j = #{k : z_j > S_h * m_k},  m_k = (c_k + c_{k+1}) / 2
// The thresholds S_h * m_k are exact in fp64 (bf16 significand times a
// midpoint of two fp32 levels), so every code is the exact one.  This file is
// built with -ffp-contract=off: no product may be fused into a sum.
#include "tq4_internal.h"

namespace tq4 {
namespace {

// fp32 -> bf16, round to nearest even, on the bit pattern; NaN -> 0x7FC0.
__device__ inline uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

struct PackArgs {
  Codebook cb;
};

// The block's 32 weights as fp32 values (every bf16 value is exact in fp32).
__device__ inline void load_weights(const float *w, float (&e)[32]) {
  const float4 *src = reinterpret_cast<const float4 *>(w);  // 128 contiguous bytes
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 q = src[i];
    e[4 * i] = q.x;
    e[4 * i + 1] = q.y;
    e[4 * i + 2] = q.z;
    e[4 * i + 3] = q.w;
  }
}

__device__ inline void load_weights(const uint16_t *w, float (&e)[32]) {
  const uint4 *src = reinterpret_cast<const uint4 *>(w);  // 64 contiguous bytes
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 q = src[i];
    const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      e[8 * i + 2 * j] = __uint_as_float(d[j] << 16);
      e[8 * i + 2 * j + 1] = __uint_as_float(d[j] & 0xFFFF0000u);
    }
  }
}

template <typename In>
__global__ __launch_bounds__(256) void pack_kernel(const In *__restrict__ w, int64_t n_blocks,
                                                   uint32_t sign_bits, PackArgs args,
                                                   uint8_t *__restrict__ packed,
                                                   int32_t *__restrict__ nonfinite) {
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (blk >= n_blocks) return;

  float e[32];
  load_weights(w + blk * 32, e);
  double v[32];
  bool finite = true;
#pragma unroll
  for (int idx = 0; idx < 32; ++idx) {
    finite = finite && isfinite(e[idx]);
    const double d = static_cast<double>(e[idx]);
    v[idx] = ((sign_bits >> idx) & 1u) ? -d : d;
  }

  // Walsh-Hadamard transform, natural (Sylvester) order.
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & h) == 0) {
        const double a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }

  const double rs32 = 0x1.6a09e667f3bcdp-3;  // correctly rounded 1/sqrt(32)
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = v[i] * rs32;

  double mid[15];
#pragma unroll
  for (int k = 0; k < 15; ++k)
    mid[k] = 0.5 * (static_cast<double>(args.cb.c[k]) + static_cast<double>(args.cb.c[k + 1]));
  const double c15 = static_cast<double>(args.cb.c[15]);

  uint32_t words[5];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    // max |z| over the half; any NaN makes the maximum NaN
    double amax = 0.0;
    bool has_nan = false;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const double a = fabs(v[16 * h + j]);
      has_nan = has_nan || isnan(a);
      amax = a > amax ? a : amax;
    }
    if (has_nan) amax = __builtin_nan("");
    const uint32_t sbits = bf16_rne_bits(static_cast<float>(amax / c15));
    const double scale = static_cast<double>(__uint_as_float(sbits << 16));

    uint32_t code_word[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const double z = v[16 * h + j];
      uint32_t q = 0;
#pragma unroll
      for (int k = 0; k < 15; ++k) q += (z > scale * mid[k]) ? 1u : 0u;
      code_word[j >> 3] |= q << (4 * (j & 7));
    }
    words[2 * h] = code_word[0];
    words[2 * h + 1] = code_word[1];
    if (h == 0)
      words[4] = sbits;
    else
      words[4] |= sbits << 16;
  }

  uint32_t *dst = reinterpret_cast<uint32_t *>(packed + blk * 20);
#pragma unroll
  for (int i = 0; i < 5; ++i) dst[i] = words[i];

  if (!finite && nonfinite != nullptr) atomicAdd(nonfinite, 1);
}

}  // namespace

namespace {
template <typename In>
hipError_t launch_pack_t(const In *w, int64_t n_blocks, uint32_t sign_bits, uint8_t *packed,
                         int32_t *nonfinite, hipStream_t s) {
  if (n_blocks == 0) return hipSuccess;
  PackArgs args;
  args.cb = codebook();
  const int threads = 256;
  const int64_t grid = (n_blocks + threads - 1) / threads;
  hipLaunchKernelGGL(pack_kernel<In>, dim3(static_cast<unsigned>(grid)), dim3(threads), 0, s, w,
                     n_blocks, sign_bits, args, packed, nonfinite);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_pack(const float *w, int64_t n_blocks, uint32_t sign_bits, uint8_t *packed,
                       int32_t *nonfinite, hipStream_t s) {
  return launch_pack_t(w, n_blocks, sign_bits, packed, nonfinite, s);
}

hipError_t launch_pack_bf16(const uint16_t *w, int64_t n_blocks, uint32_t sign_bits,
                            uint8_t *packed, int32_t *nonfinite, hipStream_t s) {
  return launch_pack_t(w, n_blocks, sign_bits, packed, nonfinite, s);
}

}  // namespace tq4
