// Test-only kernel: one v_mfma_scale_f32_16x16x128_f8f6f4 (OCP e4m3 operands,
// one E8M0 scale per 32 k on each side) on operands given by the host, so
// that tests can read off how the instruction sums a block's products.  The
// fp8 weight-cache products' error bound rests on that arithmetic.
//
//   a, b : [16][128] e4m3 codes (row m of A, column n of B, k = 0..127)
//   sa, sb : [16][4] E8M0 scale bytes (row m / column n, block k / 32)
//   c : [16][16] fp32 accumulator input, d : [16][16] fp32 output,
//   d[m][n] = c[m][n] + sum_k a[m][k] 2^(sa[m][k/32]-127) b[n][k] 2^(sb[n][k/32]-127)
//   up to the instruction's own rounding.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int intx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64) void mfma_scale_probe_kernel(const uint8_t *a, const uint8_t *b,
                                                             const uint8_t *sa, const uint8_t *sb,
                                                             const float *c, float *d) {
  const int lane = threadIdx.x;
  const int i = lane % 16;
  const int g = lane / 16;
  // lane i + 16 g: bytes 0-15 are k = 16 g .. 16 g + 15, bytes 16-31 are
  // k = 64 + 16 g .. 64 + 16 g + 15 of row (column) i; its scale byte is that
  // of block g of row (column) i
  const uint4 a0 = *reinterpret_cast<const uint4 *>(a + i * 128 + 16 * g);
  const uint4 a1 = *reinterpret_cast<const uint4 *>(a + i * 128 + 64 + 16 * g);
  const uint4 b0 = *reinterpret_cast<const uint4 *>(b + i * 128 + 16 * g);
  const uint4 b1 = *reinterpret_cast<const uint4 *>(b + i * 128 + 64 + 16 * g);
  intx8 aq, bq;
  aq[0] = a0.x; aq[1] = a0.y; aq[2] = a0.z; aq[3] = a0.w;
  aq[4] = a1.x; aq[5] = a1.y; aq[6] = a1.z; aq[7] = a1.w;
  bq[0] = b0.x; bq[1] = b0.y; bq[2] = b0.z; bq[3] = b0.w;
  bq[4] = b1.x; bq[5] = b1.y; bq[6] = b1.z; bq[7] = b1.w;
  const int sav = sa[i * 4 + g];
  const int sbv = sb[i * 4 + g];
  // accumulator layout: lane i + 16 g holds rows 4 g .. 4 g + 3 of column i
  floatx4 acc;
#pragma unroll
  for (int v = 0; v < 4; ++v) acc[v] = c[(4 * g + v) * 16 + i];
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aq, bq, acc, 0, 0, 0, sav, 0, sbv);
#pragma unroll
  for (int v = 0; v < 4; ++v) d[(4 * g + v) * 16 + i] = acc[v];
}

extern "C" int tq4test_mfma_scale_probe(const uint8_t *a, const uint8_t *b, const uint8_t *sa,
                                        const uint8_t *sb, const float *c, float *d,
                                        void *stream) {
  hipLaunchKernelGGL(mfma_scale_probe_kernel, dim3(1), dim3(64), 0,
                     reinterpret_cast<hipStream_t>(stream), a, b, sa, sb, c, d);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}
